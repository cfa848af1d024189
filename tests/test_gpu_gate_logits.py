"""GPU parity of the recurrence calls with GDR_GATE_LOGITS (the token
mixer's gating fused into the recurrence's loads): log_alpha, b and w hold
logits, the kernels use log alpha = log sigmoid(a), b = sigmoid(b_logit),
w = sigmoid(w_logit) in fp32, and the backward returns the gradients of the
logits.

The oracle side turns the same logits into gates in fp64 (oracle/mixer.py),
runs the token recurrence or its reverse mode, and takes the logits'
gradients by the chain rule: d/dz sigmoid(z) = s(1 - s), d/da log sigmoid(a)
= sigmoid(-a).  Tolerances are the bf16 ones of the plain calls: max|Δ|/rms
<= 2e-2 per output tensor."""
import numpy as np
import pytest

import gdr_synth as gs
import oracle
from oracle import mixer
from tests.helpers import rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _inputs(B, H, T, dk, dv, alpha_mode="channel", b_mode="channel", w_mode="channel",
            tied=False, seed=0, with_dO=False):
    """q, k, v (and dO) as for the plain calls; the gate logits as the token
    mixer's projections give them (decay logits ~ N(4, 1), gate logits ~ N(0, 1))."""
    base = gs.make_inputs(B, H, T, dk, dv, seed=seed, with_dO=with_dO)
    lg = gs.mixer_inputs(B, H, T, dk, dv, alpha_mode=alpha_mode, b_mode=b_mode,
                         w_mode="scalar" if tied else w_mode, seed=seed)
    a = dict(base.arrays)
    a["log_alpha"] = lg["a_pre"]
    a["b"] = lg["b_pre"]
    a["w"] = a["b"] if tied else lg["w_pre"]
    return a


def _gates(a):
    """The fp64 gates the logits stand for."""
    return mixer.log_sigmoid(a["log_alpha"]), mixer.sigmoid(a["b"]), mixer.sigmoid(a["w"])


def _dev(a, names=("q", "k", "v", "log_alpha", "b", "w", "S0", "dO")):
    import torch
    out = {}
    for n in names:
        x = a.get(n)
        if x is None:
            out[n] = None
            continue
        dt = torch.float32 if n in ("log_alpha", "S0") else torch.bfloat16
        out[n] = torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()
    if a["b"] is a["w"]:
        out["w"] = out["b"]
    return out


def _bc(g, like):
    """A scalar gate [..., T] broadcast to its channels [..., T, d]."""
    return np.broadcast_to(g[..., None], like.shape) if g.ndim == like.ndim - 1 else g


FWD = [
    ("channel_d128", dict(B=1, H=2, T=256, dk=128, dv=128)),
    ("channel_d64", dict(B=2, H=2, T=192, dk=64, dv=64)),
    ("gdn_tied_scalar", dict(B=1, H=2, T=256, dk=128, dv=128, alpha_mode="scalar",
                             b_mode="scalar", tied=True)),
    ("alpha_scalar_b_channel", dict(B=1, H=2, T=128, dk=128, dv=128, alpha_mode="scalar")),
    ("dk128_dv64", dict(B=1, H=2, T=128, dk=128, dv=64)),
]


@pytest.mark.parametrize("name,kw", FWD, ids=[c[0] for c in FWD])
def test_forward_with_gate_logits(name, kw):
    import torch
    import gated_delta_rule_24_amd as gdr
    print(f"logits fwd {name} {kw}", flush=True)
    a = _inputs(**kw)
    d = _dev(a)
    o, sf = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], chunk=64,
                          gate_logits=True)
    torch.cuda.synchronize()
    la, b, w = _gates(a)
    o_ref, s_ref = oracle.fwd(a["q"], a["k"], a["v"], la, b, w, a["S0"])
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(sf.cpu().numpy(), s_ref)
    print(f"  err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= TOL and es <= TOL


def test_forward_with_gate_logits_refused_without_workspace():
    import gated_delta_rule_24_amd as gdr
    a = _inputs(1, 1, 64, 128, 128)
    d = _dev(a)
    with pytest.raises(gdr.GdrError):
        gdr.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], chunk=64,
                      path="fused", gate_logits=True)


def _ref_bwd(a, dSf):
    """Gradients of the logits from the oracle's reverse mode on the gates."""
    la, b, w = _gates(a)
    ref = oracle.bwd(a["q"], a["k"], a["v"], la, b, w, a["S0"], a["dO"], dSf)
    q = a["q"]
    sa = mixer.sigmoid(-np.asarray(a["log_alpha"], dtype=np.float64))
    for n, logit, gate, chain in (("dlog_alpha", a["log_alpha"], None, sa),
                                  ("db", a["b"], b, None), ("dw", a["w"], w, None)):
        g = ref[n]
        scalar = np.asarray(logit).ndim == q.ndim - 1
        if scalar:
            g = g.sum(-1)
        ref[n] = g * (chain if chain is not None else gate * (1.0 - gate))
    return ref


BWD = [
    ("channel_d128", dict(B=1, H=2, T=192, dk=128, dv=128)),
    ("gdn_tied_scalar_d64", dict(B=1, H=2, T=192, dk=64, dv=64, alpha_mode="scalar",
                                 b_mode="scalar", tied=True)),
    ("alpha_scalar", dict(B=1, H=2, T=128, dk=128, dv=128, alpha_mode="scalar")),
    ("b_scalar_w_channel", dict(B=1, H=2, T=128, dk=64, dv=64, b_mode="scalar")),
]


@pytest.mark.parametrize("name,kw", BWD, ids=[c[0] for c in BWD])
def test_backward_with_gate_logits(name, kw):
    import torch
    import gated_delta_rule_24_amd as gdr
    print(f"logits bwd {name} {kw}", flush=True)
    a = _inputs(with_dO=True, **kw)
    dSf = (np.random.default_rng(9).standard_normal(a["S0"].shape) * 0.5).astype(np.float32)
    d = _dev(a)
    g = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], d["dO"],
                      torch.from_numpy(dSf).cuda(), chunk=64, gate_logits=True)
    torch.cuda.synchronize()
    ref = _ref_bwd(a, dSf)
    errs = {n: rel_err(g[n].cpu().numpy(), ref[n]) for n in ref}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    assert all(e <= TOL for e in errs.values()), errs


def _packed(lengths, H, dk, dv, seed=0, with_dO=False, **kw):
    inp = gs.packed_inputs(lengths, H, dk, dv, seed=seed, with_dO=with_dO)
    T = sum(lengths)
    lg = gs.mixer_inputs(1, H, T, dk, dv, seed=seed, **kw)
    a = dict(inp.arrays)
    a["log_alpha"], a["b"], a["w"] = lg["a_pre"], lg["b_pre"], lg["w_pre"]
    return a


def test_packed_forward_and_backward_with_gate_logits():
    """Packed sequences with empty, single-token and ragged lengths: the tokens
    past a sequence's end in its last chunk must not decay the state (their
    decay logit is taken as +inf inside the kernels)."""
    import torch
    import gated_delta_rule_24_amd as gdr
    lengths = [0, 1, 63, 65, 130, 7]
    H, D = 2, 128
    print(f"logits packed lengths={lengths}", flush=True)
    a = _packed(lengths, H, D, D, with_dO=True)
    d = _dev(a)
    cu = torch.from_numpy(a["cu_seqlens"]).cuda()
    o, sf = gdr.chunk_fwd_varlen(d["q"][0], d["k"][0], d["v"][0], d["log_alpha"][0], d["b"][0],
                                 d["w"][0], cu, d["S0"], gate_logits=True)
    g = gdr.chunk_bwd_varlen(d["q"][0], d["k"][0], d["v"][0], d["log_alpha"][0], d["b"][0],
                             d["w"][0], cu, d["S0"], d["dO"][0], None, gate_logits=True)
    torch.cuda.synchronize()
    la, b, w = _gates(a)
    cuh = a["cu_seqlens"]
    o_np, sf_np = o.cpu().numpy(), sf.cpu().numpy()
    gg = {n: t.cpu().numpy() for n, t in g.items()}
    for s in range(len(lengths)):
        lo, hi = int(cuh[s]), int(cuh[s + 1])
        if hi == lo:
            np.testing.assert_allclose(sf_np[s], a["S0"][s], rtol=0, atol=0)
            np.testing.assert_allclose(gg["dS0"][s], 0.0, rtol=0, atol=0)
            continue

        def sl(x):
            return x[0][:, lo:hi]
        o_s, s_s = oracle.fwd(sl(a["q"]), sl(a["k"]), sl(a["v"]), sl(la), sl(b), sl(w), a["S0"][s])
        assert rel_err(o_np[:, lo:hi], o_s) <= TOL and rel_err(sf_np[s], s_s) <= TOL, s
        sub = {n: sl(a[n]) for n in ("q", "k", "v", "log_alpha", "b", "w", "dO")}
        sub["S0"] = a["S0"][s]
        ref = _ref_bwd(sub, None)
        for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
            e = rel_err(gg[n][:, lo:hi], ref[n])
            assert e <= TOL, (s, n, e)
        assert rel_err(gg["dS0"][s], ref["dS0"]) <= TOL, s


def test_decode_with_gate_logits():
    import torch
    import gated_delta_rule_24_amd as gdr
    N, H, D = 4, 8, 128
    print(f"logits decode N={N} H={H} d={D}", flush=True)
    S = gs.decode_state(N, H, D, D, seed=2)
    t = gs.decode_token(N, H, D, D, 0, seed=2)
    lg = gs.mixer_inputs(N, H, 1, D, D, seed=2)
    a_pre, b_pre, w_pre = lg["a_pre"][:, :, 0], lg["b_pre"][:, :, 0], lg["w_pre"][:, :, 0]
    Sd = torch.from_numpy(S).cuda()
    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()
    o = gdr.decode_step(dev(t["q"], torch.bfloat16), dev(t["k"], torch.bfloat16),
                        dev(t["v"], torch.bfloat16), dev(a_pre, torch.float32),
                        dev(b_pre, torch.bfloat16), dev(w_pre, torch.bfloat16), Sd, gate_logits=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode(t["q"], t["k"], t["v"], mixer.log_sigmoid(a_pre), mixer.sigmoid(b_pre),
                                 mixer.sigmoid(w_pre), S)
    eo, es = rel_err(o.cpu().numpy(), o_ref), rel_err(Sd.cpu().numpy(), s_ref)
    print(f"  err o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= 1e-4 and es <= 1e-4


def test_token_mixer_with_gating_fused():
    """Prologue producing q, k, v only, the forward taking the gate logits, the
    epilogue: against the oracle's block, and against the unfused GPU block
    (prologue producing all six inputs)."""
    import torch
    import gated_delta_rule_24_amd as gdr
    B, H, T, D = 1, 2, 256, 128
    print(f"logits mixer block B={B} H={H} T={T} d={D}", flush=True)
    m = gs.mixer_inputs(B, H, T, D, D, seed=6)
    S0 = (np.random.default_rng(7).standard_normal((B, H, D, D)) * 0.02).astype(np.float32)
    dm = {n: torch.from_numpy(x).to(torch.float32 if n in ("conv_q", "conv_k", "conv_v", "a_pre",
                                                          "norm_weight") else torch.bfloat16).cuda()
          for n, x in m.items()}
    S0d = torch.from_numpy(S0).cuda()
    args = [dm[n] for n in ("q_pre", "k_pre", "v_pre", "conv_q", "conv_k", "conv_v", "a_pre", "b_pre",
                            "w_pre")]
    xf = gdr.mixer_prologue(*args, gate_logits=True)
    of, _ = gdr.chunk_fwd(xf["q"], xf["k"], xf["v"], xf["log_alpha"], xf["b"], xf["w"], S0d, chunk=64,
                          gate_logits=True)
    xu = gdr.mixer_prologue(*args)
    ou, _ = gdr.chunk_fwd(xu["q"], xu["k"], xu["v"], xu["log_alpha"], xu["b"], xu["w"], S0d, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(xf["q"], xu["q"]) and torch.equal(xf["k"], xu["k"]) and torch.equal(xf["v"], xu["v"])
    r = mixer.prologue(m["q_pre"], m["k_pre"], m["v_pre"], m["conv_q"], m["conv_k"], m["conv_v"],
                       m["a_pre"], m["b_pre"], m["w_pre"])
    qkv = {n: gs.bf16_round(r[n].astype(np.float32)) for n in ("q", "k", "v")}
    o_ref, _ = oracle.fwd(qkv["q"], qkv["k"], qkv["v"], r["log_alpha"], r["b"], r["w"], S0)
    ef, eu = rel_err(of.cpu().numpy(), o_ref), rel_err(ou.cpu().numpy(), o_ref)
    print(f"  err o fused={ef:.3e} unfused={eu:.3e}", flush=True)
    assert ef <= TOL and eu <= TOL
