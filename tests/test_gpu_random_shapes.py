"""Seeded random configurations of the forward, backward and packed calls
against the oracle: random head sizes, chunk sizes, lengths, gate modes
(channel, scalar, tied), activation dtypes, paths and gate-logit mode.  Each
configuration is drawn from its seed alone, so a failure names a reproducible
case.  Tolerances as in the fixed tests: max|Δ|/rms <= 2e-2 with bf16
activations, 1e-4 with fp32."""
import numpy as np
import pytest

import gdr_synth as gs
import oracle
from oracle import mixer
from tests.helpers import flat_heads, oracle_fwd, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _config(seed):
    r = np.random.default_rng([seed, 99])
    act = "f32" if r.random() < 0.25 else "bf16"
    d = int(r.choice([64, 128] if act == "bf16" and r.random() < 0.7 else [16, 32, 64, 128]))
    dk, dv = d, d
    if r.random() < 0.3:
        dv = int(r.choice([x for x in (16, 32, 64, 128) if x != d]))
    chunk = int(r.choice([16, 32, 64]))
    T = chunk * int(r.integers(1, 6))
    tied = r.random() < 0.3
    modes = dict(alpha_mode=str(r.choice(["channel", "scalar"])),
                 b_mode="scalar" if tied else str(r.choice(["channel", "scalar"])),
                 w_mode="scalar" if tied else str(r.choice(["channel", "scalar"])))
    return dict(B=int(r.integers(1, 3)), H=int(r.integers(1, 4)), T=T, dk=dk, dv=dv, act=act,
                chunk=chunk, tied=tied, s0_std=None if r.random() < 0.2 else 0.02, **modes)


@pytest.mark.parametrize("seed", range(16))
def test_random_forward(seed):
    import torch
    import gated_delta_rule_24_amd as gdr
    cfg = _config(seed)
    path = "fused" if seed % 3 == 0 else "auto"
    print(f"random fwd seed={seed} path={path} {cfg}", flush=True)
    inp = gs.make_inputs(seed=seed, **cfg)
    d = to_dev(inp)
    o, sf = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"],
                          chunk=cfg["chunk"], path=path)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_fwd(inp)
    tol = 1e-4 if cfg["act"] == "f32" else 2e-2
    eo = rel_err(flat_heads(o.cpu().numpy(), inp.B, inp.H), o_ref)
    es = rel_err(flat_heads(sf.cpu().numpy(), inp.B, inp.H), s_ref)
    print(f"  err o={eo:.2e} S={es:.2e} (tol {tol})", flush=True)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("seed", range(100, 110))
def test_random_backward(seed):
    import torch
    import gated_delta_rule_24_amd as gdr
    cfg = _config(seed)
    print(f"random bwd seed={seed} {cfg}", flush=True)
    inp = gs.make_inputs(seed=seed, with_dO=True, **cfg)
    d = to_dev(inp)
    s0 = d["S0"] if d["S0"] is not None else torch.zeros((inp.B, inp.H, inp.dk, inp.dv), device="cuda")
    g = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], s0, d["dO"], None,
                      chunk=cfg["chunk"])
    torch.cuda.synchronize()
    a = inp.arrays
    flat = lambda x: None if x is None else x.reshape((inp.B * inp.H,) + x.shape[2:])
    ref = oracle.bwd(*(flat(a[n]) for n in ("q", "k", "v", "log_alpha", "b", "w", "S0", "dO")))
    for n, mode in (("dlog_alpha", inp.alpha_mode), ("db", inp.b_mode), ("dw", inp.w_mode)):
        if mode == "scalar":
            ref[n] = ref[n].sum(-1)
    tol = 1e-4 if cfg["act"] == "f32" else 2e-2
    errs = {n: rel_err(flat_heads(g[n].cpu().numpy(), inp.B, inp.H) if n != "dS0"
                       else g[n].cpu().numpy().reshape(ref[n].shape), ref[n]) for n in ref}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (tol {tol})", flush=True)
    assert all(e <= tol for e in errs.values()), errs


@pytest.mark.parametrize("seed", range(300, 312))
def test_random_gate_ranges(seed):
    """Random configurations as above with random decay strength (the
    synthetic decay scale 0.05, 0.5, 2 or 20: from the workloads' mild decay to
    chunks decaying by tens of nats, which the chunk kernels that reference a
    chunk's end hand to the token-level recompute) and erase gates drawn up to
    1 or 2: forward on a random path and backward, values against the oracle."""
    import torch
    import gated_delta_rule_24_amd as gdr
    cfg = _config(seed)
    r = np.random.default_rng([seed, 97])
    cfg["decay_scale"] = float(r.choice([0.05, 0.5, 2.0, 20.0]))
    cfg["gate_hi"] = float(r.choice([1.0, 2.0]))
    path = ["auto", "fused", "split"][seed % 3]
    print(f"random gate ranges seed={seed} path={path} {cfg}", flush=True)
    inp = gs.make_inputs(seed=seed, with_dO=True, **cfg)
    d = to_dev(inp)
    tol = 1e-4 if cfg["act"] == "f32" else 2e-2
    o, sf = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"],
                          chunk=cfg["chunk"], path=path)
    s0 = d["S0"] if d["S0"] is not None else torch.zeros((inp.B, inp.H, inp.dk, inp.dv), device="cuda")
    g = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], s0, d["dO"], None,
                      chunk=cfg["chunk"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_fwd(inp)
    eo = rel_err(flat_heads(o.cpu().numpy(), inp.B, inp.H), o_ref)
    es = rel_err(flat_heads(sf.cpu().numpy(), inp.B, inp.H), s_ref)
    a = inp.arrays
    flat = lambda x: None if x is None else x.reshape((inp.B * inp.H,) + x.shape[2:])
    ref = oracle.bwd(*(flat(a[n]) for n in ("q", "k", "v", "log_alpha", "b", "w", "S0", "dO")))
    for n, mode in (("dlog_alpha", inp.alpha_mode), ("db", inp.b_mode), ("dw", inp.w_mode)):
        if mode == "scalar":
            ref[n] = ref[n].sum(-1)
    errs = {n: rel_err(flat_heads(g[n].cpu().numpy(), inp.B, inp.H) if n != "dS0"
                       else g[n].cpu().numpy().reshape(ref[n].shape), ref[n]) for n in ref}
    errs["o"], errs["S_final"] = eo, es
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (tol {tol})", flush=True)
    assert all(e <= tol for e in errs.values()), errs


@pytest.mark.parametrize("seed", range(200, 208))
def test_random_packed(seed):
    """Random length mixes (empty, short and multi-chunk documents), random
    gate modes and head sizes, optionally gate logits: forward and backward."""
    _packed_case(seed, strong=False)


@pytest.mark.parametrize("seed", range(400, 408))
def test_random_packed_gate_ranges(seed):
    """As above with a random decay strength (synthetic decay scale 0.5, 2 or
    20: the packed backward's records leave their range and its units go to
    the token-level recompute, while the packed forward references each
    chunk's start) and erase gates drawn up to 1 or 2, without gate logits."""
    _packed_case(seed, strong=True)


def _packed_case(seed, strong):
    import torch
    import gated_delta_rule_24_amd as gdr
    r = np.random.default_rng([seed, 98])
    nseq = int(r.integers(1, 7))
    lengths = [int(x) for x in r.choice([0, 1, 7, 63, 64, 65, 100, 200], size=nseq)]
    D = int(r.choice([64, 128]))
    H = int(r.integers(1, 4))
    logits = bool(r.random() < 0.4) and not strong
    modes = dict(alpha_mode=str(r.choice(["channel", "scalar"])), b_mode=str(r.choice(["channel", "scalar"])),
                 w_mode=str(r.choice(["channel", "scalar"])))
    if strong:
        modes["decay_scale"] = float(r.choice([0.5, 2.0, 20.0]))
        modes["gate_hi"] = float(r.choice([1.0, 2.0]))
    print(f"random packed seed={seed} lengths={lengths} H={H} d={D} logits={logits} {modes}", flush=True)
    inp = gs.packed_inputs(lengths, H, D, D, seed=seed, with_dO=True, **modes)
    a = dict(inp.arrays)
    if logits:
        lg = gs.mixer_inputs(1, H, inp.T, D, D, seed=seed, **modes)
        a["log_alpha"], a["b"], a["w"] = lg["a_pre"], lg["b_pre"], lg["w_pre"]   # b, w logits bf16 values
    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x[0])).to(dt).cuda()
    bf, f32 = torch.bfloat16, torch.float32
    d = dict(q=dev(a["q"], bf), k=dev(a["k"], bf), v=dev(a["v"], bf), la=dev(a["log_alpha"], f32),
             b=dev(a["b"], bf), w=dev(a["w"], bf), dO=dev(a["dO"], bf))
    S0 = torch.from_numpy(a["S0"]).cuda()
    cu = torch.from_numpy(a["cu_seqlens"]).cuda()
    o, sf = gdr.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["la"], d["b"], d["w"], cu, S0,
                                 gate_logits=logits)
    g = gdr.chunk_bwd_varlen(d["q"], d["k"], d["v"], d["la"], d["b"], d["w"], cu, S0, d["dO"],
                             gate_logits=logits)
    torch.cuda.synchronize()
    la, bb, ww = a["log_alpha"], a["b"], a["w"]
    if logits:
        la, bb, ww = mixer.log_sigmoid(la), mixer.sigmoid(bb), mixer.sigmoid(ww)
    cuh = a["cu_seqlens"]
    o_np, sf_np = o.cpu().numpy(), sf.cpu().numpy()
    gg = {n: t.cpu().numpy() for n, t in g.items()}
    for s in range(nseq):
        lo, hi = int(cuh[s]), int(cuh[s + 1])
        if hi == lo:
            assert np.array_equal(sf_np[s], a["S0"][s]) and not gg["dS0"][s].any()
            continue

        def sl(x):
            return x[0][:, lo:hi]
        o_s, s_s = oracle.fwd(sl(a["q"]), sl(a["k"]), sl(a["v"]), sl(la), sl(bb), sl(ww), a["S0"][s])
        assert rel_err(o_np[:, lo:hi], o_s) <= 2e-2 and rel_err(sf_np[s], s_s) <= 2e-2, s
        ref = oracle.bwd(sl(a["q"]), sl(a["k"]), sl(a["v"]), sl(la), sl(bb), sl(ww), a["S0"][s],
                         sl(a["dO"]))
        chain = {"dlog_alpha": mixer.sigmoid(-np.asarray(sl(a["log_alpha"]), dtype=np.float64)),
                 "db": sl(bb) * (1 - sl(bb)), "dw": sl(ww) * (1 - sl(ww))}
        for n, mode in (("dlog_alpha", modes["alpha_mode"]), ("db", modes["b_mode"]),
                        ("dw", modes["w_mode"])):
            if mode == "scalar":
                ref[n] = ref[n].sum(-1)
            if logits:
                ref[n] = ref[n] * chain[n]
        for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
            e = rel_err(gg[n][:, lo:hi], ref[n])
            assert e <= 2e-2, (s, n, e)
        assert rel_err(gg["dS0"][s], ref["dS0"]) <= 2e-2, s
