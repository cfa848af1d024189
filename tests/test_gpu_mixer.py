"""GPU parity of the token-mixer prologue and epilogue (gdr_mixer_prologue,
gdr_mixer_epilogue) against the fp64 oracle in oracle/mixer.py.

The kernels compute in fp32 and round each bf16 output once, so a bf16
output may differ from the exact value by at most one bf16 unit in the last
place: |Δ| <= 2^-7 |ref| (+1e-6 for values near zero).  log alpha stays fp32:
|Δ| <= 1e-5 |ref| + 1e-7.  The end-to-end check (prologue, two-pass forward,
epilogue) against the oracle's prologue, recurrence and epilogue holds the
recurrence output to the forward's bf16 tolerance, max|Δ|/rms <= 2e-2, and
each bf16 y to one unit in the last place plus 2e-2 of its rms."""
import numpy as np
import pytest

import gdr_synth as gs
import oracle
from oracle import mixer
from tests.helpers import rel_err

pytestmark = pytest.mark.gpu

BF16_ULP = 2.0 ** -7


def _dev(m):
    import torch
    out = {}
    for n, a in m.items():
        dt = torch.float32 if n in ("conv_q", "conv_k", "conv_v", "a_pre", "norm_weight") else torch.bfloat16
        out[n] = torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    return out


def _close_bf16(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    bad = np.abs(got - ref) > BF16_ULP * np.abs(ref) + 1e-6
    print(f"  {name}: max|d|/rms {rel_err(got, ref):.2e}, outside 1 ulp: {int(bad.sum())}", flush=True)
    assert not bad.any(), name


def _prologue_case(name, **kw):
    print(f"mixer case {name} {kw}", flush=True)
    B, H, T, dk, dv = kw.pop("B"), kw.pop("H"), kw.pop("T"), kw.pop("dk"), kw.pop("dv")
    return gs.mixer_inputs(B, H, T, dk, dv, **kw)


PROLOGUE = [
    ("d128", dict(B=2, H=3, T=200, dk=128, dv=128)),
    ("d64", dict(B=1, H=2, T=130, dk=64, dv=64)),
    ("dk128_dv64", dict(B=1, H=2, T=70, dk=128, dv=64)),
    ("dk64_dv128", dict(B=2, H=1, T=64, dk=64, dv=128)),
    ("scalar_gates_odd_T", dict(B=2, H=3, T=77, dk=128, dv=128, alpha_mode="scalar",
                                b_mode="scalar", w_mode="scalar")),
    ("mixed_gates", dict(B=1, H=2, T=100, dk=128, dv=128, alpha_mode="scalar", w_mode="scalar")),
    ("one_token", dict(B=1, H=2, T=1, dk=128, dv=128)),
    ("three_tokens", dict(B=1, H=1, T=3, dk=64, dv=64)),
]


@pytest.mark.parametrize("name,kw", PROLOGUE, ids=[c[0] for c in PROLOGUE])
def test_prologue_matches_oracle(name, kw):
    import torch
    import gated_delta_rule_24_amd as gdr
    m = _prologue_case(name, **kw)
    d = _dev(m)
    got = gdr.mixer_prologue(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                             d["conv_v"], d["a_pre"], d["b_pre"], d["w_pre"])
    torch.cuda.synchronize()
    ref = mixer.prologue(m["q_pre"], m["k_pre"], m["v_pre"], m["conv_q"], m["conv_k"], m["conv_v"],
                         m["a_pre"], m["b_pre"], m["w_pre"])
    for n in ("q", "k", "v", "b", "w"):
        _close_bf16(n, got[n].float().cpu().numpy(), ref[n])
    la = got["log_alpha"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(la - ref["log_alpha"]) <= 1e-5 * np.abs(ref["log_alpha"]) + 1e-7)


@pytest.mark.parametrize("dv,T", [(128, 200), (64, 77), (128, 1)])
def test_epilogue_matches_oracle(dv, T):
    import torch
    import gated_delta_rule_24_amd as gdr
    print(f"mixer epilogue dv={dv} T={T}", flush=True)
    m = gs.mixer_inputs(2, 3, T, 64, dv, seed=4)
    o = np.random.default_rng(5).standard_normal((2, 3, T, dv)).astype(np.float32)
    d = _dev(m)
    y = gdr.mixer_epilogue(torch.from_numpy(o).cuda(), d["g"], d["norm_weight"])
    torch.cuda.synchronize()
    _close_bf16("y", y.float().cpu().numpy(), mixer.epilogue(o, m["g"], m["norm_weight"]))


def test_token_mixer_end_to_end():
    """Prologue -> two-pass forward -> epilogue on the GPU against the oracle's
    prologue -> token recurrence -> epilogue in fp64.  The recurrence's
    inputs are stored in bf16 between the steps on both sides (the oracle
    rounds its own prologue outputs), and log alpha in fp32."""
    import torch
    import gated_delta_rule_24_amd as gdr
    B, H, T, D = 1, 2, 256, 128
    print(f"mixer end to end B={B} H={H} T={T} d={D}", flush=True)
    m = gs.mixer_inputs(B, H, T, D, D, seed=6)
    S0 = (np.random.default_rng(7).standard_normal((B, H, D, D)) * 0.02).astype(np.float32)
    d = _dev(m)
    x = gdr.mixer_prologue(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"], d["conv_v"],
                           d["a_pre"], d["b_pre"], d["w_pre"])
    o, _ = gdr.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                         torch.from_numpy(S0).cuda(), chunk=64)
    y = gdr.mixer_epilogue(o, d["g"], d["norm_weight"])
    torch.cuda.synchronize()
    r = mixer.prologue(m["q_pre"], m["k_pre"], m["v_pre"], m["conv_q"], m["conv_k"], m["conv_v"],
                       m["a_pre"], m["b_pre"], m["w_pre"])
    r = {n: (a if n == "log_alpha" else gs.bf16_round(a.astype(np.float32))) for n, a in r.items()}
    o_ref, _ = oracle.fwd(r["q"], r["k"], r["v"], r["log_alpha"], r["b"], r["w"], S0)
    y_ref = mixer.epilogue(o_ref, m["g"], m["norm_weight"])
    eo = rel_err(o.cpu().numpy(), o_ref)
    # y is bf16: one unit in the last place of each value, plus the forward's
    # tolerance carried through the normalisation (max|Δ|/rms alone cannot
    # reach 2e-2 for a bf16 output whose values run to many times its rms)
    yg = y.float().cpu().numpy().astype(np.float64)
    bound = BF16_ULP * np.abs(y_ref) + 2e-2 * np.sqrt(np.mean(y_ref * y_ref))
    worst = float(np.max(np.abs(yg - y_ref) / bound))
    print(f"  err o={eo:.3e} (tol 2e-2); y: max|d|/rms {rel_err(yg, y_ref):.3e}, "
          f"worst |d| / (1 ulp + 2e-2 rms) = {worst:.2f}", flush=True)
    assert eo <= 2e-2 and worst <= 1.0


def test_prologue_workload_shape_all_heads():
    """The forward workload's shape (B=2, H=16, T=8192, d=128): every output
    of every head against the oracle."""
    import torch
    import gated_delta_rule_24_amd as gdr
    B, H, T, D = 2, 16, 8192, 128
    print(f"mixer workload B={B} H={H} T={T} d={D}", flush=True)
    m = gs.mixer_inputs(B, H, T, D, D, seed=8)
    d = _dev(m)
    got = gdr.mixer_prologue(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                             d["conv_v"], d["a_pre"], d["b_pre"], d["w_pre"])
    torch.cuda.synchronize()
    for b, h in ((b, h) for b in range(B) for h in range(H)):
        sel = {n: (m[n][b:b + 1, h:h + 1] if m[n].ndim == 4 else m[n][h:h + 1])
               for n in ("q_pre", "k_pre", "v_pre", "a_pre", "b_pre", "w_pre", "conv_q", "conv_k",
                         "conv_v")}
        ref = mixer.prologue(sel["q_pre"], sel["k_pre"], sel["v_pre"], sel["conv_q"], sel["conv_k"],
                             sel["conv_v"], sel["a_pre"], sel["b_pre"], sel["w_pre"])
        for n in ("q", "k", "v", "b", "w"):
            _close_bf16(f"{n}[{b},{h}]", got[n][b:b + 1, h:h + 1].float().cpu().numpy(), ref[n])


BWD_TOL = 1e-4     # fp32 gradients of exact (bf16-valued) inputs


@pytest.mark.parametrize("D,T", [(128, 200), (64, 77), (128, 64), (64, 1)])
def test_prologue_backward_matches_oracle(D, T):
    """dq_pre, dk_pre, dv_pre and the tap gradients against reverse mode of the
    oracle's q / k path (conv, SiLU, L2 norm) and v path (conv, SiLU)."""
    import torch
    import gated_delta_rule_24_amd as gdr
    B, H = 2, 3
    print(f"mixer prologue bwd B={B} H={H} T={T} d={D}", flush=True)
    m = gs.mixer_inputs(B, H, T, D, D, seed=10)
    r = np.random.default_rng(11)
    dy = {n: r.standard_normal((B, H, T, D)).astype(np.float32) for n in ("q", "k", "v")}
    d = _dev(m)
    g = gdr.mixer_prologue_bwd(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                               d["conv_v"], *[torch.from_numpy(dy[n]).cuda() for n in ("q", "k", "v")])
    torch.cuda.synchronize()
    for n, l2 in (("q", True), ("k", True), ("v", False)):
        gx, gw = mixer.stream_bwd(m[f"{n}_pre"], m[f"conv_{n}"], dy[n], l2)
        ex = rel_err(g[f"d{n}_pre"].cpu().numpy(), gx)
        ew = rel_err(g[f"dconv_{n}"].cpu().numpy(), gw)
        print(f"  {n}: d_pre {ex:.2e} dconv {ew:.2e} (tol {BWD_TOL})", flush=True)
        assert ex <= BWD_TOL and ew <= BWD_TOL, (n, ex, ew)


@pytest.mark.parametrize("D,T", [(128, 200), (64, 33)])
def test_epilogue_backward_matches_oracle(D, T):
    import torch
    import gated_delta_rule_24_amd as gdr
    B, H = 2, 3
    print(f"mixer epilogue bwd B={B} H={H} T={T} d={D}", flush=True)
    m = gs.mixer_inputs(B, H, T, 64, D, seed=12)
    r = np.random.default_rng(13)
    o = r.standard_normal((B, H, T, D)).astype(np.float32)
    dy = r.standard_normal((B, H, T, D)).astype(np.float32)
    d = _dev(m)
    g = gdr.mixer_epilogue_bwd(torch.from_numpy(o).cuda(), d["g"], d["norm_weight"],
                               torch.from_numpy(dy).cuda())
    torch.cuda.synchronize()
    go, gg, gw = mixer.epilogue_bwd(o, m["g"], m["norm_weight"], dy)
    errs = {"d_o": rel_err(g["d_o"].cpu().numpy(), go), "dg": rel_err(g["dg"].cpu().numpy(), gg),
            "dnorm_weight": rel_err(g["dnorm_weight"].cpu().numpy(), gw)}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    assert all(e <= BWD_TOL for e in errs.values()), errs


def test_mixer_backward_deterministic():
    """The tap and norm-weight gradients are summed in a fixed order."""
    import torch
    import gated_delta_rule_24_amd as gdr
    m = gs.mixer_inputs(2, 2, 300, 128, 128, seed=14)
    d = _dev(m)
    dy = torch.randn((2, 2, 300, 128), device="cuda")
    a = gdr.mixer_prologue_bwd(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                               d["conv_v"], dy, dy, dy)
    b = gdr.mixer_prologue_bwd(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                               d["conv_v"], dy, dy, dy)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_training_step_through_the_block():
    """A whole training step of the token mixer on the GPU, gating fused:
    prologue (q, k, v) -> forward on the gate logits -> epilogue, then the
    epilogue's, the recurrence's and the prologue's backward, against the
    oracle's composition of the same steps (its recurrence inputs and dO stored
    in bf16 like the GPU's).  Each stage is held to its own tolerance by the
    tests above and by the recurrence's tests; here their errors add up (the
    forward's o error, amplified by the epilogue's per-row normalisation, then
    the recurrence backward's own error, measured 3-7e-2 on the logits' and
    projections' gradients), so this test checks that the stages compose:
    layouts, the chain rule and the gate-logit convention.  A mistake in any
    of those gives O(1) errors; the bound is 1e-1."""
    import torch
    import gated_delta_rule_24_amd as gdr
    B, H, T, D = 1, 2, 192, 128
    print(f"mixer training step B={B} H={H} T={T} d={D}", flush=True)
    m = gs.mixer_inputs(B, H, T, D, D, seed=15)
    S0 = (np.random.default_rng(16).standard_normal((B, H, D, D)) * 0.02).astype(np.float32)
    dy = np.random.default_rng(17).standard_normal((B, H, T, D)).astype(np.float32)
    d = _dev(m)
    S0d = torch.from_numpy(S0).cuda()
    x = gdr.mixer_prologue(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"], d["conv_v"],
                           d["a_pre"], d["b_pre"], d["w_pre"], gate_logits=True)
    o, _ = gdr.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S0d, chunk=64,
                         gate_logits=True)
    ge = gdr.mixer_epilogue_bwd(o, d["g"], d["norm_weight"], torch.from_numpy(dy).cuda())
    gr = gdr.chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S0d,
                       ge["d_o"].to(torch.bfloat16), None, chunk=64, gate_logits=True)
    gp = gdr.mixer_prologue_bwd(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                                d["conv_v"], gr["dq"], gr["dk"], gr["dv"])
    torch.cuda.synchronize()
    # oracle composition
    r = mixer.prologue(m["q_pre"], m["k_pre"], m["v_pre"], m["conv_q"], m["conv_k"], m["conv_v"],
                       m["a_pre"], m["b_pre"], m["w_pre"])
    qkv = {n: gs.bf16_round(r[n].astype(np.float32)) for n in ("q", "k", "v")}
    o_ref, _ = oracle.fwd(qkv["q"], qkv["k"], qkv["v"], r["log_alpha"], r["b"], r["w"], S0)
    go_ref, gg_ref, gw_ref = mixer.epilogue_bwd(o_ref, m["g"], m["norm_weight"], dy)
    # the GPU hands the recurrence's backward dO in bf16: the oracle rounds its own
    g_ref = oracle.bwd(qkv["q"], qkv["k"], qkv["v"], r["log_alpha"], r["b"], r["w"], S0,
                       gs.bf16_round(go_ref.astype(np.float32)), None)
    sa = mixer.sigmoid(-np.asarray(m["a_pre"], dtype=np.float64))
    ref = {"dg": gg_ref, "dnorm_weight": gw_ref,
           "da_pre": g_ref["dlog_alpha"] * sa,
           "db_pre": g_ref["db"] * r["b"] * (1 - r["b"]),
           "dw_pre": g_ref["dw"] * r["w"] * (1 - r["w"])}
    for n, l2 in (("q", True), ("k", True), ("v", False)):
        gx, gw = mixer.stream_bwd(m[f"{n}_pre"], m[f"conv_{n}"], g_ref[f"d{n}"], l2)
        ref[f"d{n}_pre"], ref[f"dconv_{n}"] = gx, gw
    got = {"dg": ge["dg"], "dnorm_weight": ge["dnorm_weight"], "da_pre": gr["dlog_alpha"],
           "db_pre": gr["db"], "dw_pre": gr["dw"], "dq_pre": gp["dq_pre"], "dk_pre": gp["dk_pre"],
           "dv_pre": gp["dv_pre"], "dconv_q": gp["dconv_q"], "dconv_k": gp["dconv_k"],
           "dconv_v": gp["dconv_v"]}
    errs = {n: rel_err(got[n].cpu().numpy(), ref[n]) for n in ref}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    assert all(e <= 1e-1 for e in errs.values()), errs
    # the bound discriminates: the decay-logit gradient without its chain-rule
    # factor sigmoid(-a) is far outside it
    assert rel_err(got["da_pre"].cpu().numpy(), g_ref["dlog_alpha"]) > 0.5


def test_mixer_calls_replay_from_a_graph():
    """Prologue, epilogue and their backward (with the deterministic
    reductions) captured into one graph replay to the eager results."""
    import torch
    import gated_delta_rule_24_amd as gdr
    m = gs.mixer_inputs(1, 2, 200, 128, 128, seed=21)
    d = _dev(m)
    o = torch.randn((1, 2, 200, 128), device="cuda")
    dy = torch.randn((1, 2, 200, 128), device="cuda")

    def run():
        x = gdr.mixer_prologue(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                               d["conv_v"], d["a_pre"], d["b_pre"], d["w_pre"])
        y = gdr.mixer_epilogue(o, d["g"], d["norm_weight"])
        gp = gdr.mixer_prologue_bwd(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                                    d["conv_v"], dy, dy, dy)
        ge = gdr.mixer_epilogue_bwd(o, d["g"], d["norm_weight"], dy)
        return dict(y=y, **x, **gp, **ge)
    eager = run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = run()
    for rep in range(3):
        x = torch.randn(1 << 20, device="cuda")
        x.mul_(2.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in eager:
            assert torch.equal(captured[n], eager[n]), (rep, n)
