"""GPU parity of gdr_chunk_fwd against the fp64 token-recurrence oracle.

Tolerances (max|Δ|/rms(ref) over the whole tensor, separately for o and
S_final): 1e-4 with fp32 activations, 2e-2 with bf16 q/k/v/b/w (fp32 state
and decay).  Sizes span several chunks and every gate mode; the full
workloads are checked on sampled heads, whose oracle finishes in seconds."""
import numpy as np
import pytest

import gdr_synth as gs
from tests.helpers import flat_heads, oracle_fwd, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _run(inp, chunk=None, S0=None, out_dtype=None, return_state=True, generic=False, path="auto"):
    import torch
    import gated_delta_rule_24_amd as gdr
    d = to_dev(inp)
    s0 = d["S0"] if S0 is None else S0
    o, sf = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], s0,
                          chunk=chunk or inp.chunk, out_dtype=out_dtype or torch.float32,
                          return_state=return_state, generic=generic, path=path)
    torch.cuda.synchronize()
    return o, sf


def _check(inp, o, sf, tol, heads=None):
    o_ref, s_ref = oracle_fwd(inp, heads=heads)
    o_g = flat_heads(o.float().cpu().numpy(), inp.B, inp.H, heads)
    s_g = flat_heads(sf.cpu().numpy(), inp.B, inp.H, heads)
    eo, es = rel_err(o_g, o_ref), rel_err(s_g, s_ref)
    print(f"  err o={eo:.3e} S={es:.3e} (tol {tol})", flush=True)
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


def _case(name, **kw):
    print(f"fwd case {name} {kw}", flush=True)
    return gs.preset(name, **kw) if name in gs.PRESETS else gs.make_inputs(**kw)


def test_tiny_gdn_fp32():
    inp = _case("gdn_tiny")
    o, sf = _run(inp)
    _check(inp, o, sf, 1e-4)


SMALL = [
    # name, kwargs, tol
    ("gdn2_bf16_c64", dict(B=2, H=2, T=320, dk=128, dv=128, chunk=64), 2e-2),
    ("gdn2_bf16_c32", dict(B=1, H=2, T=256, dk=128, dv=128, chunk=32), 2e-2),
    ("gdn2_bf16_c16", dict(B=1, H=2, T=128, dk=128, dv=128, chunk=16), 2e-2),
    ("gdn_scalar_bf16", dict(B=2, H=2, T=256, dk=128, dv=128, alpha_mode="scalar", b_mode="scalar",
                             w_mode="scalar", tied=True, s0_std=None), 2e-2),
    ("kda_bf16", dict(B=1, H=3, T=192, dk=128, dv=128, b_mode="scalar", w_mode="scalar",
                      tied=True), 2e-2),
    ("b_only_channel", dict(B=1, H=2, T=192, dk=64, dv=64, w_mode="scalar"), 2e-2),
    ("w_only_channel", dict(B=1, H=2, T=192, dk=64, dv=64, b_mode="scalar"), 2e-2),
    ("d64_c64", dict(B=2, H=2, T=256, dk=64, dv=64), 2e-2),
    ("d32_c32", dict(B=2, H=2, T=160, dk=32, dv=32, chunk=32), 2e-2),
    ("d16_c16", dict(B=2, H=2, T=96, dk=16, dv=16, chunk=16), 2e-2),
    ("dk64_dv128", dict(B=1, H=2, T=192, dk=64, dv=128), 2e-2),
    ("dk128_dv64", dict(B=1, H=2, T=192, dk=128, dv=64), 2e-2),
    ("erase_range_0_2", dict(B=1, H=2, T=256, dk=128, dv=128, gate_hi=2.0), 2e-2),
    ("alpha_scalar_only", dict(B=1, H=2, T=128, dk=128, dv=128, alpha_mode="scalar"), 2e-2),
    ("alpha_scalar_b_scalar", dict(B=1, H=2, T=128, dk=128, dv=128, alpha_mode="scalar",
                                   b_mode="scalar"), 2e-2),
    ("alpha_scalar_w_scalar", dict(B=1, H=2, T=128, dk=128, dv=128, alpha_mode="scalar",
                                   w_mode="scalar"), 2e-2),
    ("b_w_scalar_untied", dict(B=1, H=2, T=128, dk=128, dv=128, b_mode="scalar",
                               w_mode="scalar"), 2e-2),
    ("single_chunk", dict(B=3, H=1, T=64, dk=128, dv=128), 2e-2),
    ("two_chunks", dict(B=1, H=1, T=128, dk=128, dv=128), 2e-2),
    ("f32_d128_c64", dict(B=1, H=2, T=256, dk=128, dv=128, act="f32"), 1e-4),
    ("f32_d128_c32", dict(B=1, H=2, T=160, dk=128, dv=128, act="f32", chunk=32), 1e-4),
    ("f32_d64_c64", dict(B=1, H=2, T=192, dk=64, dv=64, act="f32"), 1e-4),
    ("f32_d32_c64", dict(B=2, H=2, T=192, dk=32, dv=32, act="f32"), 1e-4),
    ("f32_dk128_dv64", dict(B=1, H=2, T=128, dk=128, dv=64, act="f32", chunk=32), 1e-4),
    ("f32_scalar_gdn", dict(B=1, H=2, T=128, dk=128, dv=128, act="f32", alpha_mode="scalar",
                            b_mode="scalar", w_mode="scalar", tied=True), 1e-4),
    ("f32_strong_decay", dict(B=1, H=2, T=128, dk=64, dv=64, act="f32", chunk=32,
                              decay_scale=0.5), 1e-4),
    ("bf16_strong_decay_c16", dict(B=1, H=2, T=128, dk=64, dv=64, chunk=16, decay_scale=0.5), 2e-2),
]


@pytest.mark.parametrize("path", ["auto", "fused"])
@pytest.mark.parametrize("name,kw,tol", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases(name, kw, tol, path):
    """path "auto" runs the two-pass kernels where they apply (bf16, chunk 64,
    d in {64, 128}); "fused" runs the single-kernel path on every case."""
    inp = _case(name, **kw)
    o, sf = _run(inp, path=path)
    _check(inp, o, sf, tol)


GENERIC = [
    ("gdn2_generic", dict(B=2, H=2, T=256, dk=128, dv=128)),
    ("gdn_generic", dict(B=1, H=2, T=192, dk=128, dv=128, alpha_mode="scalar", b_mode="scalar",
                         w_mode="scalar", tied=True, s0_std=None)),
    ("d64_generic", dict(B=1, H=3, T=128, dk=64, dv=64)),
]


@pytest.mark.parametrize("name,kw", GENERIC, ids=[c[0] for c in GENERIC])
def test_generic_kernel_matches_oracle_and_pipelined(name, kw):
    """The single-role kernel (selected by GDR_FWD_GENERIC) on shapes the
    pipelined kernel also serves: both meet the tolerance, and they agree."""
    inp = _case(name, **kw)
    og, sg = _run(inp, generic=True)
    _check(inp, og, sg, 2e-2)
    for path in ("fused", "auto"):
        op, sp = _run(inp, path=path)
        assert rel_err(og.cpu().numpy(), op.cpu().numpy()) <= 1e-2, path
        assert rel_err(sg.cpu().numpy(), sp.cpu().numpy()) <= 1e-2, path


def test_zero_initial_state_pointer_equals_zeros():
    import torch
    inp = _case("s0_none", B=1, H=2, T=128, dk=128, dv=128, s0_std=None)
    o1, s1 = _run(inp)
    z = torch.zeros((1, 2, 128, 128), dtype=torch.float32, device="cuda")
    o2, s2 = _run(inp, S0=z)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    _check(inp, o1, s1, 2e-2)


def test_bf16_output_is_rounded_fp32_output():
    import torch
    inp = _case("bf16_out", B=1, H=2, T=192, dk=128, dv=128)
    o32, s32 = _run(inp)
    o16, s16 = _run(inp, out_dtype=torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(s32, s16)


@pytest.mark.parametrize("two_pass", [False, True])
def test_state_may_alias_initial_state(two_pass):
    import torch
    import gated_delta_rule_24_amd as gdr
    inp = _case("alias", B=2, H=2, T=128, dk=128, dv=128)
    o_ref, s_ref = _run(inp, path="auto" if two_pass else "fused")
    d = to_dev(inp)
    S = d["S0"].clone()
    o = torch.empty_like(o_ref)
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    nbytes = gdr.gdr_chunk_fwd_workspace_bytes(2, 2, 128, 128, 128, 64, flags) if two_pass else 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if two_pass else None
    gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S, o, S,
                      2, 2, 128, 128, 128, 64, flags, ws, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, s_ref)


def test_workspace_reused_across_calls():
    """One workspace serves a large call and then a smaller one; both match
    the oracle (the contents on entry are ignored)."""
    import torch
    import gated_delta_rule_24_amd as gdr
    big = _case("ws_big", B=2, H=2, T=256, dk=128, dv=128)
    small = _case("ws_small", B=1, H=1, T=128, dk=128, dv=128, seed=3)
    nbytes = gdr.gdr_chunk_fwd_workspace_bytes(2, 2, 256, 128, 128, 64, 0)
    ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device="cuda")
    for inp in (big, small):
        d = to_dev(inp)
        o = torch.empty((inp.B, inp.H, inp.T, inp.dv), device="cuda")
        sf = torch.empty((inp.B, inp.H, inp.dk, inp.dv), device="cuda")
        gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], o, sf,
                          inp.B, inp.H, inp.T, inp.dk, inp.dv, 64, 0, ws, nbytes)
        torch.cuda.synchronize()
        _check(inp, o, sf, 2e-2)


def test_two_pass_and_fused_paths_agree():
    inp = _case("paths", B=2, H=3, T=320, dk=128, dv=128)
    oa, sa = _run(inp, path="auto")
    of, sf_ = _run(inp, path="fused")
    assert rel_err(oa.cpu().numpy(), of.cpu().numpy()) <= 1e-2
    assert rel_err(sa.cpu().numpy(), sf_.cpu().numpy()) <= 1e-2


def test_empty_sequence_copies_state():
    import torch
    import gated_delta_rule_24_amd as gdr
    S0 = torch.randn(2, 3, 64, 64, device="cuda")
    Sf = torch.full_like(S0, 7.0)
    e = torch.empty(0, device="cuda", dtype=torch.bfloat16)
    o = torch.empty(0, device="cuda")
    gdr.gdr_chunk_fwd(e, e, e, o, e, e, S0, o, Sf, 2, 3, 0, 64, 64, 64, 0)
    torch.cuda.synchronize()
    assert torch.equal(Sf, S0)


def test_deterministic_bitwise():
    import torch
    inp = _case("det", B=2, H=2, T=256, dk=128, dv=128)
    o1, s1 = _run(inp)
    o2, s2 = _run(inp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_chunk_size_invariance():
    inp = _case("chunks", B=1, H=2, T=256, dk=128, dv=128)
    outs = {c: _run(inp, chunk=c) for c in (16, 32, 64)}
    for c, (o, sf) in outs.items():
        _check(inp, o, sf, 2e-2)
    o64 = outs[64][0].cpu().numpy()
    for c in (16, 32):
        assert rel_err(outs[c][0].cpu().numpy(), o64) <= 2e-2


def test_split_sequence_continuity():
    """fwd(T) equals fwd(T1) followed by fwd(T - T1) starting from its state."""
    import torch
    import gated_delta_rule_24_amd as gdr
    inp = _case("split", B=1, H=2, T=256, dk=128, dv=128)
    d = to_dev(inp)
    o, sf = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    h = lambda t: t[:, :, :128].contiguous()
    t2 = lambda t: t[:, :, 128:].contiguous()
    o1, s1 = gdr.chunk_fwd(*(h(d[n]) for n in ("q", "k", "v", "log_alpha", "b", "w")), d["S0"])
    o2, s2 = gdr.chunk_fwd(*(t2(d[n]) for n in ("q", "k", "v", "log_alpha", "b", "w")), s1)
    torch.cuda.synchronize()
    assert rel_err(torch.cat([o1, o2], 2).cpu().numpy(), o.cpu().numpy()) <= 1e-5
    assert rel_err(s2.cpu().numpy(), sf.cpu().numpy()) <= 1e-5


STRONG = [
    # decay_scale s: log alpha = -softplus(N(0,1)) * s per channel (0.05 in the
    # pages' workloads); about 0.8 s nats per token on average
    ("channel_0.5", dict(B=1, H=2, T=256, dk=128, dv=128, decay_scale=0.5)),
    ("channel_2", dict(B=1, H=2, T=256, dk=128, dv=128, decay_scale=2.0)),
    ("channel_2_d64", dict(B=2, H=1, T=192, dk=64, dv=64, decay_scale=2.0)),
    # Gated DeltaNet with a data-dependent gate alpha = sigmoid(z), z ~ N(0,1):
    # log alpha = log sigmoid(z) has the law of -softplus(N(0,1))
    ("gdn_sigmoid_gate", dict(B=1, H=2, T=256, dk=128, dv=128, alpha_mode="scalar", b_mode="scalar",
                              w_mode="scalar", tied=True, decay_scale=1.0)),
    # about 16 nats per token: every factor of a distant pair underflows
    ("channel_20", dict(B=1, H=2, T=192, dk=128, dv=128, decay_scale=20.0)),
    ("mixed_scalar_alpha_2", dict(B=1, H=2, T=192, dk=128, dv=64, alpha_mode="scalar",
                                  decay_scale=2.0)),
]


@pytest.mark.parametrize("name,kw", STRONG, ids=[c[0] for c in STRONG])
def test_strong_decay_two_pass(name, kw):
    """The two-pass forward gives values (not NaN) for any decay: every operand
    factor is e^{-x} with x >= 0, and blocks of strong decay take their
    diagonal tiles from exact per-element factors."""
    inp = _case(name, **kw)
    o, sf = _run(inp)
    _check(inp, o, sf, 2e-2)


STRONG_FUSED = STRONG + [
    ("channel_2_f32", dict(B=1, H=2, T=128, dk=64, dv=64, decay_scale=2.0, act="f32")),
    ("channel_2_d32x16_c16", dict(B=2, H=1, T=96, dk=32, dv=16, decay_scale=2.0, chunk=16)),
]


@pytest.mark.parametrize("name,kw", STRONG_FUSED, ids=[c[0] for c in STRONG_FUSED])
def test_strong_decay_single_kernel(name, kw):
    """Without a workspace the single-kernel forward runs; it references a
    chunk's decay to the chunk's end, and a head whose decay leaves its
    operand range is recomputed token by token in fp32, so the outputs are
    values for any decay (tolerance 1e-4 with fp32 activations)."""
    inp = _case(name, **kw)
    o, sf = _run(inp, path="fused")
    _check(inp, o, sf, 1e-4 if inp.act == "f32" else 2e-2)


def test_strong_decay_leaves_other_heads_to_the_chunk_kernel():
    """One head with strong decay among heads within range: the token-level
    recompute rewrites that head only; the others keep the chunk kernel's
    result bit for bit."""
    import torch
    import gated_delta_rule_24_amd as gdr
    from tests.helpers import to_dev
    inp = _case("mixed_heads", B=1, H=3, T=192, dk=64, dv=64)
    strong = gs.make_inputs(1, 1, 192, 64, 64, decay_scale=2.0, seed=9)
    inp.arrays["log_alpha"][:, 1] = strong.arrays["log_alpha"][:, 0]
    d = to_dev(inp)
    o, sf = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], path="fused")
    torch.cuda.synchronize()
    _check(inp, o, sf, 2e-2)
    # heads 0 and 2 alone, with the same inputs
    keep = [0, 2]
    d2 = {n: (None if t is None else t[:, keep].contiguous()) for n, t in d.items()}
    o2, s2 = gdr.chunk_fwd(d2["q"], d2["k"], d2["v"], d2["log_alpha"], d2["b"], d2["w"], d2["S0"], path="fused")
    torch.cuda.synchronize()
    assert torch.equal(o[:, keep], o2) and torch.equal(sf[:, keep], s2)


@pytest.mark.parametrize("name,kw", [
    ("gdn2_c64", dict(B=2, H=5, T=640, dk=128, dv=128)),
    ("d64", dict(B=3, H=3, T=384, dk=64, dv=64, alpha_mode="scalar")),
    ("d128x64", dict(B=1, H=9, T=256, dk=128, dv=64, b_mode="scalar", w_mode="scalar", tied=True)),
    ("d64x128_strong", dict(B=1, H=2, T=256, dk=64, dv=128, decay_scale=2.0)),
    # 80 heads of 24 chunks: three batches of chained heads per XCD, the
    # producers following the batches
    ("three_batches", dict(B=4, H=20, T=1536, dk=128, dv=128)),
])
def test_persistent_and_split_kernels_agree_bitwise(name, kw):
    """The persistent kernel (producers and chains side by side, records handed
    over through the L2 with per-chunk flags) gives bit for bit the result of
    running the two roles as two kernels, one after the other."""
    import torch
    inp = _case(name, **kw)
    o1, s1 = _run(inp)
    o2, s2 = _run(inp, path="split")
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    _check(inp, o1, s1, 2e-2)


@pytest.mark.parametrize("path", ["auto", "split", "fused"])
def test_forward_replays_from_a_graph(path):
    """The fixed-length forward captured into a graph (persistent kernel: the
    flag-clearing kernel and the producer/chain kernel; or the two-kernel form;
    or the single kernel without a workspace) replays to the eager result bit
    for bit, on several replays with eager work and synchronisations between
    them, and the eager result matches the oracle."""
    import torch
    import gated_delta_rule_24_amd as gdr
    inp = _case("graph_fwd", B=2, H=3, T=320, dk=128, dv=128)
    d = to_dev(inp)

    def run():
        return gdr.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"],
                             chunk=64, path=path)
    eager = run()
    torch.cuda.synchronize()
    _check(inp, eager[0], eager[1], 2e-2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = run()
    for rep in range(3):
        x = torch.randn(1 << 20, device="cuda")
        x.mul_(2.0)
        captured[0].fill_(float("nan"))      # the replay must write every output again
        captured[1].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(captured[0], eager[0]) and torch.equal(captured[1], eager[1]), rep


def test_many_heads_take_several_chain_batches():
    """More heads than chain workgroups per XCD: the chains of an XCD run in
    batches, and the producers follow the batches."""
    inp = _case("many_heads", B=8, H=40, T=128, dk=64, dv=64)
    o, sf = _run(inp)
    _check(inp, o, sf, 2e-2)


def test_gdn2_full_workload_all_heads():
    """Gated DeltaNet-2 at B=2, H=16, T=8192, d=128, chunk 64 (the timed
    launch), every output of every head against the oracle."""
    inp = _case("gdn2")
    o, sf = _run(inp)
    _check(inp, o, sf, 2e-2)


def test_gdn_full_workload_all_heads():
    """Gated DeltaNet (scalar gates) at B=4, H=16, T=2048, d=128, every head."""
    inp = _case("gdn")
    o, sf = _run(inp)
    _check(inp, o, sf, 2e-2)



def _full_erase(inp, repeat_key=False):
    """b = 2 on every channel of every token (the end of the expanded erase
    range, where the erase factor reflects along k); optionally the same key
    at every token of a head, the worst case for the in-chunk solve."""
    a = inp.arrays
    a["b"] = np.full_like(a["b"], 2.0)
    if repeat_key:
        a["k"] = np.ascontiguousarray(np.broadcast_to(a["k"][:, :, :1], a["k"].shape))
    return inp


@pytest.mark.parametrize("path", ["auto", "fused"])
def test_full_erase_gate(path):
    """b = 2 everywhere with model-like (random unit) keys: within the bf16
    tolerance on both forward paths."""
    inp = _full_erase(_case("full_erase", B=1, H=2, T=256, dk=128, dv=128))
    o, sf = _run(inp, path=path)
    _check(inp, o, sf, 2e-2)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_full_erase_repeated_key_fp32(chunk):
    """One key repeated through every token at b = 2: inside a chunk the
    solution of (I + A) U = X - E S' alternates in sign with entries about
    2 sqrt(C) times |x|, which the state update then sums back to O(|x|).
    That cancellation amplifies rounding by about two orders of magnitude: f16
    operands lose about 10% (bf16 activations: 0.10-0.15 at chunks 16-64).
    Such inputs need fp32 activations. This stress case is not one of the
    pages' workloads, for which the fp32 tolerance is 1e-4; it is held to
    1e-3 here (measured about 1e-4)."""
    inp = _full_erase(_case("full_erase_rk", B=1, H=2, T=256, dk=128, dv=128, act="f32",
                            chunk=chunk), repeat_key=True)
    o, sf = _run(inp)
    _check(inp, o, sf, 1e-3)
