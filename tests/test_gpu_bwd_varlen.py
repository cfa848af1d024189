"""GPU parity of gdr_chunk_bwd_varlen (packed variable-length sequences)
against the oracle's fp64 reverse mode run on each sequence by itself.

Loss L = <dO, o> + <dS_final, S_final> summed over the sequences; every
sequence's gradients depend only on its own tokens, initial state and final
state gradient, so the expected result is the oracle's backward of each
sequence's token range, concatenated.  Tolerance as for the fixed-length
backward with bf16 activations: max|Δ|/rms(ref) <= 2e-2 per gradient tensor.
For a scalar gate the oracle's per-channel gradient is summed over the
broadcast axis."""
import numpy as np
import pytest

import gdr_synth as gs
import oracle
from tests.helpers import rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def _case(name, lengths, **kw):
    shown = lengths if len(lengths) <= 12 else f"{len(lengths)} sequences, {sum(lengths)} tokens"
    print(f"bwd varlen case {name} lengths={shown} {kw}", flush=True)
    return gs.packed_inputs(lengths, with_dO=True, **kw)


def _dsf(inp, seed=7):
    nseq = len(inp.arrays["cu_seqlens"]) - 1
    r = np.random.default_rng(seed)
    return (r.standard_normal((nseq, inp.H, inp.dk, inp.dv)) * 0.5).astype(np.float32)


def _dev(inp):
    import torch
    a = inp.arrays
    out = {}
    for n in ("q", "k", "v", "log_alpha", "b", "w", "dO"):
        dt = torch.float32 if n == "log_alpha" else torch.bfloat16
        out[n] = torch.from_numpy(np.ascontiguousarray(a[n][0])).to(dt).cuda()
    if a["b"] is a["w"]:
        out["w"] = out["b"]
    out["S0"] = None if a["S0"] is None else torch.from_numpy(a["S0"]).cuda()
    out["cu"] = torch.from_numpy(a["cu_seqlens"]).cuda()
    return out


def _run(inp, dSf=None):
    import torch
    import gated_delta_rule_24_amd as gdr
    d = _dev(inp)
    dsf = None if dSf is None else torch.from_numpy(dSf).cuda()
    g = gdr.chunk_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["cu"],
                             d["S0"], d["dO"], dsf)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in g.items()}


def _oracle(inp, dSf=None, heads=None):
    """Gradients of every sequence (on `heads`, all when None), packed as the
    library returns them."""
    a = inp.arrays
    cu = a["cu_seqlens"]
    nseq = len(cu) - 1
    hs = np.arange(inp.H) if heads is None else np.asarray(heads)
    nh, T, dk, dv = len(hs), inp.T, inp.dk, inp.dv
    ref = {n: np.zeros((nh, T, dk)) for n in ("dq", "dk", "dlog_alpha", "db")}
    ref.update({n: np.zeros((nh, T, dv)) for n in ("dv", "dw")})
    ref["dS0"] = np.zeros((nseq, nh, dk, dv))
    for s in range(nseq):
        lo, hi = int(cu[s]), int(cu[s + 1])
        dsf = None if dSf is None else dSf[s][hs]
        if hi == lo:
            if dsf is not None:
                ref["dS0"][s] = dsf
            continue

        def sl(x):
            return x[0][hs, lo:hi]
        s0 = None if a["S0"] is None else a["S0"][s][hs]
        g = oracle.bwd(sl(a["q"]), sl(a["k"]), sl(a["v"]), sl(a["log_alpha"]), sl(a["b"]),
                       sl(a["w"]), s0, sl(a["dO"]), dsf)
        for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
            ref[n][:, lo:hi] = g[n]
        ref["dS0"][s] = g["dS0"]
    if inp.alpha_mode == "scalar":
        ref["dlog_alpha"] = ref["dlog_alpha"].sum(-1)
    if inp.b_mode == "scalar":
        ref["db"] = ref["db"].sum(-1)
    if inp.w_mode == "scalar":
        ref["dw"] = ref["dw"].sum(-1)
    return ref


def _check(inp, got, ref, heads=None):
    errs = {}
    for n in GRADS:
        g = got[n]
        if heads is not None:
            g = g[:, np.asarray(heads)] if n == "dS0" else g[np.asarray(heads)]
        errs[n] = rel_err(g, ref[n]) if g.size else 0.0
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (tol {TOL})", flush=True)
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, bad


CASES = [
    # name, lengths, kwargs, with dS_final
    ("mixed_d128", [0, 1, 63, 64, 65, 200, 130, 0], dict(H=2, dk=128, dv=128), True),
    ("mixed_d128_no_dsf", [5, 64, 150], dict(H=2, dk=128, dv=128), False),
    ("gdn_scalar_tied_d64", [17, 300, 64, 5, 129],
     dict(H=3, dk=64, dv=64, alpha_mode="scalar", b_mode="scalar", w_mode="scalar", tied=True),
     True),
    ("gdn_scalar_tied_d128", [100, 28, 191],
     dict(H=2, dk=128, dv=128, alpha_mode="scalar", b_mode="scalar", w_mode="scalar", tied=True),
     False),
    ("alpha_scalar", [90, 150, 33], dict(H=2, dk=128, dv=128, alpha_mode="scalar"), True),
    ("b_scalar_w_channel", [127, 129], dict(H=2, dk=128, dv=128, b_mode="scalar"), False),
    ("w_scalar_b_channel", [64, 64, 1], dict(H=2, dk=64, dv=64, w_mode="scalar"), True),
    ("erase_range_0_2", [150, 77], dict(H=2, dk=128, dv=128, gate_hi=2.0), True),
    ("zero_initial_state", [40, 200], dict(H=2, dk=64, dv=64, s0_std=None), True),
    ("one_long", [1000], dict(H=1, dk=128, dv=128), True),
    ("all_single_tokens", [1] * 37, dict(H=2, dk=64, dv=64), True),
    # decay beyond the chunk kernels' operand range: recomputed token by token
    ("strong_decay", [150, 77, 1, 0, 64], dict(H=2, dk=128, dv=128, decay_scale=2.0), True),
    ("strong_decay_gdn_d64", [90, 33], dict(H=2, dk=64, dv=64, alpha_mode="scalar", b_mode="scalar",
                                          w_mode="scalar", tied=True, decay_scale=1.0), False),
]


@pytest.mark.parametrize("name,lengths,kw,dsf", CASES, ids=[c[0] for c in CASES])
def test_packed_backward_matches_per_sequence_oracle(name, lengths, kw, dsf):
    inp = _case(name, lengths, **kw)
    dSf = _dsf(inp) if dsf else None
    _check(inp, _run(inp, dSf), _oracle(inp, dSf))


def test_many_short_sequences():
    """More sequences than the chunk-offset scan has threads (1024), every
    seventh one empty."""
    lengths = [0 if i % 7 == 0 else n for i, n in enumerate(gs.packed_lengths(1500, 20, seed=3))]
    inp = _case("many_short", lengths, H=1, dk=64, dv=64, seed=3)
    dSf = _dsf(inp)
    _check(inp, _run(inp, dSf), _oracle(inp, dSf))


def test_empty_batch_passes_state_gradient():
    inp = _case("empty", [0, 0, 0], H=2, dk=128, dv=128)
    dSf = _dsf(inp)
    got = _run(inp, dSf)
    assert got["dq"].size == 0
    assert np.array_equal(got["dS0"], dSf)


def test_equal_lengths_match_fixed_length_backward():
    """Three sequences of 192 tokens: the packed backward and the batched
    fixed-length backward run the same arithmetic.  dq, dk, dv and dS0 agree
    exactly; the packed kernel skips the stores of rows past a sequence's end
    with branches, so the compiler may fuse the multiply-adds of the
    element-wise gate gradients differently, and those agree to rounding."""
    import torch
    import gated_delta_rule_24_amd as gdr
    nseq, L, H = 3, 192, 2
    inp = _case("equal_lengths", [L] * nseq, H=H, dk=128, dv=128)
    dSf = _dsf(inp)
    got = _run(inp, dSf)
    d = _dev(inp)

    def batched(x):       # [H, nseq*L, ...] -> [nseq, H, L, ...]
        return x.reshape((H, nseq, L) + tuple(x.shape[2:])).transpose(0, 1).contiguous()
    g = gdr.chunk_bwd(batched(d["q"]), batched(d["k"]), batched(d["v"]), batched(d["log_alpha"]),
                      batched(d["b"]), batched(d["w"]), d["S0"], batched(d["dO"]),
                      torch.from_numpy(dSf).cuda(), chunk=64)
    torch.cuda.synchronize()
    for n in GRADS:
        ref = (g[n] if n == "dS0" else g[n].transpose(0, 1).reshape(got[n].shape)).cpu().numpy()
        if n in ("dlog_alpha", "db", "dw"):
            e = rel_err(got[n], ref)
            print(f"  {n}: packed vs batched {e:.2e}", flush=True)
            assert e <= 1e-5, (n, e)
        else:
            assert np.array_equal(got[n], ref), n
    _check(inp, got, _oracle(inp, dSf))


def test_packed_backward_workload_shape_all_heads():
    """Eight documents per head row with long-tailed lengths around 2048
    tokens (about 16K tokens per head, 16 heads, d=128): every gradient of
    every head against the oracle."""
    heads = list(range(16))
    lengths = gs.packed_lengths(8, 2048, seed=5)
    inp = _case("workload", lengths, H=16, dk=128, dv=128, seed=5)
    dSf = _dsf(inp)
    _check(inp, _run(inp, dSf), _oracle(inp, dSf, heads=heads), heads=heads)


def test_packed_calls_replay_from_a_graph():
    """The packed forward and backward (prep kernels, the two chains on two
    streams) captured into one graph replay to the eager results, bit for bit,
    on several replays with eager work between them."""
    import torch
    import gated_delta_rule_24_amd as gdr
    inp = _case("graph", [5, 64, 130, 0, 77], H=2, dk=128, dv=128)
    d = _dev(inp)
    dsf = torch.from_numpy(_dsf(inp)).cuda()

    def run():
        o, sf = gdr.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["cu"],
                                     d["S0"])
        g = gdr.chunk_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["cu"],
                                 d["S0"], d["dO"], dsf)
        return dict(o=o, sf=sf, **g)
    eager = run()
    torch.cuda.synchronize()
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
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in eager:
            assert torch.equal(captured[n], eager[n]), (rep, n)
