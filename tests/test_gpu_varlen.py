"""GPU parity of gdr_chunk_fwd_varlen (packed variable-length sequences)
against the fp64 token-recurrence oracle run on each sequence by itself.

Every sequence starts from its own S0 and no state crosses a sequence
boundary, so the expected output of the packed call is the oracle's forward
of each sequence's token range, concatenated.  The lengths mix empty
sequences, single tokens, lengths one below, at and one above a chunk of 64,
and several chunks with a ragged tail.  Tolerance as for the fixed-length
forward with bf16 activations: max|Δ|/rms(ref) <= 2e-2, separately for o
and S_final."""
import numpy as np
import pytest

import gdr_synth as gs
import oracle
from tests.helpers import rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _dev(inp):
    """Packed arrays on the GPU: [H, T, ...] activations, S0 [nseq, H, dk, dv]."""
    import torch
    a = inp.arrays
    out = {}
    for n in ("q", "k", "v", "log_alpha", "b", "w"):
        dt = torch.float32 if n == "log_alpha" else torch.bfloat16
        out[n] = torch.from_numpy(np.ascontiguousarray(a[n][0])).to(dt).cuda()
    if a["b"] is a["w"]:
        out["w"] = out["b"]
    out["S0"] = None if a["S0"] is None else torch.from_numpy(a["S0"]).cuda()
    out["cu"] = torch.from_numpy(a["cu_seqlens"]).cuda()
    return out


def _oracle(inp):
    """o [H, T, dv] and S_final [nseq, H, dk, dv] from one oracle call per sequence."""
    a = inp.arrays
    cu = a["cu_seqlens"]
    nseq = len(cu) - 1
    H, T, dk, dv = inp.H, inp.T, inp.dk, inp.dv
    o = np.zeros((H, T, dv))
    sf = np.zeros((nseq, H, dk, dv))
    for s in range(nseq):
        lo, hi = int(cu[s]), int(cu[s + 1])
        s0 = None if a["S0"] is None else a["S0"][s]
        if hi == lo:
            if s0 is not None:
                sf[s] = s0
            continue

        def sl(x):
            return x[0][:, lo:hi]
        o_s, sf[s] = oracle.fwd(sl(a["q"]), sl(a["k"]), sl(a["v"]), sl(a["log_alpha"]),
                                sl(a["b"]), sl(a["w"]), s0)
        o[:, lo:hi] = o_s
    return o, sf


def _run(inp, **kw):
    import torch
    import gated_delta_rule_24_amd as gdr
    d = _dev(inp)
    o, sf = gdr.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"],
                                 d["cu"], d["S0"], **kw)
    torch.cuda.synchronize()
    return o, sf


def _check(inp, o, sf):
    o_ref, s_ref = _oracle(inp)
    eo = rel_err(o.float().cpu().numpy(), o_ref) if inp.T else 0.0
    es = rel_err(sf.cpu().numpy(), s_ref)
    print(f"  err o={eo:.3e} S={es:.3e} (tol {TOL})", flush=True)
    assert eo <= TOL and es <= TOL, (eo, es)


def _case(name, lengths, **kw):
    shown = lengths if len(lengths) <= 12 else f"{len(lengths)} sequences, {sum(lengths)} tokens"
    print(f"varlen case {name} lengths={shown} {kw}", flush=True)
    return gs.packed_inputs(lengths, **kw)


CASES = [
    ("mixed_d128", [0, 1, 63, 64, 65, 200, 130, 0], dict(H=2, dk=128, dv=128)),
    ("gdn_scalar_tied_d64", [17, 300, 64, 5, 129],
     dict(H=3, dk=64, dv=64, alpha_mode="scalar", b_mode="scalar", w_mode="scalar", tied=True)),
    ("dk128_dv64", [100, 28, 191], dict(H=2, dk=128, dv=64)),
    ("dk64_dv128", [70, 1, 256], dict(H=2, dk=64, dv=128)),
    ("alpha_scalar", [90, 150, 33], dict(H=2, dk=128, dv=128, alpha_mode="scalar")),
    ("b_scalar_w_channel", [127, 129], dict(H=2, dk=128, dv=128, b_mode="scalar")),
    ("w_scalar_b_channel", [64, 64, 1], dict(H=2, dk=64, dv=64, w_mode="scalar")),
    ("erase_range_0_2", [150, 77], dict(H=2, dk=128, dv=128, gate_hi=2.0)),
    ("zero_initial_state", [40, 200], dict(H=2, dk=128, dv=128, s0_std=None)),
    ("one_long", [1000], dict(H=1, dk=128, dv=128)),
    ("all_single_tokens", [1] * 37, dict(H=2, dk=64, dv=64)),
    # decay beyond the chunk kernels' operand range: recomputed token by token
    ("strong_decay", [150, 77, 1, 0, 64], dict(H=2, dk=128, dv=128, decay_scale=2.0)),
    ("strong_decay_gdn_d64", [90, 33], dict(H=2, dk=64, dv=64, alpha_mode="scalar", b_mode="scalar",
                                          w_mode="scalar", tied=True, decay_scale=1.0)),
]


@pytest.mark.parametrize("name,lengths,kw", CASES, ids=[c[0] for c in CASES])
def test_packed_matches_per_sequence_oracle(name, lengths, kw):
    inp = _case(name, lengths, **kw)
    o, sf = _run(inp)
    _check(inp, o, sf)


def test_many_short_sequences():
    """More sequences than the chunk-offset scan has threads (1024), every
    seventh one empty."""
    lengths = [0 if i % 7 == 0 else n for i, n in enumerate(gs.packed_lengths(1500, 20, seed=3))]
    inp = _case("many_short", lengths, H=1, dk=64, dv=64, seed=3)
    o, sf = _run(inp)
    _check(inp, o, sf)


def test_empty_batch_copies_initial_state():
    import torch
    inp = _case("empty", [0, 0, 0], H=2, dk=128, dv=128)
    o, sf = _run(inp)
    assert o.numel() == 0
    assert torch.equal(sf.cpu(), torch.from_numpy(inp.arrays["S0"]))


def test_equal_lengths_match_fixed_length_forward():
    """Three sequences of 256 tokens: the packed call and the batched
    fixed-length call agree (both within the bf16 tolerance of the oracle;
    their kernels reference a chunk's decay differently, so their rounding
    differs)."""
    import torch
    import gated_delta_rule_24_amd as gdr
    nseq, L, H = 3, 256, 2
    inp = _case("equal_lengths", [L] * nseq, H=H, dk=128, dv=128)
    d = _dev(inp)
    o_p, s_p = gdr.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"],
                                    d["cu"], d["S0"])

    def batched(x):       # [H, nseq*L, ...] -> [nseq, H, L, ...]
        return x.reshape((H, nseq, L) + tuple(x.shape[2:])).transpose(0, 1).contiguous()
    o_f, s_f = gdr.chunk_fwd(batched(d["q"]), batched(d["k"]), batched(d["v"]),
                             batched(d["log_alpha"]), batched(d["b"]), batched(d["w"]), d["S0"],
                             chunk=64, path="auto")
    torch.cuda.synchronize()
    assert rel_err(batched(o_p).cpu().numpy(), o_f.cpu().numpy()) <= 2e-2
    assert rel_err(s_p.cpu().numpy(), s_f.cpu().numpy()) <= 2e-2
    _check(inp, o_p, s_p)


def test_final_state_may_alias_initial_state():
    import torch
    import gated_delta_rule_24_amd as gdr
    inp = _case("alias", [65, 130, 0, 7], H=2, dk=128, dv=128)
    d = _dev(inp)
    o_ref, s_ref = gdr.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"],
                                        d["cu"], d["S0"])
    nseq, H, T = 4, 2, inp.T
    S = d["S0"].clone()
    o = torch.empty((H, T, 128), dtype=torch.float32, device="cuda")
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    nbytes = gdr.gdr_chunk_fwd_varlen_workspace_bytes(nseq, H, T, 128, 128, flags)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gdr.gdr_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S, o, S,
                             d["cu"], nseq, H, T, 128, 128, flags, ws, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, s_ref)


def test_bf16_output_is_rounded_fp32_output():
    import torch
    inp = _case("bf16_out", [100, 60], H=2, dk=128, dv=128)
    o32, s32 = _run(inp)
    o16, s16 = _run(inp, out_dtype=torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(s32, s16)


def test_final_state_not_requested():
    inp = _case("no_state", [90, 10], H=2, dk=64, dv=64)
    o, sf = _run(inp, return_state=False)
    assert sf is None
    o_ref, _ = _oracle(inp)
    assert rel_err(o.cpu().numpy(), o_ref) <= TOL


def test_packed_workload_shape_all_heads():
    """Eight documents per head row with long-tailed lengths around 2048
    tokens (about 16K tokens per head, 16 heads, d=128): every sequence's
    output and final state on every head against the oracle."""
    H = 16
    heads = list(range(H))
    lengths = gs.packed_lengths(8, 2048, seed=5)
    inp = _case("workload", lengths, H=H, dk=128, dv=128, seed=5)
    o, sf = _run(inp)
    a = inp.arrays
    cu = a["cu_seqlens"]
    o_np, sf_np = o.cpu().numpy()[heads], sf.cpu().numpy()[:, heads]
    for s in range(len(lengths)):
        lo, hi = int(cu[s]), int(cu[s + 1])

        def sl(x):
            return x[0][heads, lo:hi]
        o_s, s_s = oracle.fwd(sl(a["q"]), sl(a["k"]), sl(a["v"]), sl(a["log_alpha"]),
                              sl(a["b"]), sl(a["w"]), a["S0"][s][heads])
        es = rel_err(sf_np[s], s_s)
        eo = rel_err(o_np[:, lo:hi], o_s)
        print(f"  seq {s} len {hi - lo}: err o={eo:.3e} S={es:.3e}", flush=True)
        assert eo <= TOL and es <= TOL, (s, eo, es)
