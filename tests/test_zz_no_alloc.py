"""gdr_chunk_fwd_noalloc (the forward without a caller workspace or any
allocation) against gdr_chunk_fwd with a caller workspace: two calls in a
row, the second smaller, each bit for bit equal to the workspace call and
within the bf16 tolerance of the oracle.  The array it uses keeps the first
call's contents when the second runs."""
import ctypes

import numpy as np
import pytest

import gdr_synth as gs
from tests.helpers import oracle_fwd, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _pair(B, H, T, seed):
    import torch
    import gated_delta_rule_24_amd as gdr
    inp = gs.make_inputs(B, H, T, 128, 128, seed=seed)
    d = to_dev(inp)
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    o_na = torch.full((B, H, T, 128), float("nan"), dtype=torch.float32, device="cuda")
    s_na = torch.full((B, H, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    need = gdr.gdr_chunk_fwd_workspace_bytes(B, H, T, 128, 128, 64, flags)
    assert 0 < need <= gdr.GDR_NOALLOC_SCRATCH_BYTES
    print(f"noalloc B={B} H={H} T={T} seed={seed} workspace {need} bytes", flush=True)
    gdr.gdr_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], o_na,
                              s_na, B, H, T, 128, 128, 64, flags)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ws = torch.empty_like(o_na)
    s_ws = torch.empty_like(s_na)
    gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], o_ws, s_ws,
                      B, H, T, 128, 128, 64, flags, ws, need)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ws) and torch.equal(s_na, s_ws)
    o_ref, s_ref = oracle_fwd(inp)
    eo = rel_err(o_na.cpu().numpy().reshape(B * H, T, 128), o_ref)
    es = rel_err(s_na.cpu().numpy().reshape(B * H, 128, 128), s_ref)
    print(f"  err o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2


def test_noalloc_matches_workspace_call_twice():
    _pair(2, 3, 1024, seed=11)       # 96 chunks
    _pair(1, 2, 192, seed=12)        # then a smaller call on the same array


def test_noalloc_rejects_calls_beyond_its_array():
    import gated_delta_rule_24_amd as gdr
    lib = gdr.lib()
    A = ctypes.c_void_p(0x10000)
    # 16 x 64 chunks of 64 tokens at d = 128 need more than the array holds
    st = lib.gdr_chunk_fwd_noalloc(A, A, A, A, A, A, None, A, None, 1, 16, 64 * 64, 128, 128, 64, 0,
                                   None)
    assert st == 3
