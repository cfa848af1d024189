"""Out-of-bounds guards on the outputs of the C ABI calls.

Every output (and the workspace) is placed inside a larger allocation whose
padding on both sides holds a sentinel pattern; the interior is filled with
the same pattern before the call.  After the call the padding must be
untouched (no store past either end of a buffer) and the interior must equal,
bit for bit, the result of the same call on plain tensors (no element left
unwritten).  Shapes include partial chunks, empty sequences and single
tokens, where the kernels skip stores."""
import numpy as np
import pytest

import gdr_synth as gs

pytestmark = pytest.mark.gpu

PAD_BYTES = 4096


class Guarded:
    """A tensor of `shape` inside a sentinel-padded buffer."""

    def __init__(self, shape, dtype):
        import torch
        n = int(np.prod(shape)) if len(shape) else 1
        item = torch.empty((), dtype=dtype).element_size()
        pad = PAD_BYTES // item
        self.buf = torch.empty(n + 2 * pad, dtype=dtype, device="cuda")
        self.buf.view(torch.uint8).fill_(0xA5)
        self.ref = self.buf.clone()
        self.pad, self.n = pad, n
        self.t = self.buf[pad:pad + n].view(shape)

    def check(self, name):
        import torch
        lo = torch.equal(self.buf[:self.pad].view(torch.uint8), self.ref[:self.pad].view(torch.uint8))
        hi = torch.equal(self.buf[self.pad + self.n:].view(torch.uint8),
                         self.ref[self.pad + self.n:].view(torch.uint8))
        assert lo and hi, f"{name}: store outside the buffer (before: {not lo}, after: {not hi})"


def _same(name, g, ref):
    import torch
    assert torch.equal(g.t.view(torch.uint8), ref.contiguous().view(torch.uint8)), \
        f"{name}: differs from the unguarded call (an element left unwritten?)"


def _dev(a, names, packed):
    import torch
    out = {}
    for n in names:
        x = a[n] if n in a else None
        if x is None:
            out[n] = None
            continue
        if packed and n not in ("S0",):
            x = x[0]
        dt = torch.float32 if n in ("log_alpha", "S0") else torch.bfloat16
        out[n] = torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()
    return out


def test_fixed_length_forward_stays_in_bounds():
    import torch
    import gated_delta_rule_24_amd as gdr
    B, H, T, D = 2, 3, 192, 128
    print(f"canary fwd B={B} H={H} T={T} d={D}", flush=True)
    inp = gs.make_inputs(B, H, T, D, D, seed=21)
    d = _dev(inp.arrays, ("q", "k", "v", "log_alpha", "b", "w", "S0"), False)
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    o_ref, s_ref = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    for out_bf16 in (False, True):
        fl = flags | (gdr.GDR_OUT_BF16 if out_bf16 else 0)
        o = Guarded((B, H, T, D), torch.bfloat16 if out_bf16 else torch.float32)
        sf = Guarded((B, H, D, D), torch.float32)
        nb = gdr.gdr_chunk_fwd_workspace_bytes(B, H, T, D, D, 64, fl)
        ws = Guarded((nb,), torch.uint8)
        gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], o.t, sf.t,
                          B, H, T, D, D, 64, fl, ws.t, nb)
        torch.cuda.synchronize()
        for name, g in (("o", o), ("S_final", sf), ("workspace", ws)):
            g.check(name)
        _same("o", o, o_ref.to(torch.bfloat16) if out_bf16 else o_ref)
        _same("S_final", sf, s_ref)


LENGTHS = [65, 1, 130, 0, 63, 7]


def test_packed_forward_stays_in_bounds():
    import torch
    import gated_delta_rule_24_amd as gdr
    H, D = 2, 128
    print(f"canary packed fwd lengths={LENGTHS}", flush=True)
    inp = gs.packed_inputs(LENGTHS, H=H, dk=D, dv=D, seed=22)
    a = inp.arrays
    d = _dev(a, ("q", "k", "v", "log_alpha", "b", "w", "S0"), True)
    cu = torch.from_numpy(a["cu_seqlens"]).cuda()
    nseq, T = len(LENGTHS), sum(LENGTHS)
    o_ref, s_ref = gdr.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], cu, d["S0"])
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    o = Guarded((H, T, D), torch.float32)
    sf = Guarded((nseq, H, D, D), torch.float32)
    nb = gdr.gdr_chunk_fwd_varlen_workspace_bytes(nseq, H, T, D, D, flags)
    ws = Guarded((nb,), torch.uint8)
    gdr.gdr_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], o.t, sf.t,
                             cu, nseq, H, T, D, D, flags, ws.t, nb)
    torch.cuda.synchronize()
    for name, g in (("o", o), ("S_final", sf), ("workspace", ws)):
        g.check(name)
    _same("o", o, o_ref)
    _same("S_final", sf, s_ref)


def test_packed_backward_stays_in_bounds():
    import torch
    import gated_delta_rule_24_amd as gdr
    H, D = 2, 128
    print(f"canary packed bwd lengths={LENGTHS}", flush=True)
    inp = gs.packed_inputs(LENGTHS, H=H, dk=D, dv=D, seed=23, with_dO=True)
    a = inp.arrays
    d = _dev(a, ("q", "k", "v", "log_alpha", "b", "w", "dO", "S0"), True)
    cu = torch.from_numpy(a["cu_seqlens"]).cuda()
    nseq, T = len(LENGTHS), sum(LENGTHS)
    ref = gdr.chunk_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], cu, d["S0"], d["dO"])
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    g = {n: Guarded(tuple(ref[n].shape), torch.float32) for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")}
    nb = gdr.gdr_chunk_bwd_varlen_workspace_bytes(nseq, H, T, D, D, flags)
    ws = Guarded((nb,), torch.uint8)
    gdr.gdr_chunk_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], d["dO"], None,
                             g["dq"].t, g["dk"].t, g["dv"].t, g["dlog_alpha"].t, g["db"].t, g["dw"].t,
                             g["dS0"].t, cu, nseq, H, T, D, D, flags, ws.t, nb)
    torch.cuda.synchronize()
    ws.check("workspace")
    for n, x in g.items():
        x.check(n)
        _same(n, x, ref[n])


def test_decode_stays_in_bounds():
    import torch
    import gated_delta_rule_24_amd as gdr
    N, H, D = 3, 5, 128
    print(f"canary decode N={N} H={H} d={D}", flush=True)
    S0 = gs.decode_state(N, H, D, D, seed=24)
    tok = gs.decode_token(N, H, D, D, 0, seed=24)
    t = {n: torch.from_numpy(x).to(torch.float32 if n == "log_alpha" else torch.bfloat16).cuda()
         for n, x in tok.items()}
    S_ref = torch.from_numpy(S0).cuda()
    o_ref = gdr.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["b"], t["w"], S_ref)
    S = Guarded((N, H, D, D), torch.float32)
    S.t.copy_(torch.from_numpy(S0))
    o = Guarded((N, H, D), torch.float32)
    gdr.gdr_decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["b"], t["w"], S.t, o.t, N, H, D, D, 0)
    torch.cuda.synchronize()
    S.check("S")
    o.check("o")
    _same("S", S, S_ref)
    _same("o", o, o_ref)
