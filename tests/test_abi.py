"""The C ABI library: it loads, exports every function include/gdr.h
declares, and rejects invalid arguments before touching a device (so these
run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "gdr.h")


def _lib():
    import gated_delta_rule_24_amd as g
    if not os.path.exists(g.LIB_PATH):
        import gated_delta_rule_24_amd.build as b
        b.build(verbose=False)
    return g.lib()


def declared_functions():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("gdr_chunk_fwd", "gdr_decode_step", "gdr_chunk_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    import gated_delta_rule_24_amd as g
    assert set(declared_functions()) == set(g.EXPORTED_SYMBOLS)


def test_abi_version_and_status_strings():
    lib = _lib()
    assert lib.gdr_abi_version() == 2
    for s in range(6):
        assert len(lib.gdr_status_string(s)) > 0
    assert lib.gdr_status_string(99) == b"unknown status"


A = ctypes.c_void_p(0x10000)      # aligned fake pointer: never dereferenced
MIS = ctypes.c_void_p(0x10004)    # misaligned


def _fwd(lib, **kw):
    args = dict(q=A, k=A, v=A, la=A, b=A, w=A, S0=None, o=A, Sf=None, B=1, H=1, T=64, dk=128,
                dv=128, chunk=64, flags=0)
    args.update(kw)
    return lib.gdr_chunk_fwd(args["q"], args["k"], args["v"], args["la"], args["b"], args["w"],
                             args["S0"], args["o"], args["Sf"], args["B"], args["H"], args["T"],
                             args["dk"], args["dv"], args["chunk"], args["flags"], args.get("ws"),
                             args.get("nbytes", 0), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(w=None), 1),
    (dict(chunk=48), 1), (dict(T=100), 1), (dict(B=0), 1), (dict(T=-64), 1),
    (dict(flags=0x100), 1), (dict(k=MIS), 1), (dict(Sf=MIS), 1),
    (dict(dk=96), 2), (dict(dv=256), 2), (dict(dk=16, dv=96), 2),
])
def test_fwd_argument_validation(kw, status):
    assert _fwd(_lib(), **kw) == status


def test_fwd_workspace_query_and_validation():
    lib = _lib()
    one = lib.gdr_chunk_fwd_workspace_bytes(1, 1, 64, 128, 128, 64, 0)
    # per chunk of 64 tokens a record (W, Kh^T, U', Q_s as 64 x 128 f16, P as
    # 64 x 64 f16, 1 KiB of decay), then one int32 flag per chunk (padded to 64)
    # and 64 int32 control words
    rec = 4 * 64 * 128 * 2 + 64 * 64 * 2 + 1024
    assert one == rec + (64 + 64) * 4
    assert lib.gdr_chunk_fwd_workspace_bytes(2, 3, 256, 128, 128, 64, 0) == 2 * 3 * 4 * rec + (64 + 64) * 4
    assert lib.gdr_chunk_fwd_workspace_bytes(1, 40, 6400, 128, 128, 64, 0) == 4000 * rec + (4032 + 64) * 4
    assert lib.gdr_chunk_fwd_workspace_bytes(1, 1, 64, 128, 128, 64, 0x1) == 0   # fp32: fused only
    assert lib.gdr_chunk_fwd_workspace_bytes(1, 1, 64, 128, 128, 32, 0) == 0
    assert lib.gdr_chunk_fwd_workspace_bytes(1, 1, 64, 32, 32, 64, 0) == 0
    assert lib.gdr_chunk_fwd_workspace_bytes(1, 1, 0, 128, 128, 64, 0) == 0
    assert lib.gdr_chunk_fwd_workspace_bytes(1, 1, 64, 128, 128, 64, 0x20) == 0  # forced fused
    assert _fwd(lib, ws=A, nbytes=one - 1) == 3
    assert _fwd(lib, ws=MIS, nbytes=one) == 1


def test_decode_argument_validation():
    lib = _lib()
    ok = dict(q=A, k=A, v=A, la=A, b=A, w=A, S=A, o=A, N=4, H=2, dk=128, dv=128, flags=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.gdr_decode_step(a["q"], a["k"], a["v"], a["la"], a["b"], a["w"], a["S"],
                                   a["o"], a["N"], a["H"], a["dk"], a["dv"], a["flags"], None)
    assert call(S=None) == 1
    assert call(N=0) == 1
    assert call(o=MIS) == 1
    assert call(flags=0x100) == 1
    assert call(flags=0x80) == 1         # a forward-only flag
    assert call(dk=48) == 2


def _exact(T, dk, dv):
    """Workspace of one unit of the backward's token-by-token recompute (run for
    heads whose decay leaves the chunk kernels' operand range): fp32 state
    checkpoints every 64 tokens, then the states of one 64-token segment."""
    return ((T + 63) // 64 + 64) * dk * dv * 4


def test_bwd_workspace_query_and_validation():
    lib = _lib()
    q = lib.gdr_chunk_bwd_workspace_bytes
    # the two-pass path: decayed chunk-start states and chunk-end gradients as f16
    # (2 x B*H x T/chunk x d_k x d_v x 2 bytes), plus the forward's records, each
    # extended by three 64 x d_k and two 64 x 64 f16 operand layouts for the
    # backward passes; at least one unit of the token-by-token recompute
    states = 2 * 2 * 2 * 128 * 128 * 2
    # the backward's own records: W, Kh^T, U', Q', P (f16) and the decay slot
    records = 2 * 2 * (4 * 64 * 128 * 2 + 64 * 64 * 2 + 768)
    extra = 2 * 2 * (3 * 64 * 128 * 2 + 2 * 64 * 64 * 2)
    assert q(1, 2, 128, 128, 128, 64, 0) == max(states + records + extra, _exact(128, 128, 128))
    per_chunk = (states + records + extra) // 4
    assert q(1, 2, 64 * 64, 128, 128, 64, 0) == 2 * 64 * per_chunk          # chunk records dominate
    # fp32 activations block the backward with chunks of 32
    assert q(1, 2, 128, 64, 64, 64, 1) == max(2 * 2 * 4 * 64 * 64 * 4, _exact(128, 64, 64))
    assert q(1, 2, 128, 128, 128, 48, 0) == 0
    assert q(1, 2, 128, 128, 96, 64, 0) == 0
    # other head shapes and chunks run the generic path: fp32 chunk-start states
    # and chunk-end gradients (2 x B*H x T/chunk x d_k x d_v x 4 bytes)
    assert q(1, 2, 128, 32, 32, 64, 0) == max(2 * 2 * 2 * 32 * 32 * 4, _exact(128, 32, 32))
    assert q(1, 2, 128, 128, 64, 64, 0) == max(2 * 2 * 2 * 128 * 64 * 4, _exact(128, 128, 64))
    assert q(1, 2, 128, 16, 128, 16, 0) == max(2 * 2 * 8 * 16 * 128 * 4, _exact(128, 16, 128))
    assert q(1, 2, 128, 64, 64, 16, 1) == max(2 * 2 * 8 * 64 * 64 * 4, _exact(128, 64, 64))
    assert q(4, 8, 1 << 14, 32, 32, 16, 0) == 2 * 32 * 1024 * 32 * 32 * 4

    def call(ws=A, nbytes=1 << 30, **kw):
        a = dict(B=1, H=2, T=128, dk=128, dv=128, chunk=64, flags=0)
        a.update(kw)
        return lib.gdr_chunk_bwd(A, A, A, A, A, A, A, A, None, A, A, A, A, A, A, A, a["B"], a["H"],
                                 a["T"], a["dk"], a["dv"], a["chunk"], a["flags"], ws, nbytes, None)
    assert call(ws=None) == 3
    assert call(nbytes=1000) == 3
    assert call(T=100) == 1
    assert call(flags=0x2) == 1          # bf16 output has no meaning for gradients
    assert call(ws=MIS) == 1
    assert call(dk=96, dv=32) == 2
    assert call(chunk=48) == 1


def _fwd_varlen(lib, **kw):
    args = dict(q=A, k=A, v=A, la=A, b=A, w=A, S0=None, o=A, Sf=None, cu=A, nseq=2, H=1, T=100,
                dk=128, dv=128, flags=0, ws=A, nbytes=1 << 30)
    args.update(kw)
    return lib.gdr_chunk_fwd_varlen(args["q"], args["k"], args["v"], args["la"], args["b"],
                                    args["w"], args["S0"], args["o"], args["Sf"], args["cu"],
                                    args["nseq"], args["H"], args["T"], args["dk"], args["dv"],
                                    args["flags"], args["ws"], args["nbytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(cu=None), 1), (dict(nseq=0), 1),
    (dict(H=0), 1), (dict(T=-1), 1), (dict(flags=0x100), 1), (dict(v=MIS), 1),
    (dict(S0=MIS), 1), (dict(ws=MIS), 1), (dict(ws=None), 3), (dict(nbytes=1024), 3),
    (dict(H=1 << 20, T=1 << 20), 1),
    (dict(dk=32, dv=32), 2), (dict(dk=96), 2), (dict(flags=0x1), 2), (dict(flags=0x20), 2),
])
def test_fwd_varlen_argument_validation(kw, status):
    assert _fwd_varlen(_lib(), **kw) == status


def test_fwd_varlen_workspace_query():
    lib = _lib()
    # one record per chunk: a sequence of n tokens has ceil(n/64) <= n//64 + 1 chunks,
    # so H * (T//64 + nseq) records cover any split of T tokens into nseq sequences;
    # then the nseq+1 chunk offsets, the (T//64 + nseq) x 2 chunk table and the
    # nseq-long sequence order (int32), each rounded up to 256 bytes
    # the packed records: W, Kh^T, U', Q_s, P as f16 (d x 64 each, P 64 x 64) and
    # a 1 KiB decay slot, as for the fixed-length forward
    rec = 4 * 64 * 128 * 2 + 64 * 64 * 2 + 1024
    assert lib.gdr_chunk_fwd_varlen_workspace_bytes(3, 2, 200, 128, 128, 0) == 2 * (3 + 3) * rec + 768
    assert lib.gdr_chunk_fwd_varlen_workspace_bytes(64, 1, 0, 128, 128, 0) == 64 * rec + 1280
    rec64 = 4 * 64 * 64 * 2 + 64 * 64 * 2 + 1024
    assert lib.gdr_chunk_fwd_varlen_workspace_bytes(1, 4, 128, 64, 64, 0x1c) == 4 * 3 * rec64 + 768
    assert lib.gdr_chunk_fwd_varlen_workspace_bytes(0, 1, 64, 128, 128, 0) == 0
    assert lib.gdr_chunk_fwd_varlen_workspace_bytes(1, 1, 64, 128, 128, 0x1) == 0   # fp32
    assert lib.gdr_chunk_fwd_varlen_workspace_bytes(1, 1, 64, 32, 32, 0) == 0


def _bwd_varlen(lib, **kw):
    args = dict(q=A, k=A, v=A, la=A, b=A, w=A, S0=None, dO=A, dSf=None, dq=A, dk_=A, dv_=A,
                dla=A, db=A, dw=A, dS0=None, cu=A, nseq=2, H=1, T=100, dk=128, dv=128, flags=0,
                ws=A, nbytes=1 << 30)
    args.update(kw)
    a = args
    return lib.gdr_chunk_bwd_varlen(a["q"], a["k"], a["v"], a["la"], a["b"], a["w"], a["S0"],
                                    a["dO"], a["dSf"], a["dq"], a["dk_"], a["dv_"], a["dla"],
                                    a["db"], a["dw"], a["dS0"], a["cu"], a["nseq"], a["H"],
                                    a["T"], a["dk"], a["dv"], a["flags"], a["ws"], a["nbytes"],
                                    None)


@pytest.mark.parametrize("kw,status", [
    (dict(dO=None), 1), (dict(dq=None), 1), (dict(cu=None), 1), (dict(nseq=0), 1),
    (dict(T=-1), 1), (dict(flags=0x2), 1), (dict(dla=MIS), 1), (dict(dS0=MIS), 1),
    (dict(ws=None), 3), (dict(nbytes=4096), 3), (dict(H=1 << 20, T=1 << 20), 1),
    (dict(dk=128, dv=64), 2), (dict(dk=32, dv=32), 2), (dict(flags=0x1), 2),
])
def test_bwd_varlen_argument_validation(kw, status):
    assert _bwd_varlen(_lib(), **kw) == status


def test_bwd_varlen_workspace_query():
    lib = _lib()
    q = lib.gdr_chunk_bwd_varlen_workspace_bytes
    # per chunk slot (H * (T//64 + nseq) of them): the forward record with the
    # backward's layouts, S' and the state gradient as f16 (2 x d_k x d_v x 2
    # bytes); then the prep arrays as for the packed forward; at least one unit
    # of the token-by-token recompute over T tokens
    slot = lib.gdr_chunk_bwd_workspace_bytes(1, 1, 64 * 64, 128, 128, 64, 0) // 64
    assert q(3, 2, 200, 128, 128, 0) == max(2 * 6 * slot + 768, _exact(200, 128, 128))
    assert 2 * 67 * slot < q(3, 2, 64 * 64, 128, 128, 0) < 2 * 67 * slot + 4096   # chunk slots dominate
    slot64 = lib.gdr_chunk_bwd_workspace_bytes(1, 1, 64 * 64, 64, 64, 64, 0) // 64
    assert q(1, 4, 128, 64, 64, 0x1c) == max(4 * 3 * slot64 + 768, _exact(128, 64, 64))
    assert q(1, 1, 64, 128, 64, 0) == 0
    assert q(1, 1, 64, 128, 128, 0x1) == 0
    assert q(0, 1, 64, 128, 128, 0) == 0


def test_mixer_argument_validation():
    lib = _lib()

    def pro(**kw):
        a = dict(ptrs=[A] * 15, B=1, H=2, T=64, dk=128, dv=128, flags=0)
        a.update(kw)
        return lib.gdr_mixer_prologue(*a["ptrs"], a["B"], a["H"], a["T"], a["dk"], a["dv"],
                                      a["flags"], None)

    def epi(**kw):
        a = dict(ptrs=[A] * 4, B=1, H=2, T=64, dv=128, flags=0)
        a.update(kw)
        return lib.gdr_mixer_epilogue(*a["ptrs"], a["B"], a["H"], a["T"], a["dv"], a["flags"], None)
    assert pro(ptrs=[A] * 14 + [None]) == 1          # w output missing
    assert pro(ptrs=[MIS] + [A] * 14) == 1
    assert pro(B=0) == 1 and pro(T=-1) == 1
    assert pro(flags=0x2) == 1 and pro(flags=0x20) == 1
    assert pro(flags=0x1) == 2                       # fp32 activations: no kernel
    assert pro(dk=32) == 2 and pro(dv=96) == 2
    assert epi(ptrs=[A, A, None, A]) == 1
    assert epi(flags=0x4) == 1 and epi(H=0) == 1
    assert epi(dv=16) == 2


def test_gate_logits_need_the_two_pass_kernels():
    """GDR_GATE_LOGITS is taken by the two-pass forward and backward (with a
    workspace) and by decode; elsewhere the call is refused as unsupported."""
    lib = _lib()
    assert _fwd(lib, flags=0x40) == 2                          # no workspace: fused path
    assert _fwd(lib, flags=0x40 | 0x1) == 2                    # fp32 activations
    assert _fwd(lib, flags=0x40 | 0x20, ws=A, nbytes=1 << 30) == 2   # forced generic kernel
    nb = lib.gdr_chunk_bwd_workspace_bytes(1, 1, 64, 128, 128, 32, 0x40)
    assert nb > 0
    st = lib.gdr_chunk_bwd(A, A, A, A, A, A, None, A, None, A, A, A, A, A, A, None, 1, 1, 64, 128, 128,
                           32, 0x40, A, nb, None)
    assert st == 2                                            # chunks of 32: no two-pass backward


def test_mixer_backward_validation():
    lib = _lib()
    nb = lib.gdr_mixer_bwd_workspace_bytes(2, 3, 200, 128, 128)
    # the larger of: three blocks of per-tile tap partials ((B*H) x ceil(T/64) tiles x
    # d x 4 taps, fp32) and the epilogue's 1024 per-workgroup rows of d partials
    assert nb == max(3 * 6 * 4 * 128 * 4 * 4, 1024 * 128 * 4)
    assert lib.gdr_mixer_bwd_workspace_bytes(4, 16, 4096, 128, 128) == 3 * 64 * 64 * 128 * 4 * 4
    assert lib.gdr_mixer_bwd_workspace_bytes(1, 1, 8, 64, 64) == 1024 * 64 * 4   # epilogue partials
    assert lib.gdr_mixer_bwd_workspace_bytes(1, 1, 64, 128, 64) == 0
    assert lib.gdr_mixer_bwd_workspace_bytes(1, 1, 0, 128, 128) == 0
    args = [A] * 15
    assert lib.gdr_mixer_prologue_bwd(*args, 2, 3, 200, 128, 128, 0, A, nb - 1, None) == 3
    assert lib.gdr_mixer_prologue_bwd(*args, 2, 3, 200, 128, 128, 1, A, nb, None) == 1
    assert lib.gdr_mixer_prologue_bwd(*args, 2, 3, 200, 128, 64, 0, A, nb, None) == 2
    assert lib.gdr_mixer_prologue_bwd(*([A] * 14 + [None]), 2, 3, 200, 128, 128, 0, A, nb, None) == 1
    assert lib.gdr_mixer_epilogue_bwd(*([A] * 7), 1, 1, 8, 64, 0, A, 1024 * 64 * 4 - 1, None) == 3
    assert lib.gdr_mixer_epilogue_bwd(*([A] * 7), 1, 1, 8, 96, 0, A, 1 << 20, None) == 2


def test_size_overflow_is_rejected_before_any_launch():
    """B*H above 2^28 or B*H*T above 2^40 would overflow the kernels' sequence
    and token arithmetic: the forward, the backward and their workspace
    queries refuse such sizes (status / 0 bytes) instead of launching."""
    lib = _lib()
    big = dict(B=1 << 15, H=1 << 14)                   # B*H = 2^29
    assert _fwd(lib, **big) == 1
    assert _fwd(lib, B=1 << 12, H=1 << 12, T=1 << 17) == 1   # B*H*T = 2^41
    assert lib.gdr_chunk_fwd_workspace_bytes(1 << 15, 1 << 14, 64, 128, 128, 64, 0) == 0
    assert lib.gdr_chunk_fwd_workspace_bytes(1 << 12, 1 << 12, 1 << 17, 128, 128, 64, 0) == 0
    assert lib.gdr_chunk_bwd_workspace_bytes(1 << 15, 1 << 14, 64, 128, 128, 64, 0) == 0
    assert lib.gdr_chunk_bwd_workspace_bytes(1 << 12, 1 << 12, 1 << 17, 128, 128, 64, 0) == 0

    def bwd(B, H, T):
        return lib.gdr_chunk_bwd(A, A, A, A, A, A, A, A, None, A, A, A, A, A, A, A, B, H, T, 128, 128,
                                 64, 0, A, 1 << 62, None)
    assert bwd(1 << 15, 1 << 14, 64) == 1
    assert bwd(1 << 12, 1 << 12, 1 << 17) == 1
