"""gated_delta_rule_24_amd — Python binding of libgdr (gated delta rule on MI355X).

Thin ctypes marshalling over the C ABI declared in ``include/gdr.h``: every
step of the computation runs in the HIP kernels of ``libgdr.so``; PyTorch is
used only for device memory and the current stream.  There is no CPU or
PyTorch fallback: if the library is missing or the device is not a gfx950,
calls raise.

The entry points keep the C names:

* :func:`gdr_chunk_fwd`   — chunkwise-parallel forward
* :func:`gdr_decode_step` — one recurrent decode step, state updated in place
* :func:`gdr_chunk_bwd`   — gate-aware backward
* :func:`gdr_chunk_fwd_varlen`, :func:`gdr_chunk_bwd_varlen` — the forward
  and backward over packed variable-length sequences

and :func:`chunk_fwd`, :func:`decode_step`, :func:`chunk_bwd`,
:func:`chunk_fwd_varlen`, :func:`chunk_bwd_varlen` are the same calls with
outputs allocated for the caller.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_ACT_BF16 = 0x0
GDR_ACT_F32 = 0x1
GDR_OUT_BF16 = 0x2
GDR_ALPHA_SCALAR = 0x4
GDR_B_SCALAR = 0x8
GDR_W_SCALAR = 0x10
GDR_FWD_GENERIC = 0x20
GDR_GATE_LOGITS = 0x40
GDR_FWD_SPLIT = 0x80

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "launch", 5: "device"}

_lib = None


class GdrError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _load().gdr_status_string(status).decode() if _lib is not None else _STATUS.get(status)
        super().__init__(f"{fn} failed with status {status} ({msg})")


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libgdr.so not found at {LIB_PATH}; build it with "
                "`python -m gated_delta_rule_24_amd.build` (no fallback path exists)")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, U, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_size_t
        lib.gdr_abi_version.restype = I
        lib.gdr_status_string.argtypes = [I]
        lib.gdr_status_string.restype = ctypes.c_char_p
        lib.gdr_chunk_fwd_workspace_bytes.argtypes = [I] * 6 + [U]
        lib.gdr_chunk_fwd_workspace_bytes.restype = S
        lib.gdr_chunk_fwd.argtypes = [P] * 9 + [I] * 6 + [U, P, S, P]
        lib.gdr_chunk_fwd.restype = I
        lib.gdr_chunk_fwd_noalloc.argtypes = [P] * 9 + [I] * 6 + [U, P]
        lib.gdr_chunk_fwd_noalloc.restype = I
        lib.gdr_chunk_fwd_varlen_workspace_bytes.argtypes = [I] * 5 + [U]
        lib.gdr_chunk_fwd_varlen_workspace_bytes.restype = S
        lib.gdr_chunk_fwd_varlen.argtypes = [P] * 10 + [I] * 5 + [U, P, S, P]
        lib.gdr_chunk_fwd_varlen.restype = I
        lib.gdr_decode_step.argtypes = [P] * 8 + [I] * 4 + [U, P]
        lib.gdr_decode_step.restype = I
        lib.gdr_chunk_bwd_workspace_bytes.argtypes = [I] * 6 + [U]
        lib.gdr_chunk_bwd_workspace_bytes.restype = S
        lib.gdr_chunk_bwd.argtypes = [P] * 16 + [I] * 6 + [U, P, S, P]
        lib.gdr_chunk_bwd.restype = I
        lib.gdr_chunk_bwd_varlen_workspace_bytes.argtypes = [I] * 5 + [U]
        lib.gdr_chunk_bwd_varlen_workspace_bytes.restype = S
        lib.gdr_chunk_bwd_varlen.argtypes = [P] * 17 + [I] * 5 + [U, P, S, P]
        lib.gdr_chunk_bwd_varlen.restype = I
        lib.gdr_mixer_prologue.argtypes = [P] * 15 + [I] * 5 + [U, P]
        lib.gdr_mixer_prologue.restype = I
        lib.gdr_mixer_epilogue.argtypes = [P] * 4 + [I] * 4 + [U, P]
        lib.gdr_mixer_epilogue.restype = I
        lib.gdr_mixer_bwd_workspace_bytes.argtypes = [I] * 5
        lib.gdr_mixer_bwd_workspace_bytes.restype = S
        lib.gdr_mixer_prologue_bwd.argtypes = [P] * 15 + [I] * 5 + [U, P, S, P]
        lib.gdr_mixer_prologue_bwd.restype = I
        lib.gdr_mixer_epilogue_bwd.argtypes = [P] * 7 + [I] * 4 + [U, P, S, P]
        lib.gdr_mixer_epilogue_bwd.restype = I
        _lib = lib
    return _lib


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


EXPORTED_SYMBOLS = ("gdr_abi_version", "gdr_status_string", "gdr_chunk_fwd_workspace_bytes",
                    "gdr_chunk_fwd", "gdr_chunk_fwd_noalloc", "gdr_chunk_fwd_varlen_workspace_bytes", "gdr_chunk_fwd_varlen",
                    "gdr_decode_step", "gdr_chunk_bwd_workspace_bytes", "gdr_chunk_bwd",
                    "gdr_chunk_bwd_varlen_workspace_bytes", "gdr_chunk_bwd_varlen",
                    "gdr_mixer_prologue", "gdr_mixer_epilogue", "gdr_mixer_bwd_workspace_bytes",
                    "gdr_mixer_prologue_bwd", "gdr_mixer_epilogue_bwd")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _act_flag(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDR_ACT_BF16
    if t.dtype == torch.float32:
        return GDR_ACT_F32
    raise ValueError(f"activation dtype must be bfloat16 or float32, got {t.dtype}")


def gate_flags(q, log_alpha, b, w, gate_logits: bool = False) -> int:
    """Flags for the dtype and gate modes implied by tensor ranks (gate_logits:
    log_alpha, b and w hold logits, see GDR_GATE_LOGITS)."""
    f = _act_flag(q) | (GDR_GATE_LOGITS if gate_logits else 0)
    if log_alpha.dim() == q.dim() - 1:
        f |= GDR_ALPHA_SCALAR
    if b.dim() == q.dim() - 1:
        f |= GDR_B_SCALAR
    if w.dim() == q.dim() - 1:
        f |= GDR_W_SCALAR
    return f


def _check(fn, st):
    if st != 0:
        raise GdrError(fn, st)


# ---------------------------------------------------------------------------
# C-named entry points (outputs provided by the caller)
# ---------------------------------------------------------------------------


def gdr_chunk_fwd_workspace_bytes(B, H, T, d_k, d_v, chunk, flags) -> int:
    return int(_load().gdr_chunk_fwd_workspace_bytes(B, H, T, d_k, d_v, chunk, flags))


def gdr_chunk_fwd(q, k, v, log_alpha, b, w, S0, o, S_final, B, H, T, d_k, d_v, chunk,
                  flags, workspace=None, workspace_bytes=0, stream=None):
    st = _load().gdr_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                               _ptr(S0), _ptr(o), _ptr(S_final), B, H, T, d_k, d_v, chunk,
                               flags, _ptr(workspace), workspace_bytes, _stream(stream))
    _check("gdr_chunk_fwd", st)


# bytes of the library-owned device array gdr_chunk_fwd_noalloc uses per GPU
GDR_NOALLOC_SCRATCH_BYTES = 64 << 20


def gdr_chunk_fwd_noalloc(q, k, v, log_alpha, b, w, S0, o, S_final, B, H, T, d_k, d_v, chunk,
                          flags, stream=None):
    st = _load().gdr_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b),
                                       _ptr(w), _ptr(S0), _ptr(o), _ptr(S_final), B, H, T, d_k, d_v,
                                       chunk, flags, _stream(stream))
    _check("gdr_chunk_fwd_noalloc", st)


def gdr_chunk_fwd_varlen_workspace_bytes(nseq, H, T, d_k, d_v, flags) -> int:
    return int(_load().gdr_chunk_fwd_varlen_workspace_bytes(nseq, H, T, d_k, d_v, flags))


def gdr_chunk_fwd_varlen(q, k, v, log_alpha, b, w, S0, o, S_final, cu_seqlens, nseq, H, T, d_k,
                         d_v, flags, workspace, workspace_bytes, stream=None):
    st = _load().gdr_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b),
                                      _ptr(w), _ptr(S0), _ptr(o), _ptr(S_final),
                                      _ptr(cu_seqlens), nseq, H, T, d_k, d_v, flags,
                                      _ptr(workspace), workspace_bytes, _stream(stream))
    _check("gdr_chunk_fwd_varlen", st)


def gdr_decode_step(q, k, v, log_alpha, b, w, S, o, N, H, d_k, d_v, flags, stream=None):
    st = _load().gdr_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                                 _ptr(S), _ptr(o), N, H, d_k, d_v, flags, _stream(stream))
    _check("gdr_decode_step", st)


def gdr_chunk_bwd_workspace_bytes(B, H, T, d_k, d_v, chunk, flags) -> int:
    return int(_load().gdr_chunk_bwd_workspace_bytes(B, H, T, d_k, d_v, chunk, flags))


def gdr_chunk_bwd(q, k, v, log_alpha, b, w, S0, dO, dS_final, dq, dk, dv, dlog_alpha, db, dw,
                  dS0, B, H, T, d_k, d_v, chunk, flags, workspace, workspace_bytes,
                  stream=None):
    st = _load().gdr_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                               _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(dq), _ptr(dk), _ptr(dv),
                               _ptr(dlog_alpha), _ptr(db), _ptr(dw), _ptr(dS0), B, H, T, d_k,
                               d_v, chunk, flags, _ptr(workspace), workspace_bytes,
                               _stream(stream))
    _check("gdr_chunk_bwd", st)


def gdr_chunk_bwd_varlen_workspace_bytes(nseq, H, T, d_k, d_v, flags) -> int:
    return int(_load().gdr_chunk_bwd_varlen_workspace_bytes(nseq, H, T, d_k, d_v, flags))


def gdr_chunk_bwd_varlen(q, k, v, log_alpha, b, w, S0, dO, dS_final, dq, dk, dv, dlog_alpha, db,
                         dw, dS0, cu_seqlens, nseq, H, T, d_k, d_v, flags, workspace,
                         workspace_bytes, stream=None):
    st = _load().gdr_chunk_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b),
                                      _ptr(w), _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(dq),
                                      _ptr(dk), _ptr(dv), _ptr(dlog_alpha), _ptr(db), _ptr(dw),
                                      _ptr(dS0), _ptr(cu_seqlens), nseq, H, T, d_k, d_v, flags,
                                      _ptr(workspace), workspace_bytes, _stream(stream))
    _check("gdr_chunk_bwd_varlen", st)


def gdr_mixer_prologue(q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, a_pre, b_pre, w_pre, q, k, v,
                       log_alpha, b, w, B, H, T, d_k, d_v, flags, stream=None):
    st = _load().gdr_mixer_prologue(_ptr(q_pre), _ptr(k_pre), _ptr(v_pre), _ptr(conv_q),
                                    _ptr(conv_k), _ptr(conv_v), _ptr(a_pre), _ptr(b_pre),
                                    _ptr(w_pre), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                    _ptr(b), _ptr(w), B, H, T, d_k, d_v, flags, _stream(stream))
    _check("gdr_mixer_prologue", st)


def gdr_mixer_epilogue(o, g, norm_weight, y, B, H, T, d_v, flags=0, stream=None):
    st = _load().gdr_mixer_epilogue(_ptr(o), _ptr(g), _ptr(norm_weight), _ptr(y), B, H, T, d_v,
                                    flags, _stream(stream))
    _check("gdr_mixer_epilogue", st)


def gdr_mixer_bwd_workspace_bytes(B, H, T, d_k, d_v) -> int:
    return int(_load().gdr_mixer_bwd_workspace_bytes(B, H, T, d_k, d_v))


def gdr_mixer_prologue_bwd(q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, dq, dk, dv, dq_pre, dk_pre,
                           dv_pre, dconv_q, dconv_k, dconv_v, B, H, T, d_k, d_v, flags, workspace,
                           workspace_bytes, stream=None):
    st = _load().gdr_mixer_prologue_bwd(*[_ptr(x) for x in (q_pre, k_pre, v_pre, conv_q, conv_k,
                                                            conv_v, dq, dk, dv, dq_pre, dk_pre,
                                                            dv_pre, dconv_q, dconv_k, dconv_v)],
                                        B, H, T, d_k, d_v, flags, _ptr(workspace), workspace_bytes,
                                        _stream(stream))
    _check("gdr_mixer_prologue_bwd", st)


def gdr_mixer_epilogue_bwd(o, g, norm_weight, dy, d_o, dg, dnorm_weight, B, H, T, d_v, flags,
                           workspace, workspace_bytes, stream=None):
    st = _load().gdr_mixer_epilogue_bwd(_ptr(o), _ptr(g), _ptr(norm_weight), _ptr(dy), _ptr(d_o),
                                        _ptr(dg), _ptr(dnorm_weight), B, H, T, d_v, flags,
                                        _ptr(workspace), workspace_bytes, _stream(stream))
    _check("gdr_mixer_epilogue_bwd", st)


# ---------------------------------------------------------------------------
# convenience wrappers (allocate outputs with torch)
# ---------------------------------------------------------------------------


def chunk_fwd(q, k, v, log_alpha, b, w, S0=None, chunk: int = 64,
              out_dtype=torch.float32, return_state: bool = True, stream=None,
              generic: bool = False, path: str = "auto", gate_logits: bool = False):
    """q, k: [B,H,T,dk]; v: [B,H,T,dv]; log_alpha, b: [B,H,T,dk] or [B,H,T];
    w: [B,H,T,dv] or [B,H,T]; S0: [B,H,dk,dv] fp32 or None.
    path "auto" passes a workspace (the chunk producer and the state chains in
    one persistent kernel where they apply), "split" the same with the two
    roles as two kernels one after the other (GDR_FWD_SPLIT), "fused" passes
    no workspace (single-kernel path).
    Returns (o [B,H,T,dv], S_final [B,H,dk,dv] or None)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    flags = gate_flags(q, log_alpha, b, w, gate_logits)
    if out_dtype == torch.bfloat16:
        flags |= GDR_OUT_BF16
    if generic:
        flags |= GDR_FWD_GENERIC
    o = torch.empty((B, H, T, dv), dtype=out_dtype, device=q.device)
    Sf = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if return_state else None
    ws, nbytes = None, 0
    if path == "split":
        flags |= GDR_FWD_SPLIT
    if path in ("auto", "split"):
        nbytes = gdr_chunk_fwd_workspace_bytes(B, H, T, dk, dv, chunk, flags)
        if nbytes > 0:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    elif path != "fused":
        raise ValueError(f"unknown path {path!r}")
    gdr_chunk_fwd(q, k, v, log_alpha, b, w, S0, o, Sf, B, H, T, dk, dv, chunk, flags, ws, nbytes,
                  stream)
    return o, Sf


def chunk_fwd_varlen(q, k, v, log_alpha, b, w, cu_seqlens, S0=None, out_dtype=torch.float32,
                     return_state: bool = True, stream=None, gate_logits: bool = False):
    """Packed sequences: q, k: [H,T,dk]; v: [H,T,dv]; log_alpha, b: [H,T,dk] or
    [H,T]; w: [H,T,dv] or [H,T]; cu_seqlens: int32 [nseq+1] on the GPU; S0:
    [nseq,H,dk,dv] fp32 or None.  Returns (o [H,T,dv], S_final [nseq,H,dk,dv] or None)."""
    H, T, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    nseq = cu_seqlens.numel() - 1
    flags = gate_flags(q, log_alpha, b, w, gate_logits)
    if out_dtype == torch.bfloat16:
        flags |= GDR_OUT_BF16
    o = torch.empty((H, T, dv), dtype=out_dtype, device=q.device)
    Sf = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=q.device) if return_state else None
    nbytes = gdr_chunk_fwd_varlen_workspace_bytes(nseq, H, T, dk, dv, flags)
    if nbytes == 0:
        raise GdrError("gdr_chunk_fwd_varlen_workspace_bytes", 2)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    gdr_chunk_fwd_varlen(q, k, v, log_alpha, b, w, S0, o, Sf, cu_seqlens, nseq, H, T, dk, dv,
                         flags, ws, nbytes, stream)
    return o, Sf


def decode_step(q, k, v, log_alpha, b, w, S, out_dtype=torch.float32, o=None, stream=None,
                gate_logits: bool = False):
    """One token per (n, h): q, k: [N,H,dk]; v: [N,H,dv]; gates channel or
    scalar ([N,H]); S: [N,H,dk,dv] fp32, updated in place.  Returns o."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    flags = gate_flags(q, log_alpha, b, w, gate_logits)
    if out_dtype == torch.bfloat16:
        flags |= GDR_OUT_BF16
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=q.device)
    gdr_decode_step(q, k, v, log_alpha, b, w, S, o, N, H, dk, dv, flags, stream)
    return o


def chunk_bwd(q, k, v, log_alpha, b, w, S0, dO, dS_final=None, chunk: int = 64, stream=None,
              gate_logits: bool = False):
    """Gradients of L = <dO, o> + <dS_final, S_final>.  Returns a dict of fp32
    tensors dq, dk, dv, dlog_alpha, db, dw (scalar gates keep their scalar
    shape) and dS0."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    flags = gate_flags(q, log_alpha, b, w, gate_logits)
    dev = q.device
    f32 = torch.float32
    out = dict(dq=torch.empty((B, H, T, dk), dtype=f32, device=dev),
               dk=torch.empty((B, H, T, dk), dtype=f32, device=dev),
               dv=torch.empty((B, H, T, dv), dtype=f32, device=dev),
               dlog_alpha=torch.empty(tuple(log_alpha.shape), dtype=f32, device=dev),
               db=torch.empty(tuple(b.shape), dtype=f32, device=dev),
               dw=torch.empty(tuple(w.shape), dtype=f32, device=dev),
               dS0=torch.empty((B, H, dk, dv), dtype=f32, device=dev))
    nbytes = gdr_chunk_bwd_workspace_bytes(B, H, T, dk, dv, chunk, flags)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    gdr_chunk_bwd(q, k, v, log_alpha, b, w, S0, dO, dS_final, out["dq"], out["dk"], out["dv"],
                  out["dlog_alpha"], out["db"], out["dw"], out["dS0"], B, H, T, dk, dv, chunk,
                  flags, ws, nbytes, stream)
    return out


def chunk_bwd_varlen(q, k, v, log_alpha, b, w, cu_seqlens, S0, dO, dS_final=None, stream=None,
                     gate_logits: bool = False):
    """Packed sequences ([H,T,...] streams, cu_seqlens int32 on the GPU): the
    gradients of L = <dO, o> + <dS_final, S_final> as a dict of fp32 tensors
    dq, dk, dv, dlog_alpha, db, dw (in the inputs' shapes) and dS0 [nseq,H,dk,dv]."""
    H, T, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    nseq = cu_seqlens.numel() - 1
    flags = gate_flags(q, log_alpha, b, w, gate_logits)
    dev = q.device
    f32 = torch.float32
    out = dict(dq=torch.empty((H, T, dk), dtype=f32, device=dev),
               dk=torch.empty((H, T, dk), dtype=f32, device=dev),
               dv=torch.empty((H, T, dv), dtype=f32, device=dev),
               dlog_alpha=torch.empty(tuple(log_alpha.shape), dtype=f32, device=dev),
               db=torch.empty(tuple(b.shape), dtype=f32, device=dev),
               dw=torch.empty(tuple(w.shape), dtype=f32, device=dev),
               dS0=torch.empty((nseq, H, dk, dv), dtype=f32, device=dev))
    nbytes = gdr_chunk_bwd_varlen_workspace_bytes(nseq, H, T, dk, dv, flags)
    if nbytes == 0:
        raise GdrError("gdr_chunk_bwd_varlen_workspace_bytes", 2)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    gdr_chunk_bwd_varlen(q, k, v, log_alpha, b, w, S0, dO, dS_final, out["dq"], out["dk"],
                         out["dv"], out["dlog_alpha"], out["db"], out["dw"], out["dS0"],
                         cu_seqlens, nseq, H, T, dk, dv, flags, ws, nbytes, stream)
    return out


def mixer_prologue(q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, a_pre, b_pre, w_pre, stream=None,
                   gate_logits: bool = False):
    """[B,H,T,d] bf16 projection outputs (a_pre fp32; gate logits [B,H,T,d]
    or [B,H,T]) and fp32 [H,d,4] convolution taps -> dict q, k, v, log_alpha,
    b, w: the inputs of chunk_fwd.  gate_logits: only q, k, v are produced;
    log_alpha, b and w are the logits themselves, for the recurrence calls
    made with gate_logits=True."""
    B, H, T, dk = q_pre.shape
    dv = v_pre.shape[-1]
    flags = GDR_GATE_LOGITS if gate_logits else 0
    if a_pre.dim() == 3:
        flags |= GDR_ALPHA_SCALAR
    if b_pre.dim() == 3:
        flags |= GDR_B_SCALAR
    if w_pre.dim() == 3:
        flags |= GDR_W_SCALAR
    out = dict(q=torch.empty_like(q_pre), k=torch.empty_like(k_pre), v=torch.empty_like(v_pre))
    if gate_logits:
        gdr_mixer_prologue(q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, None, None, None, out["q"],
                           out["k"], out["v"], None, None, None, B, H, T, dk, dv, flags, stream)
        out.update(log_alpha=a_pre, b=b_pre, w=w_pre)
        return out
    out.update(log_alpha=torch.empty_like(a_pre), b=torch.empty_like(b_pre), w=torch.empty_like(w_pre))
    gdr_mixer_prologue(q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, a_pre, b_pre, w_pre, out["q"],
                       out["k"], out["v"], out["log_alpha"], out["b"], out["w"], B, H, T, dk, dv,
                       flags, stream)
    return out


def mixer_epilogue(o, g, norm_weight, stream=None):
    """o fp32 [B,H,T,dv], g bf16 [B,H,T,dv], norm_weight fp32 [dv] -> y bf16."""
    B, H, T, dv = o.shape
    y = torch.empty(o.shape, dtype=torch.bfloat16, device=o.device)
    gdr_mixer_epilogue(o, g, norm_weight, y, B, H, T, dv, 0, stream)
    return y


def mixer_prologue_bwd(q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, dq, dk, dv, stream=None):
    """Gradients of the prologue's q, k, v paths: dict dq_pre, dk_pre, dv_pre
    (fp32 [B,H,T,d]) and dconv_q, dconv_k, dconv_v (fp32 [H,d,4])."""
    B, H, T, dk_ = q_pre.shape
    dv_ = v_pre.shape[-1]
    f32 = torch.float32
    out = dict(dq_pre=torch.empty(q_pre.shape, dtype=f32, device=q_pre.device),
               dk_pre=torch.empty(k_pre.shape, dtype=f32, device=q_pre.device),
               dv_pre=torch.empty(v_pre.shape, dtype=f32, device=q_pre.device),
               dconv_q=torch.empty_like(conv_q), dconv_k=torch.empty_like(conv_k),
               dconv_v=torch.empty_like(conv_v))
    nb = gdr_mixer_bwd_workspace_bytes(B, H, T, dk_, dv_)
    if nb == 0:
        raise GdrError("gdr_mixer_bwd_workspace_bytes", 2)
    ws = torch.empty(nb, dtype=torch.uint8, device=q_pre.device)
    gdr_mixer_prologue_bwd(q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, dq, dk, dv, out["dq_pre"],
                           out["dk_pre"], out["dv_pre"], out["dconv_q"], out["dconv_k"],
                           out["dconv_v"], B, H, T, dk_, dv_, 0, ws, nb, stream)
    return out


def mixer_epilogue_bwd(o, g, norm_weight, dy, stream=None):
    """Gradients of the epilogue: dict d_o, dg (fp32 [B,H,T,dv]), dnorm_weight (fp32 [dv])."""
    B, H, T, dv_ = o.shape
    f32 = torch.float32
    out = dict(d_o=torch.empty(o.shape, dtype=f32, device=o.device),
               dg=torch.empty(o.shape, dtype=f32, device=o.device),
               dnorm_weight=torch.empty((dv_,), dtype=f32, device=o.device))
    nb = gdr_mixer_bwd_workspace_bytes(B, H, T, dv_, dv_)
    if nb == 0:
        raise GdrError("gdr_mixer_bwd_workspace_bytes", 2)
    ws = torch.empty(nb, dtype=torch.uint8, device=o.device)
    gdr_mixer_epilogue_bwd(o, g, norm_weight, dy, out["d_o"], out["dg"], out["dnorm_weight"], B, H, T,
                           dv_, 0, ws, nb, stream)
    return out
