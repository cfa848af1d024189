"""Oracle for the gated delta rule: fp64 token-by-token recurrence on the CPU.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The HIP
library never links, imports or calls it, and the two share no code.

The arithmetic lives in ``gdr_oracle.c`` (plain C, fp64, OpenMP over
independent (batch, head) sequences).  This module only compiles it with gcc,
loads it with ctypes and marshals numpy arrays: it broadcasts scalar gates to
full channel arrays and upcasts inputs to float64, nothing else.

Update rule (Gated DeltaNet-2 Q&A page, Q3; "Gated DeltaNet-2 Review" §3-1):
    S_t = (I - k_t (b_t ⊙ k_t)^T) D_t S_{t-1} + k_t (w_t ⊙ v_t)^T,
    D_t = diag(exp(log_alpha_t)),   o_t = S_t^T q_t.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile gdr_oracle.c into liboracle.so with gcc (-O2, OpenMP, IEEE fp64)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int
            lib.oracle_fwd.argtypes = [I, I, I, I] + [P] * 9 + [I]
            lib.oracle_fwd.restype = None
            lib.oracle_decode.argtypes = [I, I, I] + [P] * 8 + [I]
            lib.oracle_decode.restype = None
            lib.oracle_bwd.argtypes = [I, I, I, I] + [P] * 16 + [I]
            lib.oracle_bwd.restype = None
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = I
            _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _f64(x, shape):
    """Upcast to contiguous float64 and broadcast a scalar gate to ``shape``."""
    a = np.asarray(x, dtype=np.float64)
    if a.shape != tuple(shape):
        a = np.broadcast_to(a.reshape(a.shape + (1,) * (len(shape) - a.ndim)), shape)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(q, k, v, log_alpha, b, w, S0=None, nthreads: int = 0):
    """Token recurrence over sequences.

    q, k: [..., T, dk]; v: [..., T, dv]; log_alpha, b: [..., T, dk] or [..., T]
    (scalar gate, broadcast over channels); w: [..., T, dv] or [..., T];
    S0: [..., dk, dv] or None.  Leading dims are flattened into independent
    sequences.  Returns (o [..., T, dv], S_final [..., dk, dv]) in float64.
    """
    q = np.asarray(q)
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = np.asarray(v).shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    sk = (BH, T, dk)
    sv = (BH, T, dv)
    qq = _f64(q, lead + (T, dk)).reshape(sk)
    kk = _f64(k, lead + (T, dk)).reshape(sk)
    vv = _f64(v, lead + (T, dv)).reshape(sv)
    la = _f64(log_alpha, lead + (T, dk)).reshape(sk)
    bb = _f64(b, lead + (T, dk)).reshape(sk)
    ww = _f64(w, lead + (T, dv)).reshape(sv)
    s0 = None if S0 is None else _f64(S0, lead + (dk, dv)).reshape(BH, dk, dv)
    o = np.empty(sv, dtype=np.float64)
    sf = np.empty((BH, dk, dv), dtype=np.float64)
    _load().oracle_fwd(BH, T, dk, dv, _ptr(qq), _ptr(kk), _ptr(vv), _ptr(la), _ptr(bb),
                       _ptr(ww), _ptr(s0), _ptr(o), _ptr(sf), int(nthreads))
    return o.reshape(lead + (T, dv)), sf.reshape(lead + (dk, dv))


def decode(q, k, v, log_alpha, b, w, S, nthreads: int = 0):
    """One recurrent step for independent states.

    q, k: [..., dk]; v: [..., dv]; log_alpha, b: [..., dk] or [...];
    w: [..., dv] or [...]; S: [..., dk, dv].  Returns (o [..., dv], S_new)
    in float64; the caller's S is not modified.
    """
    q = np.asarray(q)
    lead = q.shape[:-1]
    dk = q.shape[-1]
    dv = np.asarray(v).shape[-1]
    NH = int(np.prod(lead)) if lead else 1
    qq = _f64(q, lead + (dk,)).reshape(NH, dk)
    kk = _f64(k, lead + (dk,)).reshape(NH, dk)
    vv = _f64(v, lead + (dv,)).reshape(NH, dv)
    la = _f64(log_alpha, lead + (dk,)).reshape(NH, dk)
    bb = _f64(b, lead + (dk,)).reshape(NH, dk)
    ww = _f64(w, lead + (dv,)).reshape(NH, dv)
    s = np.array(_f64(S, lead + (dk, dv)).reshape(NH, dk, dv), copy=True)
    o = np.empty((NH, dv), dtype=np.float64)
    _load().oracle_decode(NH, dk, dv, _ptr(qq), _ptr(kk), _ptr(vv), _ptr(la), _ptr(bb),
                          _ptr(ww), _ptr(s), _ptr(o), int(nthreads))
    return o.reshape(lead + (dv,)), s.reshape(lead + (dk, dv))


def bwd(q, k, v, log_alpha, b, w, S0, dO, dS_final=None, nthreads: int = 0):
    """Reverse mode of :func:`fwd` for L = <dO, o> + <dS_final, S_T>.

    Returns a dict with dq, dk, dv, dlog_alpha, db, dw (full channel arrays,
    float64) and dS0.  For a scalar gate the caller sums the channel gradient
    over its broadcast axis.
    """
    q = np.asarray(q)
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = np.asarray(v).shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    sk = (BH, T, dk)
    sv = (BH, T, dv)
    qq = _f64(q, lead + (T, dk)).reshape(sk)
    kk = _f64(k, lead + (T, dk)).reshape(sk)
    vv = _f64(v, lead + (T, dv)).reshape(sv)
    la = _f64(log_alpha, lead + (T, dk)).reshape(sk)
    bb = _f64(b, lead + (T, dk)).reshape(sk)
    ww = _f64(w, lead + (T, dv)).reshape(sv)
    s0 = None if S0 is None else _f64(S0, lead + (dk, dv)).reshape(BH, dk, dv)
    do = _f64(dO, lead + (T, dv)).reshape(sv)
    dsf = None if dS_final is None else _f64(dS_final, lead + (dk, dv)).reshape(BH, dk, dv)
    out = {n: np.empty(sk, dtype=np.float64) for n in ("dq", "dk", "dlog_alpha", "db")}
    out.update({n: np.empty(sv, dtype=np.float64) for n in ("dv", "dw")})
    out["dS0"] = np.empty((BH, dk, dv), dtype=np.float64)
    _load().oracle_bwd(BH, T, dk, dv, _ptr(qq), _ptr(kk), _ptr(vv), _ptr(la), _ptr(bb),
                       _ptr(ww), _ptr(s0), _ptr(do), _ptr(dsf), _ptr(out["dq"]),
                       _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]),
                       _ptr(out["db"]), _ptr(out["dw"]), _ptr(out["dS0"]), int(nthreads))
    for n in ("dq", "dk", "dlog_alpha", "db"):
        out[n] = out[n].reshape(lead + (T, dk))
    for n in ("dv", "dw"):
        out[n] = out[n].reshape(lead + (T, dv))
    out["dS0"] = out["dS0"].reshape(lead + (dk, dv))
    return out
