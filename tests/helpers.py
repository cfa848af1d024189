"""Shared helpers for the GPU parity tests: device upload of generated
inputs, oracle calls on all or a sample of heads, and the error metric.

Metric: max over all elements of |x - x_ref| divided by the rms of x_ref over
the whole tensor, applied per output tensor."""
import numpy as np

import oracle


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(x - ref)) / max(rms, 1e-300))


def to_dev(inp, names=("q", "k", "v", "log_alpha", "b", "w", "S0", "dO")):
    import torch
    act = torch.bfloat16 if inp.act == "bf16" else torch.float32
    out = {}
    for n in names:
        a = inp.arrays.get(n)
        if a is None:
            out[n] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(a))
        dt = torch.float32 if n in ("log_alpha", "S0") else act
        out[n] = t.to(dt).cuda()
    if inp.arrays["b"] is inp.arrays["w"]:
        out["w"] = out["b"]
    return out


def oracle_fwd(inp, heads=None, S0=None, nthreads=0):
    """Oracle on flattened (b*H + h) heads (all when heads is None)."""
    a = inp.arrays
    B, H = inp.B, inp.H

    def sel(x):
        if x is None:
            return None
        x = x.reshape((B * H,) + x.shape[2:])
        return x if heads is None else x[np.asarray(heads)]
    s0 = sel(a["S0"]) if S0 is None else S0
    return oracle.fwd(sel(a["q"]), sel(a["k"]), sel(a["v"]), sel(a["log_alpha"]), sel(a["b"]),
                      sel(a["w"]), s0, nthreads=nthreads)


def flat_heads(x, B, H, heads=None):
    x = x.reshape((B * H,) + tuple(x.shape[2:]))
    return x if heads is None else x[np.asarray(heads)]
