"""Oracle for the token-mixer prologue and epilogue: plain fp64 numpy.

TEST INFRASTRUCTURE ONLY.  Only the test suite and bench.py's CPU-baseline
leg may import this module.  The HIP library never calls it, and the two
share no code.

The block, from the pages ("Gated DeltaNet study notes" §2 token mixer block
design; "Gated DeltaNet-2 Review" §4-3 engineering notes):
- q and k: linear projection, short causal convolution, SiLU, L2 norm;
- v: linear projection, short causal convolution, SiLU;
- log-decay from its own projection, kept in fp32;
- erase and write gates: own projections, each through a sigmoid;
- output: RMS norm of the recurrent output, times a SiLU output gate, then
  the output projection.
The projections are plain matrix products outside this module; the functions
below take their outputs.  Where the pages leave a detail open, the reading
taken is:
- the short convolution is depthwise and causal, 4 taps per channel, tap j
  weighting the token j steps back, zero before the first token;
- L2norm(x) = x / sqrt(sum x^2 + 1e-6) over a head's channels;
- RMS norm: x / sqrt(mean x^2 + 1e-6) times a per-channel weight shared by
  the heads;
- the decay gate is a sigmoid like the others (the Q&A page writes alpha as
  a sigmoid of a projection), so log alpha = log(sigmoid(a_pre)).
Every function works in float64 on whatever array it is given.
"""
from __future__ import annotations

import numpy as np

TAPS = 4
EPS = 1e-6


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def causal_conv(x, taps):
    """y[..., h, t, c] = sum_j taps[h, c, j] * x[..., h, t - j, c], over j with t - j >= 0.

    x: [..., H, T, D]; taps: [H, D, TAPS]."""
    x = _f64(x)
    taps = _f64(taps)
    T = x.shape[-2]
    y = np.zeros_like(x)
    for j in range(taps.shape[-1]):
        if j >= T:
            break
        # token t takes x[t - j]: shift the sequence down by j, zeros in front
        shifted = np.zeros_like(x)
        shifted[..., j:, :] = x[..., :T - j, :]
        y += shifted * taps[:, None, :, j]
    return y


def silu(x):
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def sigmoid(x):
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def log_sigmoid(x):
    """log(1 / (1 + exp(-x))) = -log(1 + exp(-x)), written with logaddexp so
    that neither sign overflows."""
    return -np.logaddexp(0.0, -_f64(x))


def l2norm(x):
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)


def rms_norm(x, weight):
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS) * _f64(weight)


def prologue(q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, a_pre, b_pre, w_pre):
    """The recurrence's inputs from the projection outputs ([B, H, T, d]
    streams; gate logits [B, H, T, d] or [B, H, T])."""
    return dict(q=l2norm(silu(causal_conv(q_pre, conv_q))),
                k=l2norm(silu(causal_conv(k_pre, conv_k))),
                v=silu(causal_conv(v_pre, conv_v)),
                log_alpha=log_sigmoid(a_pre),
                b=sigmoid(b_pre),
                w=sigmoid(w_pre))


def epilogue(o, g, norm_weight):
    """RMS-normalised output times the SiLU output gate ([B, H, T, d_v])."""
    return rms_norm(o, norm_weight) * silu(g)
