"""Oracle for the token-mixer prologue and epilogue: plain fp64 on the CPU.

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
- the decay gate is a sigmoid like the others (the "Gated DeltaNet"
  explainer, data-dependent gating section, writes alpha as a sigmoid of a
  projection of the input), so log alpha = log(sigmoid(a_pre)).

The definitions are written once, as plain float64 torch operations on the
CPU (numpy arrays in and out).  The backward functions differentiate exactly
these definitions with torch.autograd (reverse mode as a library step); the
tests pin them with central finite differences of the forward.
"""
from __future__ import annotations

import numpy as np
import torch

TAPS = 4
EPS = 1e-6


def _t(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


# ------------------------------------------------------------ definitions (torch fp64)

def _causal_conv(x, taps):
    """y[..., h, t, c] = sum_j taps[h, c, j] * x[..., h, t - j, c], over j with t - j >= 0."""
    T = x.shape[-2]
    y = torch.zeros_like(x)
    for j in range(min(taps.shape[-1], T)):
        # token t takes x[t - j]: shift the sequence down by j, zeros in front
        shifted = torch.zeros_like(x)
        shifted[..., j:, :] = x[..., :T - j, :]
        y = y + shifted * taps[:, None, :, j]
    return y


def _silu(x):
    return x / (1.0 + torch.exp(-x))


def _sigmoid(x):
    return 1.0 / (1.0 + torch.exp(-x))


def _log_sigmoid(x):
    # -log(1 + exp(-x)), in a form that overflows for neither sign
    return -torch.logaddexp(torch.zeros_like(x), -x)


def _l2norm(x):
    return x / torch.sqrt(torch.sum(x * x, dim=-1, keepdim=True) + EPS)


def _rms_norm(x, weight):
    return x / torch.sqrt(torch.mean(x * x, dim=-1, keepdim=True) + EPS) * weight


def _stream(x, taps, l2):
    y = _silu(_causal_conv(x, taps))
    return _l2norm(y) if l2 else y


def _epilogue(o, g, weight):
    return _rms_norm(o, weight) * _silu(g)


# ------------------------------------------------------------ numpy-facing forward

def causal_conv(x, taps):
    """x: [..., H, T, D]; taps: [H, D, TAPS]."""
    return _causal_conv(_t(x), _t(taps)).numpy()


def silu(x):
    return _silu(_t(x)).numpy()


def sigmoid(x):
    return _sigmoid(_t(x)).numpy()


def log_sigmoid(x):
    return _log_sigmoid(_t(x)).numpy()


def l2norm(x):
    return _l2norm(_t(x)).numpy()


def rms_norm(x, weight):
    return _rms_norm(_t(x), _t(weight)).numpy()


def prologue(q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, a_pre, b_pre, w_pre):
    """The recurrence's inputs from the projection outputs ([B, H, T, d]
    streams; gate logits [B, H, T, d] or [B, H, T])."""
    return dict(q=_stream(_t(q_pre), _t(conv_q), True).numpy(),
                k=_stream(_t(k_pre), _t(conv_k), True).numpy(),
                v=_stream(_t(v_pre), _t(conv_v), False).numpy(),
                log_alpha=log_sigmoid(a_pre),
                b=sigmoid(b_pre),
                w=sigmoid(w_pre))


def epilogue(o, g, norm_weight):
    """RMS-normalised output times the SiLU output gate ([B, H, T, d_v])."""
    return _epilogue(_t(o), _t(g), _t(norm_weight)).numpy()


# ------------------------------------------------------------ reverse mode

def _grad(f, inputs, cotangent):
    xs = [_t(x).requires_grad_(True) for x in inputs]
    y = f(*xs)
    (y * _t(cotangent)).sum().backward()
    return [x.grad.numpy() for x in xs]


def stream_bwd(x_pre, taps, dy, l2):
    """Gradients of <dy, stream(x_pre, taps)> (the q / k path with l2=True,
    the v path with l2=False) w.r.t. x_pre and the taps."""
    return tuple(_grad(lambda x, w: _stream(x, w, l2), (x_pre, taps), dy))


def epilogue_bwd(o, g, norm_weight, dy):
    """Gradients of <dy, epilogue(o, g, w)> w.r.t. o, g and w."""
    return tuple(_grad(_epilogue, (o, g, norm_weight), dy))
