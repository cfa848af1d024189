"""Seeded synthetic inputs for the gated delta rule workloads.

This module holds none of the method's arithmetic: it only draws random
numbers, applies the input transforms that define each workload (L2
normalisation of q and k per token and head, sigmoid gates, the negative
softplus log-decay, bf16 rounding of activations), and packs bf16 bit patterns.
Both the HIP path (through its tests and the benchmark) and the oracle consume
exactly the arrays produced here.

Shapes follow the pages' workloads: heads H=16 with d_k=d_v=128 ("Gated
DeltaNet-2 Review" §4 training setup) and sequence lengths in the 2K-16K sweep
of the H100 throughput figure (Gated DeltaNet-2 Q&A page, Q7).  The pages
measure model quality on public suites; those do not affect the kernels,
whose cost depends only on shapes, so seeded Gaussian inputs stand in.

Draw order (one numpy PCG64 stream per ``seed``): q, k, v, gate-decay, b, w,
S0, dO.  Activations are drawn in fp32, transformed in fp32, then rounded to
bf16 with round-to-nearest-even when the activation dtype is bf16, so the
oracle receives exactly the values the GPU receives.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# ---------------------------------------------------------------------------
# bf16 helpers (bit manipulation only)
# ---------------------------------------------------------------------------


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.view(np.uint32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    # finite values cannot carry past bit 31 here
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array is not bf16-representable; call bf16_round first")
    return (u >> 16).astype(np.uint16)


def bf16_from_bits(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint32) << 16).view(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _l2n(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


# ---------------------------------------------------------------------------
# generic generator
# ---------------------------------------------------------------------------


@dataclass
class Inputs:
    """A bundle of inputs; float arrays are float32 holding dtype-exact values."""
    B: int
    H: int
    T: int
    dk: int
    dv: int
    act: str                      # "bf16" or "f32": dtype of q, k, v, b, w, dO
    alpha_mode: str               # "channel" ([B,H,T,dk]) or "scalar" ([B,H,T])
    b_mode: str                   # "channel" or "scalar"
    w_mode: str                   # "channel" or "scalar"
    chunk: int
    arrays: Dict[str, Optional[np.ndarray]] = field(default_factory=dict)
    recipe: str = ""

    def __getitem__(self, k):
        return self.arrays[k]


def make_inputs(B: int, H: int, T: int, dk: int, dv: int, *, act: str = "bf16",
                alpha_mode: str = "channel", b_mode: str = "channel",
                w_mode: str = "channel", tied: bool = False,
                alpha_dist: str = "softplus", decay_scale: float = 0.05,
                normalize_q: bool = True, s0_std: Optional[float] = 0.02,
                with_dO: bool = False, chunk: int = 64, seed: int = 0,
                gate_hi: float = 1.0) -> Inputs:
    """Draw one workload.

    alpha_dist "softplus": log_alpha = -softplus(N(0,1)) * decay_scale (fp32);
    alpha_dist "uniform":  alpha ~ U(0.90, 1.00), log_alpha = log(alpha).
    Gates: sigmoid(N(0,1)) * gate_hi (gate_hi=2 gives the expanded erase range).
    tied=True uses one scalar beta per token for both b and w (GDN / KDA form);
    then b_mode and w_mode must be "scalar" and b is w.
    """
    rng = np.random.default_rng(seed)
    rnd = (lambda a: bf16_round(a)) if act == "bf16" else (lambda a: a.astype(np.float32))
    q = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    if normalize_q:
        q = _l2n(q)
    k = _l2n(rng.standard_normal((B, H, T, dk), dtype=np.float32))
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    ash = (B, H, T, dk) if alpha_mode == "channel" else (B, H, T)
    if alpha_dist == "softplus":
        la = (-_softplus(rng.standard_normal(ash, dtype=np.float32)) * np.float32(decay_scale))
    elif alpha_dist == "uniform":
        la = np.log(rng.uniform(0.90, 1.00, size=ash).astype(np.float32))
    else:
        raise ValueError(alpha_dist)
    la = la.astype(np.float32)
    if tied:
        if b_mode != "scalar" or w_mode != "scalar":
            raise ValueError("tied gates are scalar per token")
        beta = rnd(_sigmoid(rng.standard_normal((B, H, T), dtype=np.float32)) * np.float32(gate_hi))
        b = w = beta
    else:
        bsh = (B, H, T, dk) if b_mode == "channel" else (B, H, T)
        wsh = (B, H, T, dv) if w_mode == "channel" else (B, H, T)
        b = rnd(_sigmoid(rng.standard_normal(bsh, dtype=np.float32)) * np.float32(gate_hi))
        w = rnd(_sigmoid(rng.standard_normal(wsh, dtype=np.float32)) * np.float32(gate_hi))
    S0 = None
    if s0_std is not None:
        S0 = (rng.standard_normal((B, H, dk, dv), dtype=np.float32) * np.float32(s0_std))
    dO = None
    if with_dO:
        dO = rnd(rng.standard_normal((B, H, T, dv), dtype=np.float32))
    arrays = dict(q=rnd(q), k=rnd(k), v=rnd(v), log_alpha=la, b=b, w=w, S0=S0, dO=dO)
    return Inputs(B, H, T, dk, dv, act, alpha_mode, b_mode, w_mode, chunk, arrays)


# ---------------------------------------------------------------------------
# named workloads
# ---------------------------------------------------------------------------

PRESETS = {
    # tiny Gated DeltaNet check, all fp32, scalar gates
    "gdn_tiny": dict(B=1, H=1, T=64, dk=16, dv=16, act="f32", alpha_mode="scalar",
                     b_mode="scalar", w_mode="scalar", tied=True, alpha_dist="uniform",
                     normalize_q=False, s0_std=None, chunk=16),
    # Gated DeltaNet, scalar decay and tied scalar gate, bf16 activations
    "gdn": dict(B=4, H=16, T=2048, dk=128, dv=128, act="bf16", alpha_mode="scalar",
                b_mode="scalar", w_mode="scalar", tied=True, s0_std=None, chunk=64),
    # Gated DeltaNet-2: channel decay, decoupled channel erase/write gates
    "gdn2": dict(B=2, H=16, T=8192, dk=128, dv=128, act="bf16", alpha_mode="channel",
                 b_mode="channel", w_mode="channel", s0_std=0.02, chunk=64),
    # Gated DeltaNet-2 backward workload
    "gdn2_bwd": dict(B=1, H=32, T=16384, dk=128, dv=128, act="bf16", alpha_mode="channel",
                     b_mode="channel", w_mode="channel", s0_std=0.02, with_dO=True, chunk=64),
}


def preset(name: str, seed: int = 0, **over) -> Inputs:
    kw = dict(PRESETS[name])
    kw.update(over)
    inp = make_inputs(seed=seed, **kw)
    inp.recipe = name
    return inp


def packed_inputs(lengths, H: int, dk: int, dv: int, seed: int = 0,
                  s0_std: Optional[float] = 0.02, **kw) -> Inputs:
    """Packed variable-length sequences: one stream of sum(lengths) tokens per
    head (arrays [1, H, T, ...], the tokens drawn as by make_inputs), S0 of
    shape [nseq, H, dk, dv] from its own stream, and arrays["cu_seqlens"]
    (int32 [nseq + 1], the running sum of the lengths)."""
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    inp = make_inputs(1, H, T, dk, dv, seed=seed, s0_std=None, **kw)
    nseq = len(lengths)
    if s0_std is not None:
        rng = np.random.default_rng([seed, 7])
        inp.arrays["S0"] = rng.standard_normal((nseq, H, dk, dv), dtype=np.float32) * np.float32(s0_std)
    inp.arrays["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    inp.recipe = f"packed {nseq} sequences"
    return inp


def mixer_inputs(B: int, H: int, T: int, dk: int, dv: int, *, alpha_mode: str = "channel",
                 b_mode: str = "channel", w_mode: str = "channel", seed: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of the token-mixer prologue and epilogue: the projections'
    outputs q_pre, k_pre, v_pre ~ N(0, 1) (bf16 values), depthwise causal
    convolution taps [H, d, 4] ~ N(0, 1/4) (fp32), decay logits a_pre ~
    N(4, 1) (fp32; alpha = sigmoid(a_pre) is about 0.98, so a chunk of 64
    tokens decays by about 1 nat), erase/write gate logits ~ N(0, 1), the
    output-gate logits g ~ N(0, 1) and the RMS-norm weight 1 + N(0, 0.01)."""
    rng = np.random.default_rng([seed, 13])
    n = lambda *shape: rng.standard_normal(shape, dtype=np.float32)
    ash = (B, H, T, dk) if alpha_mode == "channel" else (B, H, T)
    bsh = (B, H, T, dk) if b_mode == "channel" else (B, H, T)
    wsh = (B, H, T, dv) if w_mode == "channel" else (B, H, T)
    return dict(q_pre=bf16_round(n(B, H, T, dk)), k_pre=bf16_round(n(B, H, T, dk)),
                v_pre=bf16_round(n(B, H, T, dv)),
                conv_q=n(H, dk, 4) * np.float32(0.5), conv_k=n(H, dk, 4) * np.float32(0.5),
                conv_v=n(H, dv, 4) * np.float32(0.5),
                a_pre=(n(*ash) + np.float32(4.0)).astype(np.float32),
                b_pre=bf16_round(n(*bsh)), w_pre=bf16_round(n(*wsh)),
                g=bf16_round(n(B, H, T, dv)),
                norm_weight=(np.float32(1.0) + n(dv) * np.float32(0.1)).astype(np.float32))


def packed_lengths(n: int, mean: int, seed: int = 0, lo: int = 1) -> list:
    """n sequence lengths with a long-tailed mix (geometric around mean,
    at least lo), as packed training batches of documents have."""
    rng = np.random.default_rng([seed, 11])
    return [int(max(lo, x)) for x in rng.geometric(1.0 / max(mean, 1), size=n)]


# decode workload: 256 sequences x 32 heads, d=128, fp32 state from N(0, 0.02)
DECODE = dict(N=256, H=32, dk=128, dv=128, steps=128)


def decode_state(N: int, H: int, dk: int, dv: int, seed: int = 0, std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng([seed, 0])
    return rng.standard_normal((N, H, dk, dv), dtype=np.float32) * np.float32(std)


def decode_token(N: int, H: int, dk: int, dv: int, step: int, seed: int = 0,
                 act: str = "bf16", decay_scale: float = 0.05,
                 alpha_mode: str = "channel", b_mode: str = "channel",
                 w_mode: str = "channel") -> Dict[str, np.ndarray]:
    """One token per (sequence, head) for decode step ``step`` (own stream)."""
    rng = np.random.default_rng([seed, 1 + step])
    rnd = (lambda a: bf16_round(a)) if act == "bf16" else (lambda a: a.astype(np.float32))
    q = _l2n(rng.standard_normal((N, H, dk), dtype=np.float32))
    k = _l2n(rng.standard_normal((N, H, dk), dtype=np.float32))
    v = rng.standard_normal((N, H, dv), dtype=np.float32)
    ash = (N, H, dk) if alpha_mode == "channel" else (N, H)
    la = (-_softplus(rng.standard_normal(ash, dtype=np.float32)) * np.float32(decay_scale)).astype(np.float32)
    b = _sigmoid(rng.standard_normal((N, H, dk) if b_mode == "channel" else (N, H), dtype=np.float32))
    w = _sigmoid(rng.standard_normal((N, H, dv) if w_mode == "channel" else (N, H), dtype=np.float32))
    return dict(q=rnd(q), k=rnd(k), v=rnd(v), log_alpha=la, b=rnd(b), w=rnd(w))
