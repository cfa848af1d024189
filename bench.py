#!/usr/bin/env python3
"""Benchmark of the gated delta rule hot path on one MI355X.

Headline: the chunkwise Gated DeltaNet-2 forward (gate prep and intra-chunk
WY operands for all chunks in parallel, and the inter-chunk state pass with
the output) at B=2, H=16, T=8192, d_k=d_v=128, chunk 64, bf16 activations,
fp32 log-decay and state.  One step = one gdr_chunk_fwd call over that batch
(a flag-clearing launch, then one persistent kernel whose producer and chain
workgroups run side by side, with a workspace), inputs resident in HBM.
value = B*H*T head-tokens per second of wall time over the timed steps.

Also reported in the same JSON line: the recurrent decode step (256
sequences x 32 heads, fp32 state streamed in place) in GB/s, the same
forward over packed documents of varied lengths, the backward
(1 x 32 heads x 16384 tokens), the roofline position of the forward call
(the method's algorithmic HBM bytes per call over the measured call
duration, with the measured HBM traffic of the call), and the fp64 CPU
oracle timed on this host as a reference baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("tokens/s (B·H·T) GDN-2 chunk fwd T=8K d=128 bf16; % MFMA peak; "
          "decode GB/s")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense f16/bf16 MFMA

# forward workload
FB, FH, FT, FD, FC = 2, 16, 8192, 128, 64
# algorithmic HBM bytes per head-token: q,k,v bf16 + log_alpha fp32 + b,w bf16
# + o fp32, plus S0 read and S_final written once per head
FWD_BYTES_PER_TOKEN = 3 * FD * 2 + FD * 4 + 2 * FD * 2 + FD * 4
FWD_STATE_BYTES_PER_HEAD = 2 * FD * FD * 4
# dense MFMA work per head-token: W'S-type state products 6 d_k d_v and the
# in-chunk products 2C(3 d_k + 2 d_v)
FWD_FLOPS_PER_TOKEN = 6 * FD * FD + 2 * FC * (3 * FD + 2 * FD)

# Gated DeltaNet workload (scalar decay, one tied scalar beta as b and w, no
# S0): B=4 H=16 T=2048 d=128 chunk 64; algorithmic bytes per head-token: q, k,
# v bf16 + log-decay fp32 (one per token) + beta bf16 (one per token) + o fp32,
# plus S_final written once per head
GDN_BYTES_PER_TOKEN = 3 * FD * 2 + 4 + 2 + FD * 4
GDN_STATE_BYTES_PER_HEAD = FD * FD * 4

# decode workload
DN, DH, DD = 256, 32, 128
SMALL_DECODE_N = (1, 16)          # small-batch (latency) decode lines
DEC_BYTES_PER_HEAD = 2 * DD * DD * 4 + (2 * DD * 2 + DD * 2 + DD * 4 + DD * 2 + DD * 2) + DD * 4

# packed-sequence forward workload: the headline's 16 heads x 16384 tokens per
# head, cut into documents of long-tailed lengths (mean 1024) instead of two
# sequences of 8192
VH, VT, VMEAN = 16, 16384, 1024

# token-mixer prologue / epilogue on the forward workload's shape; algorithmic
# HBM bytes per head-token (channel gates): the prologue reads q, k, v, b, w
# logits (bf16) and the log-decay logits (fp32) and writes the same shapes;
# the epilogue reads o (fp32) and the output-gate logits (bf16), writes y (bf16)
MIX_PRO_BYTES_PER_TOKEN = 2 * (3 * FD * 2 + FD * 4 + 2 * FD * 2)
MIX_EPI_BYTES_PER_TOKEN = FD * 4 + FD * 2 + FD * 2
# with the gating fused into the recurrence's loads (GDR_GATE_LOGITS) the
# prologue reads and writes q, k, v only
MIX_QKV_BYTES_PER_TOKEN = 2 * 3 * FD * 2
# backward: the prologue's q, k, v paths read the projection outputs (bf16) and
# the gradients of q, k, v (fp32) and write the projections' gradients (fp32);
# the epilogue reads o, dy (fp32) and the gate (bf16), writes d_o and dg (fp32)
MIX_PRO_BWD_BYTES_PER_TOKEN = 3 * (FD * 2 + FD * 4 + FD * 4)
MIX_EPI_BWD_BYTES_PER_TOKEN = FD * 4 + FD * 4 + FD * 2 + 2 * FD * 4

# backward workload: B=1, H=32, T=16384, d=128, chunk 64; algorithmic bytes per
# head-token: inputs q, k, b, v, w, dO bf16 + log-decay fp32, gradients dq, dk,
# d log-decay, db, dv, dw fp32; plus S0 read and dS0 written per head
BB, BH_, BT = 1, 32, 16384
BWD_BYTES_PER_TOKEN = 6 * FD * 2 + FD * 4 + 6 * FD * 4
BWD_STATE_BYTES_PER_HEAD = 2 * FD * FD * 4

# the timed call runs the persistent producer/chain kernel; the counters in
# the traffic summary are only used while these sources are unchanged
FWD_KERNEL_SOURCES = ["gated_delta_rule_24_amd/csrc/gdr_fwd_fz.hip",
                      "gated_delta_rule_24_amd/csrc/gdr_wy.h",
                      "gated_delta_rule_24_amd/csrc/gdr_device.h",
                      "gated_delta_rule_24_amd/csrc/gdr_launch.h",
                      "gated_delta_rule_24_amd/build.py"]   # the compiler flags
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fwd_gdn2_B2H16T8192_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per forward launch from committed PMC counters, or None if
    absent or taken on a different version of the kernel source."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    txt = open(TRAFFIC_SUMMARY).read()
    m_h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_h or not m_b or m_h.group(1) != source_hash(FWD_KERNEL_SOURCES):
        return None
    return float(m_b.group(1))


def upload(inp):
    import torch
    act = torch.bfloat16 if inp.act == "bf16" else torch.float32
    out = {}
    for n, a in inp.arrays.items():
        if a is None:
            out[n] = None
            continue
        dt = torch.float32 if n in ("log_alpha", "S0") else act
        out[n] = torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    if inp.arrays["b"] is inp.arrays["w"]:
        out["w"] = out["b"]
    return out


def time_loop(fn, steps, warmup):
    """Average wall ms and event ms per call over `steps` back-to-back timed
    calls; the events are recorded on torch's current stream, where libgdr
    launches."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


_FLUSH = []


def time_cold(fn, steps):
    """Per-call event ms with the caches emptied before each call: a 1 GiB
    buffer (four times the 256 MiB Infinity Cache) is read outside the event
    window, so every call starts from HBM.  The flush reads rather than
    writes: written lines would stay dirty in the caches and be written back
    inside the next call's window.  Returns (median, min, max)."""
    import torch
    if not _FLUSH:
        _FLUSH.append(torch.zeros(1 << 28, dtype=torch.float32, device="cuda"))
    buf = _FLUSH[0]
    evs = []
    for i in range(steps):
        buf.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return ms[len(ms) // 2], ms[0], ms[-1]


def cold_stats(fn, steps, nbytes=None):
    """The cold-call (cache-flushed) median and range of one call, in us, and
    the rate of its algorithmic bytes at the median."""
    med, lo, hi = time_cold(fn, steps)
    out = {"cold_median_us": med * 1e3, "cold_min_us": lo * 1e3, "cold_max_us": hi * 1e3,
           "cold_calls": steps}
    if nbytes is not None:
        out["cold_GB_per_s"] = nbytes / (med * 1e-3) / 1e9
        out["cold_frac_hbm_peak"] = nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS
    return out


def bench_fwd(steps, warmup, name="gdn2"):
    """One gdr_chunk_fwd call per step on the named synthetic workload
    (gdn2: B=2 H=16 T=8192 channel gates; gdn: B=4 H=16 T=2048 scalar decay,
    tied scalar beta, no S0)."""
    import torch
    import gdr_synth as gs
    import gated_delta_rule_24_amd as gdr
    inp = gs.preset(name, seed=0)
    d = upload(inp)
    B, H, T, dk, dv, C = inp.B, inp.H, inp.T, inp.dk, inp.dv, inp.chunk
    o = torch.empty((B, H, T, dv), dtype=torch.float32, device="cuda")
    Sf = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda")
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    nbytes = gdr.gdr_chunk_fwd_workspace_bytes(B, H, T, dk, dv, C, flags)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda") if nbytes else None

    def step():
        gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], o, Sf,
                          B, H, T, dk, dv, C, flags, ws, nbytes)
    wall_ms, ev_ms = time_loop(step, steps, warmup)
    return inp, wall_ms, ev_ms, step


def bench_decode(steps, warmup, N=None, graph=False):
    """One decode step of N sequences x 32 heads (N defaults to the 256-sequence
    workload; small N is the low-latency decode of a few sequences).  graph:
    the timed steps are captured once into a HIP graph and replayed (no launch
    per step, as a serving loop runs them); the result is per step."""
    import torch
    import gdr_synth as gs
    import gated_delta_rule_24_amd as gdr
    N = DN if N is None else N
    S = torch.from_numpy(gs.decode_state(N, DH, DD, DD, seed=0)).cuda()
    toks = []
    for st in range(8):
        t = gs.decode_token(N, DH, DD, DD, st, seed=0)
        toks.append({n: torch.from_numpy(a).to(torch.float32 if n == "log_alpha"
                                               else torch.bfloat16).cuda() for n, a in t.items()})
    o = torch.empty((N, DH, DD), dtype=torch.float32, device="cuda")
    i = [0]

    def step():
        t = toks[i[0] % 8]
        i[0] += 1
        gdr.gdr_decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["b"], t["w"], S, o,
                            N, DH, DD, DD, 0)
    if not graph:
        wall_ms, ev_ms = time_loop(step, steps, warmup)
        return wall_ms, ev_ms, step
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            step()
    g.replay()
    wall_ms, ev_ms = time_loop(g.replay, 5, 1)
    return wall_ms / steps, ev_ms / steps


def varlen_lengths():
    """Document lengths of the packed workload: long-tailed draws, the last
    one cut so that they sum to VT."""
    import gdr_synth as gs
    out, tot = [], 0
    for n in gs.packed_lengths(4 * VT // VMEAN, VMEAN, seed=0):
        n = min(n, VT - tot)
        out.append(n)
        tot += n
        if tot == VT:
            return out
    out.append(VT - tot)
    return out


def bench_varlen(steps, warmup):
    import torch
    import gdr_synth as gs
    import gated_delta_rule_24_amd as gdr
    lengths = varlen_lengths()
    inp = gs.packed_inputs(lengths, VH, FD, FD, seed=0)
    a = inp.arrays
    d = {n: torch.from_numpy(np.ascontiguousarray(a[n][0])).to(
        torch.float32 if n == "log_alpha" else torch.bfloat16).cuda()
        for n in ("q", "k", "v", "log_alpha", "b", "w")}
    S0 = torch.from_numpy(a["S0"]).cuda()
    cu = torch.from_numpy(a["cu_seqlens"]).cuda()
    nseq = len(lengths)
    o = torch.empty((VH, VT, FD), dtype=torch.float32, device="cuda")
    Sf = torch.empty((nseq, VH, FD, FD), dtype=torch.float32, device="cuda")
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    nbytes = gdr.gdr_chunk_fwd_varlen_workspace_bytes(nseq, VH, VT, FD, FD, flags)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step():
        gdr.gdr_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0, o,
                                 Sf, cu, nseq, VH, VT, FD, FD, flags, ws, nbytes)
    wall_ms, ev_ms = time_loop(step, steps, warmup)
    return lengths, wall_ms, ev_ms, step


def bench_bwd_varlen(steps, warmup):
    """The backward workload's 32 heads x 16384 tokens packed as documents of
    the lengths varlen_lengths() gives."""
    import torch
    import gdr_synth as gs
    import gated_delta_rule_24_amd as gdr
    lengths = varlen_lengths()
    inp = gs.packed_inputs(lengths, BH_, FD, FD, seed=0, with_dO=True)
    a = inp.arrays
    d = {n: torch.from_numpy(np.ascontiguousarray(a[n][0])).to(
        torch.float32 if n == "log_alpha" else torch.bfloat16).cuda()
        for n in ("q", "k", "v", "log_alpha", "b", "w", "dO")}
    S0 = torch.from_numpy(a["S0"]).cuda()
    cu = torch.from_numpy(a["cu_seqlens"]).cuda()
    nseq = len(lengths)
    f32 = torch.float32
    g = {n: torch.empty((BH_, VT, FD), dtype=f32, device="cuda")
         for n in ("dq", "dk", "dv", "dla", "db", "dw")}
    dS0 = torch.empty((nseq, BH_, FD, FD), dtype=f32, device="cuda")
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    nbytes = gdr.gdr_chunk_bwd_varlen_workspace_bytes(nseq, BH_, VT, FD, FD, flags)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step():
        gdr.gdr_chunk_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0,
                                 d["dO"], None, g["dq"], g["dk"], g["dv"], g["dla"], g["db"],
                                 g["dw"], dS0, cu, nseq, BH_, VT, FD, FD, flags, ws, nbytes)
    wall_ms, ev_ms = time_loop(step, steps, warmup)
    return lengths, wall_ms, ev_ms, step


def bench_mixer(steps, warmup):
    """Token-mixer prologue and epilogue at B=2, H=16, T=8192, d=128 (channel
    gates), each timed on its own; returns event ms per call of each."""
    import torch
    import gdr_synth as gs
    import gated_delta_rule_24_amd as gdr
    m = gs.mixer_inputs(FB, FH, FT, FD, FD, seed=0)
    d = {n: torch.from_numpy(a).to(torch.float32 if n in ("conv_q", "conv_k", "conv_v", "a_pre",
                                                         "norm_weight") else torch.bfloat16).cuda()
         for n, a in m.items()}
    out = {n: torch.empty_like(d[src]) for n, src in (("q", "q_pre"), ("k", "k_pre"), ("v", "v_pre"),
                                                      ("la", "a_pre"), ("b", "b_pre"), ("w", "w_pre"))}
    o = torch.randn((FB, FH, FT, FD), dtype=torch.float32, device="cuda")
    y = torch.empty((FB, FH, FT, FD), dtype=torch.bfloat16, device="cuda")

    def pro():
        gdr.gdr_mixer_prologue(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                               d["conv_v"], d["a_pre"], d["b_pre"], d["w_pre"], out["q"], out["k"],
                               out["v"], out["la"], out["b"], out["w"], FB, FH, FT, FD, FD, 0)

    def epi():
        gdr.gdr_mixer_epilogue(o, d["g"], d["norm_weight"], y, FB, FH, FT, FD, 0)

    def qkv():
        gdr.gdr_mixer_prologue(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                               d["conv_v"], None, None, None, out["q"], out["k"], out["v"], None, None,
                               None, FB, FH, FT, FD, FD, gdr.GDR_GATE_LOGITS)
    # the forward taking the gate logits straight from the projections
    S0 = torch.zeros((FB, FH, FD, FD), dtype=torch.float32, device="cuda")
    of = torch.empty((FB, FH, FT, FD), dtype=torch.float32, device="cuda")
    fl = gdr.GDR_GATE_LOGITS
    nb = gdr.gdr_chunk_fwd_workspace_bytes(FB, FH, FT, FD, FD, FC, fl)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def fwd_logits():
        gdr.gdr_chunk_fwd(out["q"], out["k"], out["v"], d["a_pre"], d["b_pre"], d["w_pre"], S0, of, None,
                          FB, FH, FT, FD, FD, FC, fl, ws, nb)
    # backward of the prologue's q, k, v paths and of the epilogue
    gq = torch.randn((FB, FH, FT, FD), dtype=torch.float32, device="cuda")
    gb = {n: torch.empty((FB, FH, FT, FD), dtype=torch.float32, device="cuda")
          for n in ("dq_pre", "dk_pre", "dv_pre", "d_o", "dg")}
    gt = {n: torch.empty_like(d[n]) for n in ("conv_q", "conv_k", "conv_v")}
    dwn = torch.empty((FD,), dtype=torch.float32, device="cuda")
    nbw = gdr.gdr_mixer_bwd_workspace_bytes(FB, FH, FT, FD, FD)
    wsb = torch.empty(nbw, dtype=torch.uint8, device="cuda")

    def pro_bwd():
        gdr.gdr_mixer_prologue_bwd(d["q_pre"], d["k_pre"], d["v_pre"], d["conv_q"], d["conv_k"],
                                   d["conv_v"], gq, gq, gq, gb["dq_pre"], gb["dk_pre"], gb["dv_pre"],
                                   gt["conv_q"], gt["conv_k"], gt["conv_v"], FB, FH, FT, FD, FD, 0,
                                   wsb, nbw)

    def epi_bwd():
        gdr.gdr_mixer_epilogue_bwd(o, d["g"], d["norm_weight"], gq, gb["d_o"], gb["dg"], dwn, FB, FH,
                                   FT, FD, 0, wsb, nbw)
    _, pro_ms = time_loop(pro, steps, warmup)
    _, epi_ms = time_loop(epi, steps, warmup)
    _, qkv_ms = time_loop(qkv, steps, warmup)
    _, fl_ms = time_loop(fwd_logits, steps, warmup)
    _, pb_ms = time_loop(pro_bwd, steps, warmup)
    _, eb_ms = time_loop(epi_bwd, steps, warmup)
    return pro_ms, epi_ms, qkv_ms, fl_ms, pb_ms, eb_ms


def bench_copy(steps, warmup):
    """Plain 1 GiB device copy, the calibration kernel for HBM counters."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    wall_ms, ev_ms = time_loop(lambda: dst.copy_(src), steps, warmup)
    return wall_ms, ev_ms


def bench_bwd(steps, warmup):
    import torch
    import gdr_synth as gs
    import gated_delta_rule_24_amd as gdr
    inp = gs.preset("gdn2_bwd", seed=0)
    d = upload(inp)
    f32 = torch.float32
    shp_k, shp_v = (BB, BH_, BT, FD), (BB, BH_, BT, FD)
    g = {n: torch.empty(shp_k, dtype=f32, device="cuda") for n in ("dq", "dk", "dla", "db")}
    g.update({n: torch.empty(shp_v, dtype=f32, device="cuda") for n in ("dv", "dw")})
    dS0 = torch.empty((BB, BH_, FD, FD), dtype=f32, device="cuda")
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    nbytes = gdr.gdr_chunk_bwd_workspace_bytes(BB, BH_, BT, FD, FD, FC, flags)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step():
        gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], d["dO"],
                          None, g["dq"], g["dk"], g["dv"], g["dla"], g["db"], g["dw"], dS0,
                          BB, BH_, BT, FD, FD, FC, flags, ws, nbytes)
    wall_ms, ev_ms = time_loop(step, steps, warmup)
    return wall_ms, ev_ms, nbytes, step


def bench_strong(steps, warmup):
    """The backward workload (B=1, H=32, T=16384, d=128) with strong decay
    (synthetic decay scale 0.5: chunks of 64 tokens decay by tens of nats, so
    the chunk kernels that reference a chunk's end hand every head to the
    token-level recompute): the backward at chunk 64 and chunk 16, and the
    forward without a workspace.  Mean event ms per call of each."""
    import torch
    import gdr_synth as gs
    import gated_delta_rule_24_amd as gdr
    inp = gs.preset("gdn2_bwd", seed=0, decay_scale=0.5)
    d = upload(inp)
    f32 = torch.float32
    shp = (BB, BH_, BT, FD)
    g = {n: torch.empty(shp, dtype=f32, device="cuda") for n in ("dq", "dk", "dla", "db", "dv", "dw")}
    dS0 = torch.empty((BB, BH_, FD, FD), dtype=f32, device="cuda")
    flags = gdr.gate_flags(d["q"], d["log_alpha"], d["b"], d["w"])
    out = {}
    for chunk in (64, 16):
        nbytes = gdr.gdr_chunk_bwd_workspace_bytes(BB, BH_, BT, FD, FD, chunk, flags)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

        def step():
            gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], d["dO"],
                              None, g["dq"], g["dk"], g["dv"], g["dla"], g["db"], g["dw"], dS0,
                              BB, BH_, BT, FD, FD, chunk, flags, ws, nbytes)
        out[f"bwd_chunk{chunk}_ms"] = time_loop(step, steps, warmup)[1]
        del ws
    o = torch.empty(shp, dtype=f32, device="cuda")
    Sf = torch.empty((BB, BH_, FD, FD), dtype=f32, device="cuda")

    def fstep():
        gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], o, Sf,
                          BB, BH_, BT, FD, FD, FC, flags, None, 0)
    out["fwd_no_workspace_ms"] = time_loop(fstep, steps, warmup)[1]
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, min_seconds=10.0, max_passes=50, one_thread_seconds=4.0):
    """The fp64 oracle on this host over the same GDN-2 workload, repeated
    until about `min_seconds` of CPU work have been timed with all cores
    (OpenMP over the heads), then on one thread over the first head's first
    tokens for about `one_thread_seconds`."""
    import oracle
    a = inp.arrays
    sel = lambda x: x.reshape((FB * FH,) + x.shape[2:])
    args = [sel(a[n]) for n in ("q", "k", "v", "log_alpha", "b", "w", "S0")]
    passes = 0
    cores = oracle.num_threads()
    t0 = time.perf_counter()
    while True:
        oracle.fwd(*args)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    # one thread: one head, 2048 tokens per pass
    one = [x[:1] for x in args]
    one = [x[:, :2048] if i < 6 else x for i, x in enumerate(one)]
    p1, t1 = 0, time.perf_counter()
    while True:
        oracle.fwd(*one, nthreads=1)
        p1 += 1
        dt1 = time.perf_counter() - t1
        if dt1 >= one_thread_seconds:
            break
    return dict(value=passes * FB * FH * FT / dt, unit="tokens/s", cores=cores,
                kind="oracle", cpu_model=cpu_model(), nproc=os.cpu_count(),
                value_1thread=p1 * 2048 / dt1,
                sample=f"full workload ({FB * FH} heads x {FT} tokens, d=128), {passes} passes of "
                       f"the fp64 token recurrence, OpenMP over heads, {dt:.1f} s wall; "
                       f"value_1thread: one head x 2048 tokens on one thread, {p1} passes, "
                       f"{dt1:.1f} s wall")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["fwd", "gdn", "decode", "bwd", "copy", "varlen", "bwd_varlen",
                                       "mixer", "strong"],
                    default=None,
                    help="run one kernel only (for profiler runs); prints timings to stderr")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(heads shard across GPUs with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.only == "copy":
        w, e = bench_copy(args.steps, args.warmup)
        log(f"copy 1 GiB: {e:.3f} ms/launch, {2 * (1 << 30) / e / 1e6:.1f} GB/s")
        return
    if args.only == "decode":
        w, e, _ = bench_decode(args.steps, args.warmup)
        log(f"decode: {e * 1e3:.1f} us/step, {DN * DH * DEC_BYTES_PER_HEAD / e / 1e6:.1f} GB/s")
        return
    if args.only == "varlen":
        lengths, w, e, _ = bench_varlen(args.steps, args.warmup)
        log(f"varlen fwd ({len(lengths)} sequences): {e * 1e3:.1f} us/step")
        return
    bwd_bytes = BB * BH_ * BT * BWD_BYTES_PER_TOKEN + BB * BH_ * BWD_STATE_BYTES_PER_HEAD
    if args.only == "bwd":
        w, e, _, _ = bench_bwd(args.steps, args.warmup)
        log(f"bwd: {e * 1e3:.1f} us/step, {bwd_bytes / e / 1e6:.1f} GB/s")
        return
    if args.only == "mixer":
        pm, em, qm, fm, pbm, ebm = bench_mixer(args.steps, args.warmup)
        log(f"mixer prologue {pm * 1e3:.1f} us, epilogue {em * 1e3:.1f} us, q/k/v-only prologue "
            f"{qm * 1e3:.1f} us, forward on gate logits {fm * 1e3:.1f} us, prologue backward "
            f"{pbm * 1e3:.1f} us, epilogue backward {ebm * 1e3:.1f} us")
        return
    if args.only == "strong":
        r = bench_strong(min(args.steps, 3), min(args.warmup, 1))
        log("strong decay (decay scale 0.5): " + ", ".join(f"{k} {v:.2f}" for k, v in r.items()))
        return
    if args.only == "bwd_varlen":
        lengths, w, e, _ = bench_bwd_varlen(args.steps, args.warmup)
        log(f"bwd varlen ({len(lengths)} sequences): {e * 1e3:.1f} us/step")
        return

    if args.only == "gdn":
        inp, w, e, _ = bench_fwd(args.steps, args.warmup, "gdn")
        log(f"gdn fwd: {e * 1e3:.1f} us/step")
        return
    inp, wall_ms, ev_ms, fwd_step = bench_fwd(args.steps, args.warmup)
    ntok = FB * FH * FT
    fwd_bytes = ntok * FWD_BYTES_PER_TOKEN + FB * FH * FWD_STATE_BYTES_PER_HEAD
    fwd_flops = ntok * FWD_FLOPS_PER_TOKEN
    achieved = fwd_bytes / (ev_ms * 1e-3) / 1e9
    log(f"fwd: wall {wall_ms * 1e3:.1f} us/step, kernel {ev_ms * 1e3:.1f} us/launch, "
        f"{achieved:.0f} GB/s, {fwd_flops / (ev_ms * 1e-3) / 1e12:.1f} TFLOP/s")
    if args.only == "fwd":
        return

    fwd_cold = cold_stats(fwd_step, args.steps, fwd_bytes)
    log(f"fwd cold (caches flushed before each call): median {fwd_cold['cold_median_us']:.1f} us")

    # Gated DeltaNet (scalar decay, tied scalar beta): B=4 H=16 T=2048
    ginp, g_wall, g_ev, g_step = bench_fwd(args.steps, args.warmup, "gdn")
    g_ntok = ginp.B * ginp.H * ginp.T
    g_bytes = g_ntok * GDN_BYTES_PER_TOKEN + ginp.B * ginp.H * GDN_STATE_BYTES_PER_HEAD
    g_cold = cold_stats(g_step, args.steps, g_bytes)
    log(f"gdn fwd: {g_ev * 1e3:.1f} us/call back to back, cold median {g_cold['cold_median_us']:.1f} us")

    dec_wall, dec_ev, dec_step = bench_decode(max(args.steps, 10), args.warmup)
    dec_gbs = DN * DH * DEC_BYTES_PER_HEAD / (dec_ev * 1e-3) / 1e9
    dec_cold = cold_stats(dec_step, 10, DN * DH * DEC_BYTES_PER_HEAD)
    log(f"decode: {dec_ev * 1e3:.1f} us/step, {dec_gbs:.0f} GB/s; cold median "
        f"{dec_cold['cold_median_us']:.1f} us")
    small = {}
    for n in SMALL_DECODE_N:
        _, ev, _ = bench_decode(max(args.steps, 20), args.warmup, N=n)
        _, evg = bench_decode(64, args.warmup, N=n, graph=True)
        small[f"N={n}"] = {"us_per_step": ev * 1e3,
                           "us_per_step_graph": evg * 1e3,
                           "GB_per_s": n * DH * DEC_BYTES_PER_HEAD / (ev * 1e-3) / 1e9}
        log(f"decode N={n}: {ev * 1e3:.1f} us/step, {evg * 1e3:.1f} us/step replayed from a graph")

    lengths, var_wall, var_ev, _ = bench_varlen(args.steps, args.warmup)
    var_bytes = VH * VT * FWD_BYTES_PER_TOKEN + len(lengths) * VH * FWD_STATE_BYTES_PER_HEAD
    var_gbs = var_bytes / (var_ev * 1e-3) / 1e9
    log(f"varlen fwd ({len(lengths)} sequences, longest {max(lengths)}): "
        f"{var_ev * 1e3:.1f} us/step, {var_gbs:.0f} GB/s")

    mix_pro_ms, mix_epi_ms, mix_qkv_ms, mix_fl_ms, mix_pb_ms, mix_eb_ms = bench_mixer(args.steps, args.warmup)
    ntok_mix = FB * FH * FT
    mix_pro_gbs = ntok_mix * MIX_PRO_BYTES_PER_TOKEN / (mix_pro_ms * 1e-3) / 1e9
    mix_epi_gbs = ntok_mix * MIX_EPI_BYTES_PER_TOKEN / (mix_epi_ms * 1e-3) / 1e9
    log(f"mixer: prologue {mix_pro_ms * 1e3:.1f} us ({mix_pro_gbs:.0f} GB/s), "
        f"epilogue {mix_epi_ms * 1e3:.1f} us ({mix_epi_gbs:.0f} GB/s)")

    bwd_wall, bwd_ev, bwd_ws, bwd_step = bench_bwd(max(3, args.steps // 4), min(args.warmup, 2))
    bwd_cold = cold_stats(bwd_step, 5, bwd_bytes)
    bwd_gbs = bwd_bytes / (bwd_ev * 1e-3) / 1e9
    log(f"bwd: {bwd_ev * 1e3:.1f} us/step, {bwd_gbs:.0f} GB/s")

    _, bv_wall, bv_ev, _ = bench_bwd_varlen(max(3, args.steps // 4), min(args.warmup, 2))
    bv_bytes = BH_ * VT * BWD_BYTES_PER_TOKEN + len(lengths) * BH_ * BWD_STATE_BYTES_PER_HEAD
    log(f"bwd varlen: {bv_ev * 1e3:.1f} us/step, {bv_bytes / (bv_ev * 1e-3) / 1e9:.0f} GB/s")

    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": ntok / (wall_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "gdn2_chunk_fwd B=2 H=16 T=8192 d_k=d_v=128 chunk=64",
            "B": FB, "H": FH, "T": FT, "d_k": FD, "d_v": FD, "chunk": FC,
            "activations": "bf16", "mfma_operands": "f16", "accumulate": "f32",
            "state": "f32", "log_decay": "f32", "o": "f32",
            "gates": "channel log_alpha, channel b (erase), channel w (write)",
            "parallelism": "single GPU",
        },
        "roofline": {
            "scope": "one gdr_chunk_fwd call: fz_clear + fused_kernel (producer and chain roles)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "event_scope": "HIP events on the launch stream around the timed region's back-to-back "
                           "calls (mean per call)",
            **fwd_cold,
        },
        "gdn_fwd": {
            "workload": "gdn_chunk_fwd (Gated DeltaNet: scalar decay, tied scalar beta, S0 = 0) "
                        "B=4 H=16 T=2048 d_k=d_v=128 chunk=64",
            "us_per_call": g_ev * 1e3,
            "head_tokens_per_s": g_ntok / (g_wall * 1e-3),
            "GB_per_s": g_bytes / (g_ev * 1e-3) / 1e9,
            "frac_hbm_peak": g_bytes / (g_ev * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_call": g_bytes,
            "bytes_per_head_token": GDN_BYTES_PER_TOKEN + GDN_STATE_BYTES_PER_HEAD / ginp.T,
            **g_cold,
        },
        "mfma": {
            "achieved": fwd_flops / (ev_ms * 1e-3) / 1e12,
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": fwd_flops / (ev_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "flops_per_launch": fwd_flops,
        },
        "fwd_kernel_us": ev_ms * 1e3,
        "fwd_bytes_per_launch": fwd_bytes,
        "decode": {
            "workload": "decode N=256 H=32 d=128 fp32 state in place",
            "us_per_step": dec_ev * 1e3,
            "GB_per_s": dec_gbs,
            "frac_hbm_peak": dec_gbs / HBM_PEAK_GBS,
            "bytes_per_step": DN * DH * DEC_BYTES_PER_HEAD,
            **dec_cold,
            "small_batch": {"workload": "decode H=32 d=128, N sequences (latency); us_per_step: "
                                        "back-to-back launches, us_per_step_graph: 64 steps "
                                        "replayed from one HIP graph", **small},
        },
        "varlen_fwd": {
            "workload": (f"gdn2_chunk_fwd_varlen H={VH}, {VT} tokens per head packed as "
                         f"{len(lengths)} documents (long-tailed lengths, mean {VMEAN}), "
                         f"d_k=d_v=128"),
            "lengths_min_max": [min(lengths), max(lengths)],
            "us_per_step": var_ev * 1e3,
            "wall_us_per_step": var_wall * 1e3,
            "head_tokens_per_s": VH * VT / (var_wall * 1e-3),
            "GB_per_s": var_gbs,
            "frac_hbm_peak": var_gbs / HBM_PEAK_GBS,
            "bytes_per_step": var_bytes,
        },
        "mixer": {
            "workload": "token-mixer prologue (conv+SiLU+L2 norm of q, k; conv+SiLU of v; "
                        "gates) and epilogue (RMS norm x SiLU gate) at B=2 H=16 T=8192 d=128",
            "prologue_us": mix_pro_ms * 1e3,
            "prologue_GB_per_s": mix_pro_gbs,
            "prologue_frac_hbm_peak": mix_pro_gbs / HBM_PEAK_GBS,
            "epilogue_us": mix_epi_ms * 1e3,
            "epilogue_GB_per_s": mix_epi_gbs,
            "epilogue_frac_hbm_peak": mix_epi_gbs / HBM_PEAK_GBS,
            "bytes_per_head_token": [MIX_PRO_BYTES_PER_TOKEN, MIX_EPI_BYTES_PER_TOKEN],
            "gating_fused": {
                "what": "prologue producing q, k, v only; the forward reading the gate logits "
                        "(GDR_GATE_LOGITS)",
                "prologue_qkv_us": mix_qkv_ms * 1e3,
                "prologue_qkv_GB_per_s": ntok_mix * MIX_QKV_BYTES_PER_TOKEN / (mix_qkv_ms * 1e-3) / 1e9,
                "fwd_on_logits_us": mix_fl_ms * 1e3,
                "block_us": (mix_qkv_ms + mix_fl_ms + mix_epi_ms) * 1e3,
                "block_us_unfused": (mix_pro_ms + ev_ms + mix_epi_ms) * 1e3,
            },
            "backward": {
                "prologue_qkv_bwd_us": mix_pb_ms * 1e3,
                "prologue_qkv_bwd_GB_per_s":
                    ntok_mix * MIX_PRO_BWD_BYTES_PER_TOKEN / (mix_pb_ms * 1e-3) / 1e9,
                "epilogue_bwd_us": mix_eb_ms * 1e3,
                "epilogue_bwd_GB_per_s":
                    ntok_mix * MIX_EPI_BWD_BYTES_PER_TOKEN / (mix_eb_ms * 1e-3) / 1e9,
            },
        },
        "backward": {
            "workload": "gdn2_chunk_bwd B=1 H=32 T=16384 d_k=d_v=128 chunk=64, dO only",
            "us_per_step": bwd_ev * 1e3,
            "head_tokens_per_s": BB * BH_ * BT / (bwd_ev * 1e-3),
            "GB_per_s": bwd_gbs,
            "frac_hbm_peak": bwd_gbs / HBM_PEAK_GBS,
            "bytes_per_step": bwd_bytes,
            "workspace_bytes": bwd_ws,
            **bwd_cold,
        },
        "varlen_bwd": {
            "workload": (f"gdn2_chunk_bwd_varlen H={BH_}, {VT} tokens per head packed as "
                         f"{len(lengths)} documents (the varlen_fwd lengths), d_k=d_v=128, dO only"),
            "us_per_step": bv_ev * 1e3,
            "head_tokens_per_s": BH_ * VT / (bv_wall * 1e-3),
            "GB_per_s": bv_bytes / (bv_ev * 1e-3) / 1e9,
            "frac_hbm_peak": bv_bytes / (bv_ev * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_step": bv_bytes,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
