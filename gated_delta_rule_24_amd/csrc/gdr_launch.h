// Internal interface between the C-ABI layer (gdr_api.cpp) and the kernel
// translation units.  Not installed; callers use include/gdr.h.
#pragma once

#include <atomic>

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdr.h"

namespace gdr {

// Raise a kernel's dynamic-LDS limit to `bytes` once per device: the setting
// belongs to the function on the current device, so a process that uses
// several GPUs sets it on each.  `done` keeps one bit per device (devices
// numbered 64 and up set it on every launch); safe to call from several threads.
inline hipError_t ensure_dyn_lds(const void* fn, int bytes, std::atomic<unsigned long long>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const float* la;
    const void* b;
    const void* w;
    float* S;
    void* o;
    long long NH;          // N * H
    uint32_t flags;
};

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    const float* la;
    const void* b;
    const void* w;
    const float* S0;       // may be null
    void* o;               // may be null (state-only passes)
    float* Sf;             // may be null
    float* states;         // optional: chunk-start states [BH][NC][DK][DV] (backward recompute,
                           // generic forward)
    void* state_frags;     // optional: decayed chunk-start states S' as f16 fragments
                           // (backward recompute, two-pass forward; wy::StateFrag layout)
    int BH;                // fixed length: B*H sequences of T tokens each
    int T;                 // packed (cu_seqlens set): BH = H heads, T = total tokens per head
    uint32_t flags;
    // packed variable-length sequences (two-pass forward only), or null:
    const int* cu_seqlens; // [nseq + 1] token offsets of the sequences within each head
    int* chunk_off;        // [nseq + 1] offsets of their chunks (filled on the device)
    int* chunk_tab;        // [chunks][2] first token and token count of each chunk (device)
    int* seq_order;        // [nseq] sequences, longest first by power-of-two chunk-count class
    int nseq;
};

hipError_t launch_decode(const DecodeParams& p, int dk, int dv, hipStream_t st);

// Returns hipErrorInvalidValue for an unsupported (dk, dv, chunk, dtype).
// *chunk_used receives the chunk size the kernel blocks with.
hipError_t launch_fwd(const FwdParams& p, int dk, int dv, int chunk, hipStream_t st,
                      int* chunk_used);
bool fwd_supported(int dk, int dv, int chunk, uint32_t flags);

// Pipelined fast path (bf16 activations, chunk 64, d_k and d_v in {64, 128}).
bool fwd_pipe_supported(int dk, int dv, int chunk, uint32_t flags);
hipError_t launch_fwd_pipe(const FwdParams& p, int dk, int dv, hipStream_t st);

// Two-pass path (chunk-parallel WY operands into a workspace, then the state
// chain): bf16 activations, chunk 64, d_k and d_v in {64, 128}, T > 0.
// bwd_layouts: also write the fragment layouts the backward's reverse chain
// reads (d_k == d_v only).
bool fwd_wy_supported(int dk, int dv, int chunk, uint32_t flags);
size_t fwd_wy_workspace_bytes(int BH, int T, int dk, int dv, bool bwd_layouts = false);
// passes: the WY pass, the state chain, or both (in that order on st).
constexpr int kWyPass = 1, kChainPass = 2;
hipError_t launch_fwd_wy(const FwdParams& p, int dk, int dv, void* ws, hipStream_t st,
                         bool bwd_layouts = false, int passes = kWyPass | kChainPass);
// The forward's producer / state-chain path (gdr_fwd_fz.hip): bf16
// activations, chunk 64, d_k and d_v in {64, 128}, T > 0 (the shapes of
// fwd_wy_supported without the backward layouts).
size_t fwd_fz_workspace_bytes(int BH, int T, int dk, int dv);
hipError_t launch_fwd_fz(const FwdParams& p, int dk, int dv, void* ws, hipStream_t st);
// Packed variable-length sequences on the same producer and chain (two
// kernels after the prep step): workspace = records, then the prep arrays.
size_t fwd_fz_varlen_workspace_bytes(int H, long long T, int nseq, int dk, int dv);
hipError_t launch_fwd_fz_varlen(const FwdParams& p, int dk, int dv, void* ws, size_t ws_bytes, hipStream_t st);
// Packed variable-length sequences.  Each head holds at most T/64 + nseq
// chunks; records and fragments are numbered head * (chunk count) + chunk.
// The prep step fills, in prep_bytes of device memory: the chunk offsets of
// the sequences, the chunk table and the longest-first sequence order.
size_t packed_max_chunks(long long T, int nseq);
size_t packed_prep_bytes(long long T, int nseq);
hipError_t launch_packed_prep(const int* cu_seqlens, int nseq, long long T, void* mem, int** chunk_off,
                              int** chunk_tab, int** seq_order, hipStream_t st);
// The two passes over packed sequences (p's prep pointers set).
hipError_t launch_fwd_wy_packed(const FwdParams& p, int dk, int dv, void* records, hipStream_t st,
                                bool bwd_layouts, int passes);

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const float* la;
    const void* b;
    const void* w;
    const float* S0;
    const void* dO;
    const float* dSf;
    float* dq;
    float* dk;
    float* dv;
    float* dla;
    float* db;
    float* dw;
    float* dS0;
    float* states;         // workspace: chunk-start states (generic path, fp32)
    float* dstates;        // workspace: state gradients at chunk ends (generic path, fp32)
    void* records;         // workspace: per-chunk WY operands of the two-pass forward (or null)
    void* state_frags;     // workspace, two-pass path: S' per chunk, f16 fragments
    void* dstate_frags;    // workspace, two-pass path: chunk-end state gradients, f16 fragments
    int BH;                // packed sequences: BH = H heads, T = total tokens per head
    int T;
    uint32_t flags;
    // packed variable-length sequences (as FwdParams), or null
    const int* cu_seqlens;
    const int* chunk_off;
    const int* chunk_tab;
    const int* seq_order;
    int nseq;
};

size_t bwd_workspace_bytes(int BH, int T, int dk, int dv, int chunk, uint32_t flags);

// Token-by-token recompute (gdr_exact.hip) of the units (fixed-length heads,
// or packed (sequence, head) pairs) whose chunkwise results are NaN because a
// chunk's decay left the operand range: the forward rewrites o and S_final,
// the backward every gradient.  Clean units cost one marker read.  The
// backward needs exact_bwd_slot_bytes() of workspace per unit processed at
// once (it processes as many as fit, at least one).
size_t exact_bwd_slot_bytes(int T, int dk, int dv);
hipError_t launch_exact_fwd(const FwdParams& p, int dk, int dv, hipStream_t st);
hipError_t launch_exact_bwd(const BwdParams& p, int dk, int dv, void* ws, size_t ws_bytes, hipStream_t st);
// Reverse state-gradient chain over the records of launch_fwd_wy(..., bwd_layouts = true).
hipError_t launch_bwd_dchain(const BwdParams& p, int dk, int dv, const void* records, hipStream_t st);
// Per-chunk gradients over those records and the f16 state fragments.
hipError_t launch_bwd_wgrad(const BwdParams& p, int dk, int dv, const void* records, hipStream_t st);
// split of that workspace: states, then state gradients, then the forward records
size_t bwd_states_bytes(int BH, int T, int dk, int dv, int chunk, uint32_t flags);
bool bwd_supported(int dk, int dv, int chunk, uint32_t flags);
// the two-pass backward (WY records, reverse chain, per-chunk gradients):
// bf16, chunk 64, d_k = d_v in {64, 128}; the only one taking GDR_GATE_LOGITS
bool bwd_two_pass_supported(int dk, int dv, int chunk, uint32_t flags);
hipError_t launch_bwd(const BwdParams& p, int dk, int dv, int chunk, hipStream_t st);
// Packed sequences (bf16, d_k == d_v in {64, 128}): workspace = records, S'
// fragments, D fragments (each for packed_max_chunks per head), prep arrays.
size_t bwd_varlen_workspace_bytes(int H, long long T, int nseq, int dk, int dv);
hipError_t launch_bwd_varlen(const BwdParams& p, int dk, int dv, void* ws, size_t ws_bytes, hipStream_t st);

// Token-mixer prologue and epilogue (bf16 streams, d in {64, 128}).
constexpr int kConvTaps = 4;   // causal convolution taps per channel
struct MixerParams {
    const void* q_pre;     // [BH, T, DK] bf16 projection outputs
    const void* k_pre;
    const void* v_pre;     // [BH, T, DV]
    const float* conv_q;   // [H, DK, kConvTaps] fp32; tap j weights token t - j
    const float* conv_k;
    const float* conv_v;   // [H, DV, kConvTaps]
    const float* a_pre;    // log-decay logits, fp32 [BH, T, DK] or [BH, T]
    const void* b_pre;     // erase-gate logits, bf16 [BH, T, DK] or [BH, T]
    const void* w_pre;     // write-gate logits, bf16 [BH, T, DV] or [BH, T]
    void* q;               // outputs: bf16 q, k [BH, T, DK], v [BH, T, DV]
    void* k;
    void* v;
    float* la;             // fp32 log alpha, shaped as a_pre
    void* b;               // bf16 gates, shaped as b_pre / w_pre
    void* w;
    int BH;
    int H;
    int T;
    uint32_t flags;        // GDR_ALPHA_SCALAR, GDR_B_SCALAR, GDR_W_SCALAR
};
struct EpilogueParams {
    const float* o;        // [rows, DV] fp32 recurrence output
    const void* g;         // [rows, DV] bf16 output-gate logits
    const float* norm_weight;  // [DV] fp32
    void* y;               // [rows, DV] bf16
    long long rows;        // B * H * T
};
struct MixerBwdParams {
    const void* q_pre;     // forward inputs, as MixerParams
    const void* k_pre;
    const void* v_pre;
    const float* conv_q;
    const float* conv_k;
    const float* conv_v;
    const float* dq;       // gradients of the prologue's q, k, v outputs, fp32
    const float* dk;
    const float* dv;
    float* dq_pre;         // outputs, fp32, shaped as the inputs
    float* dk_pre;
    float* dv_pre;
    float* dconv_q;        // fp32 [H, d, kConvTaps], written
    float* dconv_k;
    float* dconv_v;
    float* part;           // workspace: per-tile tap-gradient partials
    int BH;
    int H;
    int T;
};
struct EpilogueBwdParams {
    const float* o;
    const void* g;
    const float* norm_weight;
    const float* dy;       // gradient of y, fp32
    float* d_o;            // outputs, fp32
    float* dg;
    float* dnorm_weight;   // [DV], written
    float* part;           // workspace: per-workgroup norm-weight partials
    long long rows;
};
constexpr int kEpilogueBwdBlocks = 1024;   // workgroups of the epilogue backward
bool mixer_supported(int d);
size_t mixer_prologue_bwd_workspace_bytes(int BH, int T, int dk, int dv);
size_t mixer_epilogue_bwd_workspace_bytes(int dv);
hipError_t launch_mixer_prologue_bwd(const MixerBwdParams& p, int dk, int dv, hipStream_t st);
hipError_t launch_mixer_epilogue_bwd(const EpilogueBwdParams& p, int dv, hipStream_t st);
hipError_t launch_mixer_prologue(const MixerParams& p, int dk, int dv, hipStream_t st);
hipError_t launch_mixer_epilogue(const EpilogueParams& p, int dv, hipStream_t st);

}  // namespace gdr
