// C ABI of libgdr: argument validation, kernel selection and launch on the
// caller's stream.  Declarations and the contract are in include/gdr.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string.h>

#include "gdr_launch.h"

namespace {

constexpr uint32_t kKnownFlags = GDR_ACT_F32 | GDR_OUT_BF16 | GDR_ALPHA_SCALAR | GDR_B_SCALAR |
                                 GDR_W_SCALAR | GDR_FWD_GENERIC | GDR_GATE_LOGITS | GDR_FWD_SPLIT;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool head_size_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Sequences are counted in 32-bit integers inside the kernels and token
// offsets in 64-bit ones: B*H must stay below 2^28 and B*H*T below 2^40, so
// that no product the kernels form can overflow.
bool sizes_ok(int B, int H, int T) {
    return (long long)B * H <= (1LL << 28) && (long long)B * H * (long long)T <= (1LL << 40);
}

// Lazily checks, per device, that the current device is a gfx950.
gdr_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GDR_ERR_DEVICE;
    static std::mutex mu;
    static int known[64];  // 0 unknown, 1 ok, 2 bad
    if (dev >= 64) return GDR_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(mu);
    if (known[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GDR_ERR_DEVICE;
        known[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    }
    return known[dev] == 1 ? GDR_OK : GDR_ERR_DEVICE;
}

// A backward workspace also holds, after the chunk kernels are done with it,
// one slot of the token-by-token recompute (checkpoints every 64 tokens and one
// segment's states), for the heads whose decay left the chunk kernels' range.
size_t bwd_need(size_t fast, int T, int d_k, int d_v) {
    if (fast == 0 || T <= 0) return fast;
    const size_t slot = gdr::exact_bwd_slot_bytes(T, d_k, d_v);
    return fast > slot ? fast : slot;
}

gdr_status from_hip(hipError_t e) {
    if (e == hipSuccess) return GDR_OK;
    if (e == hipErrorInvalidValue) return GDR_ERR_UNSUPPORTED;
    return GDR_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char* gdr_status_string(gdr_status s) {
    switch (s) {
        case GDR_OK: return "ok";
        case GDR_ERR_INVALID_ARG: return "invalid argument";
        case GDR_ERR_UNSUPPORTED: return "unsupported shape, chunk or dtype";
        case GDR_ERR_WORKSPACE: return "workspace missing or too small";
        case GDR_ERR_LAUNCH: return "kernel launch failed";
        case GDR_ERR_DEVICE: return "no usable gfx950 device";
    }
    return "unknown status";
}

size_t gdr_chunk_fwd_workspace_bytes(int B, int H, int T, int d_k, int d_v, int chunk,
                                     uint32_t flags) {
    if (B < 1 || H < 1 || T < 1 || !(chunk == 16 || chunk == 32 || chunk == 64)) return 0;
    if (T % chunk != 0 || !sizes_ok(B, H, T)) return 0;
    if (!gdr::fwd_wy_supported(d_k, d_v, chunk, flags)) return 0;
    return gdr::fwd_fz_workspace_bytes(B * H, T, d_k, d_v);
}

gdr_status gdr_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                         const void* b, const void* w, const float* S0, void* o, float* S_final,
                         int B, int H, int T, int d_k, int d_v, int chunk, uint32_t flags,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if (flags & ~kKnownFlags) return GDR_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || T < 0) return GDR_ERR_INVALID_ARG;
    if (!(chunk == 16 || chunk == 32 || chunk == 64)) return GDR_ERR_INVALID_ARG;
    if (T % chunk != 0) return GDR_ERR_INVALID_ARG;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return GDR_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !log_alpha || !b || !w || !o)) return GDR_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, log_alpha, b, w, S0, o, S_final, workspace};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDR_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, T)) return GDR_ERR_INVALID_ARG;
    if (!gdr::fwd_supported(d_k, d_v, chunk, flags)) return GDR_ERR_UNSUPPORTED;
    const size_t need = gdr_chunk_fwd_workspace_bytes(B, H, T, d_k, d_v, chunk, flags);
    const bool two_pass = workspace != nullptr && need > 0;
    if (two_pass && workspace_bytes < need) return GDR_ERR_WORKSPACE;
    if ((flags & GDR_GATE_LOGITS) && T > 0 && !two_pass) return GDR_ERR_UNSUPPORTED;
    gdr_status ds = check_device();
    if (ds != GDR_OK) return ds;

    gdr::FwdParams p;
    p.q = q; p.k = k; p.v = v; p.la = log_alpha; p.b = b; p.w = w;
    p.S0 = S0; p.o = o; p.Sf = S_final; p.states = nullptr; p.state_frags = nullptr;
    p.cu_seqlens = nullptr; p.chunk_off = nullptr; p.chunk_tab = nullptr; p.seq_order = nullptr; p.nseq = 0;
    p.BH = B * H; p.T = T; p.flags = flags;
    if (two_pass) return from_hip(gdr::launch_fwd_fz(p, d_k, d_v, workspace, (hipStream_t)stream));
    int used = 0;
    const hipError_t e = gdr::launch_fwd(p, d_k, d_v, chunk, (hipStream_t)stream, &used);
    if (e != hipSuccess) return from_hip(e);
    // heads whose decay left the chunk kernel's operand range: token by token
    return from_hip(gdr::launch_exact_fwd(p, d_k, d_v, (hipStream_t)stream));
}

size_t gdr_chunk_fwd_varlen_workspace_bytes(int nseq, int H, int T, int d_k, int d_v,
                                            uint32_t flags) {
    if (nseq < 1 || H < 1 || T < 0 || (long long)nseq * H > (1LL << 28)) return 0;
    if ((flags & ~kKnownFlags) || !gdr::fwd_wy_supported(d_k, d_v, 64, flags)) return 0;
    return gdr::fwd_fz_varlen_workspace_bytes(H, T, nseq, d_k, d_v);
}

gdr_status gdr_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                                const float* log_alpha, const void* b, const void* w,
                                const float* S0, void* o, float* S_final,
                                const int* cu_seqlens, int nseq, int H, int T,
                                int d_k, int d_v, uint32_t flags, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (flags & ~kKnownFlags) return GDR_ERR_INVALID_ARG;
    if (nseq < 1 || H < 1 || T < 0 || !cu_seqlens) return GDR_ERR_INVALID_ARG;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return GDR_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !log_alpha || !b || !w || !o)) return GDR_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, log_alpha, b, w, S0, o, S_final, workspace};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDR_ERR_INVALID_ARG;
    // work items (head, chunk) are numbered in 32-bit integers
    if ((long long)nseq * H > (1LL << 28) || (long long)H * (T / 64 + nseq) > (1LL << 30))
        return GDR_ERR_INVALID_ARG;
    if (!gdr::fwd_wy_supported(d_k, d_v, 64, flags)) return GDR_ERR_UNSUPPORTED;
    const size_t need = gdr::fwd_fz_varlen_workspace_bytes(H, T, nseq, d_k, d_v);
    if (!workspace || workspace_bytes < need) return GDR_ERR_WORKSPACE;
    gdr_status ds = check_device();
    if (ds != GDR_OK) return ds;

    gdr::FwdParams p;
    p.q = q; p.k = k; p.v = v; p.la = log_alpha; p.b = b; p.w = w;
    p.S0 = S0; p.o = o; p.Sf = S_final; p.states = nullptr; p.state_frags = nullptr;
    p.cu_seqlens = cu_seqlens; p.chunk_off = nullptr; p.chunk_tab = nullptr; p.seq_order = nullptr; p.nseq = nseq;
    p.BH = H; p.T = T; p.flags = flags;
    // the producer over every packed chunk, then one chain per (sequence, head);
    // their operands reference each block's own decay, so any decay gives values
    return from_hip(gdr::launch_fwd_fz_varlen(p, d_k, d_v, workspace, workspace_bytes, (hipStream_t)stream));
}

gdr_status gdr_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                           const void* b, const void* w, float* S, void* o, int N, int H,
                           int d_k, int d_v, uint32_t flags, void* stream) {
    if (flags & ~(kKnownFlags & ~GDR_FWD_SPLIT)) return GDR_ERR_INVALID_ARG;
    if (N < 1 || H < 1) return GDR_ERR_INVALID_ARG;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return GDR_ERR_UNSUPPORTED;
    if (!q || !k || !v || !log_alpha || !b || !w || !S || !o) return GDR_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, log_alpha, b, w, S, o};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return GDR_ERR_INVALID_ARG;
    if ((long long)N * H > (1LL << 31) - 1) return GDR_ERR_INVALID_ARG;
    gdr_status ds = check_device();
    if (ds != GDR_OK) return ds;

    gdr::DecodeParams p;
    p.q = q; p.k = k; p.v = v; p.la = log_alpha; p.b = b; p.w = w; p.S = S; p.o = o;
    p.NH = (long long)N * H; p.flags = flags;
    return from_hip(gdr::launch_decode(p, d_k, d_v, (hipStream_t)stream));
}

size_t gdr_chunk_bwd_workspace_bytes(int B, int H, int T, int d_k, int d_v, int chunk,
                                     uint32_t flags) {
    if (B < 1 || H < 1 || T < 0 || !(chunk == 16 || chunk == 32 || chunk == 64)) return 0;
    if (T % chunk != 0 || !sizes_ok(B, H, T)) return 0;
    if (!gdr::bwd_supported(d_k, d_v, chunk, flags)) return 0;
    return bwd_need(gdr::bwd_workspace_bytes(B * H, T, d_k, d_v, chunk, flags), T, d_k, d_v);
}

gdr_status gdr_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha,
                         const void* b, const void* w, const float* S0, const void* dO,
                         const float* dS_final, float* dq, float* dk, float* dv,
                         float* dlog_alpha, float* db, float* dw, float* dS0, int B, int H,
                         int T, int d_k, int d_v, int chunk, uint32_t flags, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (flags & ~(kKnownFlags & ~GDR_OUT_BF16)) return GDR_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || T < 0) return GDR_ERR_INVALID_ARG;
    if (!(chunk == 16 || chunk == 32 || chunk == 64)) return GDR_ERR_INVALID_ARG;
    if (T % chunk != 0) return GDR_ERR_INVALID_ARG;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return GDR_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !log_alpha || !b || !w || !dO || !dq || !dk || !dv ||
                  !dlog_alpha || !db || !dw))
        return GDR_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, log_alpha, b, w, S0, dO, dS_final, dq, dk, dv,
                          dlog_alpha, db, dw, dS0, workspace};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDR_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, T)) return GDR_ERR_INVALID_ARG;
    if (!gdr::bwd_supported(d_k, d_v, chunk, flags)) return GDR_ERR_UNSUPPORTED;
    if ((flags & GDR_GATE_LOGITS) && T > 0 && !gdr::bwd_two_pass_supported(d_k, d_v, chunk, flags))
        return GDR_ERR_UNSUPPORTED;
    const size_t need = gdr::bwd_workspace_bytes(B * H, T, d_k, d_v, chunk, flags);
    if (need > 0 && (!workspace || workspace_bytes < bwd_need(need, T, d_k, d_v))) return GDR_ERR_WORKSPACE;
    gdr_status ds = check_device();
    if (ds != GDR_OK) return ds;

    gdr::BwdParams p;
    p.q = q; p.k = k; p.v = v; p.la = log_alpha; p.b = b; p.w = w; p.S0 = S0;
    p.dO = dO; p.dSf = dS_final;
    p.dq = dq; p.dk = dk; p.dv = dv; p.dla = dlog_alpha; p.db = db; p.dw = dw; p.dS0 = dS0;
    p.states = nullptr; p.dstates = nullptr; p.records = nullptr;
    p.state_frags = nullptr; p.dstate_frags = nullptr;
    p.cu_seqlens = nullptr; p.chunk_off = nullptr; p.chunk_tab = nullptr; p.seq_order = nullptr; p.nseq = 0;
    p.BH = B * H; p.T = T; p.flags = flags;
    if (need > 0) {
        const size_t sb = gdr::bwd_states_bytes(B * H, T, d_k, d_v, chunk, flags);
        char* base = reinterpret_cast<char*>(workspace);
        // states, then state gradients (fp32 rows for the generic path, f16
        // fragments for the two-pass path), then the two-pass forward's records
        p.states = reinterpret_cast<float*>(base);
        p.dstates = reinterpret_cast<float*>(base + sb);
        p.state_frags = base;
        p.dstate_frags = base + sb;
        if (need > 2 * sb) p.records = base + 2 * sb;
    }
    const hipError_t e = gdr::launch_bwd(p, d_k, d_v, chunk, (hipStream_t)stream);
    if (e != hipSuccess) return from_hip(e);
    // heads whose decay left the chunk kernels' operand range: token by token,
    // in the workspace the chunk kernels are done with
    return from_hip(gdr::launch_exact_bwd(p, d_k, d_v, workspace, workspace_bytes, (hipStream_t)stream));
}

size_t gdr_chunk_bwd_varlen_workspace_bytes(int nseq, int H, int T, int d_k, int d_v, uint32_t flags) {
    if (nseq < 1 || H < 1 || T < 0 || (long long)nseq * H > (1LL << 28)) return 0;
    if ((flags & ~(kKnownFlags & ~GDR_OUT_BF16)) || !gdr::fwd_wy_supported(d_k, d_v, 64, flags)) return 0;
    return bwd_need(gdr::bwd_varlen_workspace_bytes(H, T, nseq, d_k, d_v), T, d_k, d_v);
}

gdr_status gdr_chunk_bwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                                const void* b, const void* w, const float* S0, const void* dO,
                                const float* dS_final, float* dq, float* dk, float* dv,
                                float* dlog_alpha, float* db, float* dw, float* dS0,
                                const int* cu_seqlens, int nseq, int H, int T, int d_k, int d_v,
                                uint32_t flags, void* workspace, size_t workspace_bytes, void* stream) {
    if (flags & ~(kKnownFlags & ~GDR_OUT_BF16)) return GDR_ERR_INVALID_ARG;
    if (nseq < 1 || H < 1 || T < 0 || !cu_seqlens) return GDR_ERR_INVALID_ARG;
    if (!head_size_ok(d_k) || !head_size_ok(d_v)) return GDR_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !log_alpha || !b || !w || !dO || !dq || !dk || !dv ||
                  !dlog_alpha || !db || !dw))
        return GDR_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, log_alpha, b, w, S0, dO, dS_final, dq, dk, dv,
                          dlog_alpha, db, dw, dS0, workspace};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDR_ERR_INVALID_ARG;
    // work items (head, chunk) are numbered in 32-bit integers
    if ((long long)nseq * H > (1LL << 28) || (long long)H * (T / 64 + nseq) > (1LL << 30))
        return GDR_ERR_INVALID_ARG;
    if (d_k != d_v || !gdr::fwd_wy_supported(d_k, d_v, 64, flags)) return GDR_ERR_UNSUPPORTED;
    const size_t need = bwd_need(gdr::bwd_varlen_workspace_bytes(H, T, nseq, d_k, d_v), T, d_k, d_v);
    if (!workspace || workspace_bytes < need) return GDR_ERR_WORKSPACE;
    gdr_status ds = check_device();
    if (ds != GDR_OK) return ds;

    gdr::BwdParams p;
    p.q = q; p.k = k; p.v = v; p.la = log_alpha; p.b = b; p.w = w; p.S0 = S0;
    p.dO = dO; p.dSf = dS_final;
    p.dq = dq; p.dk = dk; p.dv = dv; p.dla = dlog_alpha; p.db = db; p.dw = dw; p.dS0 = dS0;
    p.states = nullptr; p.dstates = nullptr; p.records = nullptr;
    p.state_frags = nullptr; p.dstate_frags = nullptr;
    p.cu_seqlens = cu_seqlens; p.chunk_off = nullptr; p.chunk_tab = nullptr; p.seq_order = nullptr;
    p.nseq = nseq;
    p.BH = H; p.T = T; p.flags = flags;
    const hipError_t e = gdr::launch_bwd_varlen(p, d_k, d_v, workspace, workspace_bytes, (hipStream_t)stream);
    if (e != hipSuccess) return from_hip(e);
    // sequences whose decay left the chunk kernels' operand range: token by token
    return from_hip(gdr::launch_exact_bwd(p, d_k, d_v, workspace, workspace_bytes, (hipStream_t)stream));
}

gdr_status gdr_mixer_prologue(const void* q_pre, const void* k_pre, const void* v_pre,
                              const float* conv_q, const float* conv_k, const float* conv_v,
                              const float* a_pre, const void* b_pre, const void* w_pre, void* q,
                              void* k, void* v, float* log_alpha, void* b, void* w, int B, int H,
                              int T, int d_k, int d_v, uint32_t flags, void* stream) {
    const uint32_t gate_modes = GDR_ALPHA_SCALAR | GDR_B_SCALAR | GDR_W_SCALAR | GDR_GATE_LOGITS;
    if (flags & ~(kKnownFlags & ~GDR_OUT_BF16 & ~GDR_FWD_GENERIC)) return GDR_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || T < 0) return GDR_ERR_INVALID_ARG;
    if ((long long)B * H > (1LL << 28) || (long long)B * H * (((long long)T + 63) / 64) > (1LL << 31) - 1)
        return GDR_ERR_INVALID_ARG;
    if (!gdr::mixer_supported(d_k) || !gdr::mixer_supported(d_v) || (flags & ~gate_modes))
        return GDR_ERR_UNSUPPORTED;
    // with GDR_GATE_LOGITS the gates stay logits for the recurrence to take:
    // only q, k and v are produced and the gate pointers are not used
    const bool gates = !(flags & GDR_GATE_LOGITS);
    const void* ptrs[] = {q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, q, k, v,
                          a_pre, b_pre, w_pre, log_alpha, b, w};
    for (int i = 0; i < 15; ++i) {
        const void* ptr = ptrs[i];
        if (T > 0 && !ptr && (i < 9 || gates)) return GDR_ERR_INVALID_ARG;
        if (ptr && !aligned16(ptr)) return GDR_ERR_INVALID_ARG;
    }
    gdr_status ds = check_device();
    if (ds != GDR_OK) return ds;
    gdr::MixerParams p;
    p.q_pre = q_pre; p.k_pre = k_pre; p.v_pre = v_pre;
    p.conv_q = conv_q; p.conv_k = conv_k; p.conv_v = conv_v;
    p.a_pre = a_pre; p.b_pre = b_pre; p.w_pre = w_pre;
    p.q = q; p.k = k; p.v = v; p.la = log_alpha; p.b = b; p.w = w;
    p.BH = B * H; p.H = H; p.T = T; p.flags = flags;
    return from_hip(gdr::launch_mixer_prologue(p, d_k, d_v, (hipStream_t)stream));
}

gdr_status gdr_mixer_epilogue(const float* o, const void* g, const float* norm_weight, void* y,
                              int B, int H, int T, int d_v, uint32_t flags, void* stream) {
    if (flags != 0) return GDR_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || T < 0) return GDR_ERR_INVALID_ARG;
    if ((long long)B * H > (1LL << 28) || (long long)B * H * T > (1LL << 40)) return GDR_ERR_INVALID_ARG;
    if (!gdr::mixer_supported(d_v)) return GDR_ERR_UNSUPPORTED;
    const void* ptrs[] = {o, g, norm_weight, y};
    for (const void* ptr : ptrs) {
        if (T > 0 && !ptr) return GDR_ERR_INVALID_ARG;
        if (ptr && !aligned16(ptr)) return GDR_ERR_INVALID_ARG;
    }
    gdr_status ds = check_device();
    if (ds != GDR_OK) return ds;
    gdr::EpilogueParams p;
    p.o = o; p.g = g; p.norm_weight = norm_weight; p.y = y;
    p.rows = (long long)B * H * T;
    return from_hip(gdr::launch_mixer_epilogue(p, d_v, (hipStream_t)stream));
}

size_t gdr_mixer_bwd_workspace_bytes(int B, int H, int T, int d_k, int d_v) {
    if (B < 1 || H < 1 || T < 1 || d_k != d_v || !gdr::mixer_supported(d_k)) return 0;
    if ((long long)B * H > (1LL << 28) || (long long)B * H * (((long long)T + 63) / 64) > (1LL << 31) - 1) return 0;
    const size_t pro = gdr::mixer_prologue_bwd_workspace_bytes(B * H, T, d_k, d_v);
    const size_t epi = gdr::mixer_epilogue_bwd_workspace_bytes(d_v);
    return pro > epi ? pro : epi;
}

gdr_status gdr_mixer_prologue_bwd(const void* q_pre, const void* k_pre, const void* v_pre,
                                  const float* conv_q, const float* conv_k, const float* conv_v,
                                  const float* dq, const float* dk, const float* dv, float* dq_pre,
                                  float* dk_pre, float* dv_pre, float* dconv_q, float* dconv_k,
                                  float* dconv_v, int B, int H, int T, int d_k, int d_v,
                                  uint32_t flags, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    if (flags != 0) return GDR_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || T < 1) return GDR_ERR_INVALID_ARG;
    if (d_k != d_v || !gdr::mixer_supported(d_k)) return GDR_ERR_UNSUPPORTED;
    const void* ptrs[] = {q_pre, k_pre, v_pre, conv_q, conv_k, conv_v, dq, dk, dv, dq_pre, dk_pre,
                          dv_pre, dconv_q, dconv_k, dconv_v, workspace};
    for (const void* ptr : ptrs)
        if (!ptr || !aligned16(ptr)) return GDR_ERR_INVALID_ARG;
    const size_t need = gdr_mixer_bwd_workspace_bytes(B, H, T, d_k, d_v);
    if (need == 0) return GDR_ERR_INVALID_ARG;
    if (workspace_bytes < need) return GDR_ERR_WORKSPACE;
    gdr_status ds = check_device();
    if (ds != GDR_OK) return ds;
    gdr::MixerBwdParams p;
    p.q_pre = q_pre; p.k_pre = k_pre; p.v_pre = v_pre;
    p.conv_q = conv_q; p.conv_k = conv_k; p.conv_v = conv_v;
    p.dq = dq; p.dk = dk; p.dv = dv; p.dq_pre = dq_pre; p.dk_pre = dk_pre; p.dv_pre = dv_pre;
    p.dconv_q = dconv_q; p.dconv_k = dconv_k; p.dconv_v = dconv_v;
    p.part = reinterpret_cast<float*>(workspace);
    p.BH = B * H; p.H = H; p.T = T;
    return from_hip(gdr::launch_mixer_prologue_bwd(p, d_k, d_v, (hipStream_t)stream));
}

gdr_status gdr_mixer_epilogue_bwd(const float* o, const void* g, const float* norm_weight,
                                  const float* dy, float* d_o, float* dg, float* dnorm_weight,
                                  int B, int H, int T, int d_v, uint32_t flags, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (flags != 0) return GDR_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || T < 1) return GDR_ERR_INVALID_ARG;
    if ((long long)B * H > (1LL << 28) || (long long)B * H * T > (1LL << 40)) return GDR_ERR_INVALID_ARG;
    if (!gdr::mixer_supported(d_v)) return GDR_ERR_UNSUPPORTED;
    const void* ptrs[] = {o, g, norm_weight, dy, d_o, dg, dnorm_weight, workspace};
    for (const void* ptr : ptrs)
        if (!ptr || !aligned16(ptr)) return GDR_ERR_INVALID_ARG;
    if (workspace_bytes < gdr::mixer_epilogue_bwd_workspace_bytes(d_v)) return GDR_ERR_WORKSPACE;
    gdr_status ds = check_device();
    if (ds != GDR_OK) return ds;
    gdr::EpilogueBwdParams p;
    p.o = o; p.g = g; p.norm_weight = norm_weight; p.dy = dy;
    p.d_o = d_o; p.dg = dg; p.dnorm_weight = dnorm_weight;
    p.part = reinterpret_cast<float*>(workspace);
    p.rows = (long long)B * H * T;
    return from_hip(gdr::launch_mixer_epilogue_bwd(p, d_v, (hipStream_t)stream));
}

}  // extern "C"
