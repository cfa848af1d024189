// Pieces shared by the two-pass chunkwise kernels (forward WY pass, state
// chain, and the backward passes that consume the WY records): chunk size,
// f16 fragment helpers for the 16x16 MFMA tiles, and the per-chunk record.
#pragma once
#include "gdr_device.h"

namespace gdr {

namespace wy {

constexpr int C = 64;
constexpr int NT = 256;
constexpr float kDecayLimit = 10.0f;    // f16 operand range, as in the other kernels
constexpr float kLog2e = 1.4426950408889634f;

// Per-chunk record in the workspace (bytes).  The WY pass writes records with
// non-temporal stores (streamed to memory rather than allocated in L2); that
// takes the chain pass from about 174 to 162 us on the 2 x 16 x 8192 workload.
// Fragment blocks are 64 lanes x 16 bytes; lane l = r + 16 g (r = l & 15,
// g = l >> 4) holds, for a 32-wide K step kk, the K positions 32kk + 4g .. +3
// followed by 32kk + 16 + 4g .. +3.
//   W, Q̃  block (rt, kk): row t = 16 rt + r of W (Q̃), K = channels
//   Kh^T   block (mt, kk): channel 16 mt + r of Kh^T, K = tokens
//   P      block (rt, kk): row 16 rt + r of P, K = tokens
//   Ũ      strip nt, block kk: column 16 nt + r of Ũ, K = tokens
//   G      e^{g_C} per channel (fp32), then an int flag (decay out of range)
template <int DK, int DV>
struct Rec {
    // what the state wave of the chain reads first (W, Kh^T, Ũ, G), then what
    // only the output wave reads (Q̃, P; not written when the backward runs)
    static constexpr size_t W = 0;
    static constexpr size_t K = W + (size_t)C * DK * 2;
    static constexpr size_t U = K + (size_t)DK * C * 2;
    static constexpr size_t G = U + (size_t)C * DV * 2;
    static constexpr size_t Q = G + (((size_t)DK * 4 + 16 + 255) & ~size_t(255));
    static constexpr size_t state_bytes = Q;
    static constexpr size_t P = Q + (size_t)C * DK * 2;
    static constexpr size_t bytes = P + (size_t)C * C * 2;
    static constexpr size_t strip = (size_t)C * 16 * 2;   // Ũ bytes per 16-column strip
    // appended when the backward consumes the records:
    //   KW  block (rt, kk): row t = 16 rt + r of Kh, K = channels
    //   WT  block (mt, kk): channel 16 mt + r of W^T, K = tokens
    //   QT  block (mt, kk): channel 16 mt + r of Q̃^T, K = tokens
    //   PT  block (rt, kk): column 16 rt + r of P, K = tokens (rows of P^T)
    //   TT  block (rt, kk): column 16 rt + r of T, K = tokens (rows of T^T)
    // (PT and TT blocks with kk < rt / 2 are zero and are neither written nor read)
    static constexpr size_t KW = bytes;
    static constexpr size_t WT = KW + (size_t)C * DK * 2;
    static constexpr size_t QT = WT + (size_t)C * DK * 2;
    static constexpr size_t PT = QT + (size_t)C * DK * 2;
    static constexpr size_t TT = PT + (size_t)C * C * 2;
    static constexpr size_t bwd_bytes = TT + (size_t)C * C * 2;
};

// The backward keeps, per chunk, the decayed chunk-start state S' and the
// chunk-end state gradient D as f16 fragments in the layout the state chains
// hold them in: block (nt, kk) = column 16 nt + r of the d_k x d_v matrix, K =
// channels 32 kk + ..  (lane order as above), at byte offset (nt * d_k/32 + kk) * 1024.
template <int DK, int DV>
struct StateFrag {
    static constexpr size_t bytes = (size_t)DK * DV * 2;
    static constexpr size_t block(int nt, int kk) { return ((size_t)nt * (DK / 32) + kk) * 1024; }
};

// a 16-byte record store, streamed to memory (non-temporal)
template <typename V>
__device__ __forceinline__ void st_nt(unsigned char* p, V v) {
    __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}
__device__ __forceinline__ half4 to_h4(floatx4 v) {
    half4 h;
    h[0] = (_Float16)v[0]; h[1] = (_Float16)v[1]; h[2] = (_Float16)v[2]; h[3] = (_Float16)v[3];
    return h;
}
__device__ __forceinline__ half8 cat8(half4 a, half4 b) {
    half8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}
__device__ __forceinline__ half4 lo4(half8 v) {
    half4 r;
    r[0] = v[0]; r[1] = v[1]; r[2] = v[2]; r[3] = v[3];
    return r;
}
__device__ __forceinline__ half4 hi4(half8 v) {
    half4 r;
    r[0] = v[4]; r[1] = v[5]; r[2] = v[6]; r[3] = v[7];
    return r;
}
__device__ __forceinline__ floatx4 f4(half4 h) {
    floatx4 v;
    v[0] = (float)h[0]; v[1] = (float)h[1]; v[2] = (float)h[2]; v[3] = (float)h[3];
    return v;
}
__device__ __forceinline__ floatx4 mfma16(half4 a, half4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma32(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// The 16x16x16 MFMA with the identity as B: a lane holding four consecutive
// columns 4g..4g+3 of row r of a tile gets back four consecutive rows 4g..4g+3 of
// column r, and vice versa (a transpose of the lane layout; exact).
__device__ __forceinline__ half4 ident4(int lane) {
    const int r = lane & 15, g4 = 4 * (lane >> 4);
    half4 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = (_Float16)(g4 + i == r ? 1.f : 0.f);
    return h;
}
__device__ __forceinline__ floatx4 swap16(half4 a, half4 id) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, id, zero4(), 0, 0, 0);
}
__device__ __forceinline__ half4 ld_h4(const _Float16* p) { return *reinterpret_cast<const half4*>(p); }
__device__ __forceinline__ half8 ld_h8(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }
// four halves from a 4-byte aligned address, as two 4-byte reads
__device__ __forceinline__ half4 ld_h4w(const _Float16* p) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 a = *reinterpret_cast<const h2*>(p), b = *reinterpret_cast<const h2*>(p + 2);
    half4 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    return r;
}
// four K values of a column (stride ld)
__device__ __forceinline__ half4 ld_col4(const _Float16* p, int ld) {
    half4 h;
    h[0] = p[0]; h[1] = p[ld]; h[2] = p[2 * ld]; h[3] = p[3 * ld];
    return h;
}

// Packed sequences: the chain that workgroup bid of nblk serves, as sequence *
// H + head, and its strip ng of NG.  The longest sequences go first (order),
// dealt round-robin over the XCDs (workgroup b runs on XCD b % 8), with the NG
// strips of one chain on one XCD so that they share its L2.
__device__ __forceinline__ int packed_chain(const int* order, int H, int NG, int bid, int nblk, int& ng) {
    int rank;
    if (nblk % (8 * NG) == 0) {
        const int pos = bid / 8;
        rank = (pos / NG) * 8 + bid % 8;
        ng = pos % NG;
    } else {
        rank = bid / NG;
        ng = bid % NG;
    }
    return order[rank / H] * H + rank % H;
}

// Packed sequences: the chunks of chain bh (sequence bh / H of head bh % H):
// their count, the sequence's length, its first token in the [H, T] streams
// and its first chunk in the per-head chunk numbering (records, fragments).
struct PackedSpan {
    int NC, len;
    size_t tok0, chunk0;
};
__device__ __forceinline__ PackedSpan packed_span(const int* cu, const int* off, int nseq, int H, int T, int bh) {
    const int s = bh / H, h = bh % H;
    PackedSpan r;
    r.NC = off[s + 1] - off[s];
    r.len = cu[s + 1] - cu[s];
    r.tok0 = (size_t)h * T + (size_t)cu[s];
    r.chunk0 = (size_t)h * off[nseq] + (size_t)off[s];
    return r;
}

}  // namespace wy
}  // namespace gdr
