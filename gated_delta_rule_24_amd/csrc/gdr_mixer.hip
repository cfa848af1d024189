// Token-mixer prologue and epilogue around the gated delta rule: the
// element-wise and short-window parts of the block ("Gated DeltaNet study
// notes" §2 token mixer block design; "Gated DeltaNet-2 Review" §4-3
// engineering notes), between the caller's linear projections and the
// recurrence, and between the recurrence and the output projection.
//
// Prologue, per (sequence, head), from the projections' outputs:
//   q = L2norm(SiLU(conv(q_pre))),  k = L2norm(SiLU(conv(k_pre))),
//   v = SiLU(conv(v_pre)),
//   log_alpha = log(sigmoid(a_pre))   (fp32 throughout),
//   b = sigmoid(b_pre),  w = sigmoid(w_pre).
// conv is the depthwise causal convolution with kConvTaps taps per channel,
// tap j weighting the token j steps back, zeros before the sequence start;
// L2norm(x) = x / sqrt(sum x^2 + eps) over the head's channels.
// Epilogue, per (token, head):
//   y = o / sqrt(mean(o^2) + eps) * norm_weight * SiLU(g).
//
// Both are one pass over HBM with all arithmetic in fp32: the prologue reads
// each projection output once (the convolution's three-token look-back comes
// from the cache) and writes the recurrence's inputs once; the epilogue reads
// o and the gate once and writes y once.  A token's channels are spread over
// D/8 lanes of one wave (8 channels, one 16-byte access per lane), so the
// per-token norms are lane shuffles.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {
namespace mixer {

constexpr int NT = 256;       // threads per workgroup
constexpr int TILE = 128;     // tokens per prologue workgroup
constexpr float kEps = 1e-6f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sigmoid(float x) { return gate_sigmoid(x); }
__device__ __forceinline__ float silu(float x) { return x * gate_sigmoid(x); }
__device__ __forceinline__ float log_sigmoid(float z) { return gate_log_sigmoid(z); }

__device__ __forceinline__ void unpack8(u32x4 u, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        u[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
    return u;
}

// conv, SiLU and (L2) the L2 norm of tokens t0 .. t0+TILE-1 of stream bh (head h).
// Each thread takes TPT consecutive tokens of 8 channels: it loads them and the
// kConvTaps-1 tokens before them once (a sliding window in registers), so each
// input row passes the memory pipeline (TPT + 3) / TPT times, not kConvTaps times.
template <int D, bool L2>
__device__ __forceinline__ void conv_tile(const uint16_t* src, const float* taps, uint16_t* dst, int h, size_t bh,
                                          int T, int t0) {
    constexpr int LPT = D / 8;                  // lanes per token
    constexpr int TPT = TILE * LPT / NT;        // consecutive tokens per thread
    constexpr int NR = TPT + kConvTaps - 1;     // rows a thread reads
    static_assert(TPT * NT == TILE * LPT && 64 % LPT == 0, "token mapping");
    const int tid = threadIdx.x, co = tid % LPT, tl = tid / LPT;
    floatx4 w[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
        w[c] = *reinterpret_cast<const floatx4*>(taps + ((size_t)h * D + 8 * co + c) * kConvTaps);
    const uint16_t* s = src + bh * (size_t)T * D + 8 * co;
    uint16_t* d = dst + bh * (size_t)T * D + 8 * co;
    const int ta = t0 + tl * TPT;               // this thread's first token
    // rows ta-3 .. ta+TPT-1; rows before the sequence or past its end read as zero
    u32x4 raw[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int t = ta - (kConvTaps - 1) + r;
        const bool in = t >= 0 && t < T;
        raw[r] = *reinterpret_cast<const u32x4*>(s + (size_t)(in ? t : 0) * D);
        if (!in) raw[r] = u32x4{0u, 0u, 0u, 0u};
    }
    float acc[TPT][8];
#pragma unroll
    for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        float x[8];
        unpack8(raw[r], x);
        // row r is token ta + r - 3: it is tap j of output i = r - 3 + j
#pragma unroll
        for (int j = 0; j < kConvTaps; ++j) {
            const int i = r - (kConvTaps - 1) + j;
            if (i >= 0 && i < TPT) {
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[i][c] += w[c][j] * x[c];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = silu(acc[i][c]);
        if constexpr (L2) {
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) ss += acc[i][c] * acc[i][c];
#pragma unroll
            for (int off = 1; off < LPT; off *= 2) ss += __shfl_xor(ss, off, 64);
            const float sc = rsqrtf(ss + kEps);
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[i][c] *= sc;
        }
        if (ta + i < T) *reinterpret_cast<u32x4*>(d + (size_t)(ta + i) * D) = pack8(acc[i]);
    }
}

// A gate stream over one tile: n tokens of CH values each (CH = 1 in scalar
// mode) from element e0 on, through sigmoid (bf16 in and out) or log-sigmoid
// (fp32).  Every 16-byte load of the tile is issued before any value is used.
template <int CH, bool LOG>
__device__ __forceinline__ void gate_tile(const void* src, void* dst, size_t e0, int n) {
    constexpr int VEC = LOG ? 4 : 8;                    // values per 16-byte access
    const int tid = threadIdx.x, count = n * CH;
    if constexpr (CH % VEC == 0) {
        constexpr int PER = (TILE * CH / VEC + NT - 1) / NT;
        u32x4 x[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = VEC * (tid + m * NT);
            const size_t off = (e0 + (e < count ? e : 0)) * (LOG ? 4 : 2);
            x[m] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const unsigned char*>(src) + off);
        }
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = VEC * (tid + m * NT);
            if (e >= count) continue;
            u32x4 y;
            if constexpr (LOG) {
#pragma unroll
                for (int c = 0; c < 4; ++c) y[c] = __float_as_uint(log_sigmoid(__uint_as_float(x[m][c])));
            } else {
                float f[8];
                unpack8(x[m], f);
#pragma unroll
                for (int c = 0; c < 8; ++c) f[c] = sigmoid(f[c]);
                y = pack8(f);
            }
            *reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(dst) + (e0 + e) * (LOG ? 4 : 2)) = y;
        }
    } else {
        // one value per token (scalar gates): no alignment to rely on
        for (int e = tid; e < count; e += NT) {
            if constexpr (LOG) {
                reinterpret_cast<float*>(dst)[e0 + e] = log_sigmoid(reinterpret_cast<const float*>(src)[e0 + e]);
            } else {
                const uint16_t u = reinterpret_cast<const uint16_t*>(src)[e0 + e];
                reinterpret_cast<uint16_t*>(dst)[e0 + e] = f32_to_bf16(sigmoid(bf16_to_f32(u)));
            }
        }
    }
}

// One workgroup per (stream bh, tile of TILE tokens) and per part: blockIdx.y
// 0 = q, 1 = k, 2 = v, 3 = log alpha, 4 = b, 5 = w.
template <int DK, int DV>
__global__ __launch_bounds__(NT) void prologue_kernel(MixerParams p) {
    const int ntile = (p.T + TILE - 1) / TILE;
    const size_t bh = blockIdx.x / ntile;
    const int t0 = (int)(blockIdx.x % ntile) * TILE;
    const int h = (int)(bh % p.H);
    const int n = min(TILE, p.T - t0);
    const size_t tok = bh * (size_t)p.T + t0;
    switch (blockIdx.y) {
        case 0:
            conv_tile<DK, true>(reinterpret_cast<const uint16_t*>(p.q_pre), p.conv_q,
                                reinterpret_cast<uint16_t*>(p.q), h, bh, p.T, t0);
            break;
        case 1:
            conv_tile<DK, true>(reinterpret_cast<const uint16_t*>(p.k_pre), p.conv_k,
                                reinterpret_cast<uint16_t*>(p.k), h, bh, p.T, t0);
            break;
        case 2:
            conv_tile<DV, false>(reinterpret_cast<const uint16_t*>(p.v_pre), p.conv_v,
                                 reinterpret_cast<uint16_t*>(p.v), h, bh, p.T, t0);
            break;
        case 3:
            if (p.flags & GDR_ALPHA_SCALAR) gate_tile<1, true>(p.a_pre, p.la, tok, n);
            else gate_tile<DK, true>(p.a_pre, p.la, tok * DK, n);
            break;
        case 4:
            if (p.flags & GDR_B_SCALAR) gate_tile<1, false>(p.b_pre, p.b, tok, n);
            else gate_tile<DK, false>(p.b_pre, p.b, tok * DK, n);
            break;
        default:
            if (p.flags & GDR_W_SCALAR) gate_tile<1, false>(p.w_pre, p.w, tok, n);
            else gate_tile<DV, false>(p.w_pre, p.w, tok * DV, n);
            break;
    }
}

// One row (token, head) per D/8 lanes; rows strided over the grid.
template <int DV>
__global__ __launch_bounds__(NT) void epilogue_kernel(EpilogueParams p) {
    constexpr int LPT = DV / 8, RPP = NT / LPT;
    const int tid = threadIdx.x, co = tid % LPT, rl = tid / LPT;
    float wn[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) wn[c] = p.norm_weight[8 * co + c];
    for (size_t r0 = (size_t)blockIdx.x * RPP; r0 < (size_t)p.rows; r0 += (size_t)gridDim.x * RPP) {
        const size_t r = r0 + rl;
        const bool ok = r < (size_t)p.rows;
        float o[8], g[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = g[c] = 0.f;
        if (ok) {
            const floatx4 o0 = *reinterpret_cast<const floatx4*>(p.o + r * DV + 8 * co);
            const floatx4 o1 = *reinterpret_cast<const floatx4*>(p.o + r * DV + 8 * co + 4);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                o[c] = o0[c];
                o[c + 4] = o1[c];
            }
            unpack8(*reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.g) + r * DV + 8 * co), g);
        }
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) ss += o[c] * o[c];
#pragma unroll
        for (int off = 1; off < LPT; off *= 2) ss += __shfl_xor(ss, off, 64);
        const float sc = rsqrtf(ss * (1.f / DV) + kEps);
        float y[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) y[c] = o[c] * sc * wn[c] * silu(g[c]);
        if (ok) *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.y) + r * DV + 8 * co) = pack8(y);
    }
}

}  // namespace mixer

bool mixer_supported(int d) { return d == 64 || d == 128; }

hipError_t launch_mixer_prologue(const MixerParams& p, int dk, int dv, hipStream_t st) {
    const int ntile = (p.T + mixer::TILE - 1) / mixer::TILE;
    if (p.T == 0) return hipSuccess;
    // with GDR_GATE_LOGITS the gates are left to the recurrence: q, k, v only
    dim3 grid((unsigned)((size_t)p.BH * ntile), (p.flags & GDR_GATE_LOGITS) ? 3 : 6), block(mixer::NT);
    if (dk == 128 && dv == 128) hipLaunchKernelGGL((mixer::prologue_kernel<128, 128>), grid, block, 0, st, p);
    else if (dk == 64 && dv == 64) hipLaunchKernelGGL((mixer::prologue_kernel<64, 64>), grid, block, 0, st, p);
    else if (dk == 128 && dv == 64) hipLaunchKernelGGL((mixer::prologue_kernel<128, 64>), grid, block, 0, st, p);
    else if (dk == 64 && dv == 128) hipLaunchKernelGGL((mixer::prologue_kernel<64, 128>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_mixer_epilogue(const EpilogueParams& p, int dv, hipStream_t st) {
    if (p.rows == 0) return hipSuccess;
    const long long rpp = mixer::NT / (dv / 8);
    const long long blocks = (p.rows + rpp - 1) / rpp;
    dim3 grid((unsigned)(blocks < 8192 ? blocks : 8192)), block(mixer::NT);
    if (dv == 128) hipLaunchKernelGGL((mixer::epilogue_kernel<128>), grid, block, 0, st, p);
    else if (dv == 64) hipLaunchKernelGGL((mixer::epilogue_kernel<64>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdr
