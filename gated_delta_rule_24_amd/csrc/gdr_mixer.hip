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
#include <type_traits>

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

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// CPL bf16 values (CPL = 4 or 8) packed two per 32-bit word, to fp32
template <int CPL, typename V>
__device__ __forceinline__ void unpack_n(V u, float (&f)[CPL]) {
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}

// channels per lane in the forward convolution tiles (4 measured slightly slower:
// its 8-byte accesses cost more than the shorter halo saves)
constexpr int kFwdCPL = 8;

// conv, SiLU and (L2) the L2 norm of tokens t0 .. t0+TILE-1 of stream bh (head h).
// Each thread takes TPT consecutive tokens of CPL channels: it loads them and the
// kConvTaps-1 tokens before them once (a sliding window in registers), so each
// input row passes the memory pipeline (TPT + 3) / TPT times, not kConvTaps times.
template <int D, bool L2, int CPL = kFwdCPL>
__device__ __forceinline__ void conv_tile(const uint16_t* src, const float* taps, uint16_t* dst, int h, size_t bh,
                                          int T, int t0) {
    static_assert(CPL == 4 || CPL == 8, "channels per lane");
    using Raw = typename std::conditional<CPL == 8, u32x4, u32x2>::type;
    constexpr int LPT = D / CPL;                // lanes per token
    constexpr int TPT = TILE * LPT / NT;        // consecutive tokens per thread
    constexpr int NR = TPT + kConvTaps - 1;     // rows a thread reads
    static_assert(TPT * NT == TILE * LPT && 64 % LPT == 0, "token mapping");
    const int tid = threadIdx.x, co = tid % LPT, tl = tid / LPT;
    floatx4 w[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        w[c] = *reinterpret_cast<const floatx4*>(taps + ((size_t)h * D + CPL * co + c) * kConvTaps);
    const uint16_t* s = src + bh * (size_t)T * D + CPL * co;
    uint16_t* d = dst + bh * (size_t)T * D + CPL * co;
    const int ta = t0 + tl * TPT;               // this thread's first token
    // rows ta-3 .. ta+TPT-1; rows before the sequence or past its end read as zero
    Raw raw[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int t = ta - (kConvTaps - 1) + r;
        const bool in = t >= 0 && t < T;
        raw[r] = *reinterpret_cast<const Raw*>(s + (size_t)(in ? t : 0) * D);
        if (!in) raw[r] = Raw{};
    }
    float acc[TPT][CPL];
#pragma unroll
    for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[i][c] = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        float x[CPL];
        unpack_n<CPL>(raw[r], x);
        // row r is token ta + r - 3: it is tap j of output i = r - 3 + j
#pragma unroll
        for (int j = 0; j < kConvTaps; ++j) {
            const int i = r - (kConvTaps - 1) + j;
            if (i >= 0 && i < TPT) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[i][c] += w[c][j] * x[c];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[i][c] = silu(acc[i][c]);
        if constexpr (L2) {
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) ss += acc[i][c] * acc[i][c];
#pragma unroll
            for (int off = 1; off < LPT; off *= 2) ss += __shfl_xor(ss, off, 64);
            const float sc = rsqrtf(ss + kEps);
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[i][c] *= sc;
        }
        if (ta + i < T) {
            Raw o;
#pragma unroll
            for (int c = 0; c < CPL / 2; ++c)
                o[c] = (uint32_t)f32_to_bf16(acc[i][2 * c]) | ((uint32_t)f32_to_bf16(acc[i][2 * c + 1]) << 16);
            *reinterpret_cast<Raw*>(d + (size_t)(ta + i) * D) = o;
        }
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

// ---------------------------------------------------------------------------
// Backward.  Prologue streams (q, k: conv -> SiLU -> L2 norm; v: conv -> SiLU),
// given dy = dL/d(output) in fp32, per token with s = SiLU(c), c = conv(x):
//   L2:  r = (sum s^2 + eps)^(-1/2),  ds = r dy - r^3 (s . dy) s;   else ds = dy
//   dc = ds * SiLU'(c),  SiLU'(c) = sigmoid(c) (1 + c (1 - sigmoid(c)))
//   dx_t = sum_j w_j dc_{t+j}        (the transposed, anti-causal convolution)
//   dw_j = sum_t dc_t x_{t-j}        (over all tokens of all sequences of the head)
// Each thread takes BTPT consecutive tokens of CPL channels and recomputes c for
// them and the 3 tokens after them (whose dc its dx needs).  dw is summed per
// workgroup in LDS, written as one partial per (sequence, tile), and the
// partials are added in a fixed order by reduce_taps (deterministic).
constexpr int BTILE = 64;     // tokens per prologue-backward workgroup
// channels per lane: 4 rather than the forward's 8 halves the per-token
// register arrays (3 waves per SIMD instead of 2 at d = 128) and, with twice the
// lanes per token, gives each thread twice the tokens, so fewer halo tokens are
// recomputed (11 per 8 tokens instead of 7 per 4)
constexpr int kBwdCPL = 4;

__device__ __forceinline__ float silu_grad(float c) {
    const float sg = gate_sigmoid(c);
    return sg * (1.f + c * (1.f - sg));
}

template <int D, bool L2, int CPL = kBwdCPL>
__device__ __forceinline__ void stream_bwd_tile(const uint16_t* src, const float* taps, const float* dy, float* dx,
                                                float* part, int h, size_t bh, int T, int t0) {
    static_assert(CPL == 4 || CPL == 8, "channels per lane");
    using Raw = typename std::conditional<CPL == 8, u32x4, u32x2>::type;
    constexpr int LPT = D / CPL, BTPT = BTILE * LPT / NT, NQ = CPL / 4;
    constexpr int NU = BTPT + kConvTaps - 1;        // tokens whose dc this thread forms
    constexpr int NR = NU + kConvTaps - 1;          // input rows it reads
    static_assert(BTPT * NT == BTILE * LPT && 64 % LPT == 0, "token mapping");
    __shared__ floatx4 sW[NT / 64][D];              // per wave: dw partial per channel
    const int tid = threadIdx.x, co = tid % LPT, tl = tid / LPT;
    floatx4 w[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        w[c] = *reinterpret_cast<const floatx4*>(taps + ((size_t)h * D + CPL * co + c) * kConvTaps);
    const size_t base = bh * (size_t)T * D + CPL * co;
    const int ta = t0 + tl * BTPT;
    // input rows ta-3 .. ta+NU-1 (zero outside the sequence)
    Raw raw[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int t = ta - (kConvTaps - 1) + r;
        const bool in = t >= 0 && t < T;
        raw[r] = *reinterpret_cast<const Raw*>(src + base + (size_t)(in ? t : 0) * D);
        if (!in) raw[r] = Raw{};
    }
    // gradients of this thread's tokens (loaded up front), zero past the end
    floatx4 gy[NU][NQ];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int t = ta + u;
        const bool in = t < T;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            gy[u][q] = *reinterpret_cast<const floatx4*>(dy + base + (size_t)(in ? t : 0) * D + 4 * q);
            if (!in) gy[u][q] = zero4();
        }
    }
    // dc of tokens ta .. ta+NU-1, one token at a time, each added at once into
    // dx of the tokens it reaches (ta+u-j for tap j) and, for this thread's own
    // tokens, into dw
    float dxa[BTPT][CPL];
#pragma unroll
    for (int i2 = 0; i2 < BTPT; ++i2)
#pragma unroll
        for (int c = 0; c < CPL; ++c) dxa[i2][c] = 0.f;
    floatx4 dw[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) dw[c] = zero4();
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        float g[CPL], cv[CPL], sl[CPL], dcu[CPL];
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) g[4 * q + c] = gy[u][q][c];
#pragma unroll
        for (int c = 0; c < CPL; ++c) cv[c] = 0.f;
#pragma unroll
        for (int j = 0; j < kConvTaps; ++j) {
            float x[CPL];
            unpack_n<CPL>(raw[u + kConvTaps - 1 - j], x);
#pragma unroll
            for (int c = 0; c < CPL; ++c) cv[c] += w[c][j] * x[c];
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) sl[c] = silu(cv[c]);
        if constexpr (L2) {
            float ss = 0.f, sd = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) { ss += sl[c] * sl[c]; sd += sl[c] * g[c]; }
#pragma unroll
            for (int off = 1; off < LPT; off *= 2) {
                ss += __shfl_xor(ss, off, 64);
                sd += __shfl_xor(sd, off, 64);
            }
            const float r = rsqrtf(ss + kEps), r3sd = r * r * r * sd;
#pragma unroll
            for (int c = 0; c < CPL; ++c) g[c] = r * g[c] - r3sd * sl[c];
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) dcu[c] = g[c] * silu_grad(cv[c]);
#pragma unroll
        for (int j = 0; j < kConvTaps; ++j) {
            const int i2 = u - j;                   // dx of token ta+i2 takes w_j dc_{ta+u}
            if (i2 >= 0 && i2 < BTPT) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) dxa[i2][c] += w[c][j] * dcu[c];
            }
        }
        if (u < BTPT && ta + u < T) {
#pragma unroll
            for (int j = 0; j < kConvTaps; ++j) {
                float x[CPL];
                unpack_n<CPL>(raw[u + kConvTaps - 1 - j], x);
#pragma unroll
                for (int c = 0; c < CPL; ++c) dw[c][j] += dcu[c] * x[c];
            }
        }
    }
#pragma unroll
    for (int i2 = 0; i2 < BTPT; ++i2) {
        const int t = ta + i2;
        if (t < T) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                *reinterpret_cast<floatx4*>(dx + base + (size_t)t * D + 4 * q) =
                    floatx4{dxa[i2][4 * q], dxa[i2][4 * q + 1], dxa[i2][4 * q + 2], dxa[i2][4 * q + 3]};
        }
    }
    // over the token groups of the wave (lanes LPT apart hold the same channels),
    // then over the waves in LDS
#pragma unroll
    for (int off = LPT; off < 64; off *= 2)
#pragma unroll
        for (int i = 0; i < CPL; ++i)
#pragma unroll
            for (int j = 0; j < kConvTaps; ++j) dw[i][j] += __shfl_xor(dw[i][j], off, 64);
    if ((tid & 63) < LPT) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) sW[tid >> 6][CPL * co + i] = dw[i];
    }
    __syncthreads();
    for (int c = tid; c < D; c += NT) {
        floatx4 acc = zero4();
#pragma unroll
        for (int w2 = 0; w2 < NT / 64; ++w2) acc += sW[w2][c];
        *reinterpret_cast<floatx4*>(part + (size_t)c * kConvTaps) = acc;
    }
}

// grid.y 0 = q, 1 = k, 2 = v; part: [3][BH][ntile][D][kConvTaps] partial tap gradients
template <int DK, int DV>
__global__ __launch_bounds__(NT) void prologue_bwd_kernel(MixerBwdParams p) {
    const int ntile = (p.T + BTILE - 1) / BTILE;
    const size_t bh = blockIdx.x / ntile;
    const int tile = (int)(blockIdx.x % ntile), t0 = tile * BTILE;
    const int h = (int)(bh % p.H);
    const size_t slot = bh * ntile + tile;
    const size_t per_k = (size_t)p.BH * ntile * DK * kConvTaps;
    switch (blockIdx.y) {
        case 0:
            stream_bwd_tile<DK, true>(reinterpret_cast<const uint16_t*>(p.q_pre), p.conv_q, p.dq, p.dq_pre,
                                      p.part + slot * DK * kConvTaps, h, bh, p.T, t0);
            break;
        case 1:
            stream_bwd_tile<DK, true>(reinterpret_cast<const uint16_t*>(p.k_pre), p.conv_k, p.dk, p.dk_pre,
                                      p.part + per_k + slot * DK * kConvTaps, h, bh, p.T, t0);
            break;
        default:
            stream_bwd_tile<DV, false>(reinterpret_cast<const uint16_t*>(p.v_pre), p.conv_v, p.dv, p.dv_pre,
                                       p.part + 2 * per_k + slot * DV * kConvTaps, h, bh, p.T, t0);
            break;
    }
}

// A workgroup's values summed in a fixed order: thread-strided partial sums,
// then a fixed tree in LDS (so the result does not depend on timing).
__device__ __forceinline__ floatx4 block_sum4(floatx4 v) {
    __shared__ floatx4 red[NT];
    const int tid = threadIdx.x;
    red[tid] = v;
    __syncthreads();
#pragma unroll
    for (int s = NT / 2; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    return red[0];
}

// dconv[h][c][0..3] = sum over b and tiles of the partials: one workgroup per
// (stream, head, channel); blockIdx.y = stream
template <int DK, int DV>
__global__ __launch_bounds__(NT) void reduce_taps_kernel(MixerBwdParams p) {
    const int ntile = (p.T + BTILE - 1) / BTILE;
    const int B = p.BH / p.H;
    const size_t per_k = (size_t)p.BH * ntile * DK * kConvTaps;
    const int which = blockIdx.y;
    const int D = which == 2 ? DV : DK;
    const int h = (int)blockIdx.x / D, c = (int)blockIdx.x % D;
    if (h >= p.H) return;
    const float* part = p.part + which * per_k;
    float* out = which == 0 ? p.dconv_q : which == 1 ? p.dconv_k : p.dconv_v;
    const int n = B * ntile;                       // partials of this head
    floatx4 acc = zero4();
    for (int i = threadIdx.x; i < n; i += NT) {
        const int b = i / ntile, tile = i % ntile;
        acc += *reinterpret_cast<const floatx4*>(
            part + ((((size_t)(b * p.H + h)) * ntile + tile) * D + c) * kConvTaps);
    }
    acc = block_sum4(acc);
    if (threadIdx.x == 0) *reinterpret_cast<floatx4*>(out + ((size_t)h * D + c) * kConvTaps) = acc;
}

// Epilogue backward, per row with r = (mean o^2 + eps)^(-1/2), z = o r:
//   dz = dy * w * SiLU(g),  d_o = r dz - (r^3 / D) (o . dz) o,
//   dg = dy * z * w * SiLU'(g),  dw = sum over rows of dy * z * SiLU(g).
// One workgroup per block of rows (grid-strided); dw is summed per workgroup
// and the per-workgroup partials are added in a fixed order by reduce_norm.
template <int DV>
__global__ __launch_bounds__(NT) void epilogue_bwd_kernel(EpilogueBwdParams p) {
    constexpr int LPT = DV / 8, RPP = NT / LPT;
    __shared__ float sW[RPP][DV];
    const int tid = threadIdx.x, co = tid % LPT, rl = tid / LPT;
    float wn[8], dwn[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        wn[c] = p.norm_weight[8 * co + c];
        dwn[c] = 0.f;
    }
    for (size_t r0 = (size_t)blockIdx.x * RPP; r0 < (size_t)p.rows; r0 += (size_t)gridDim.x * RPP) {
        const size_t r = r0 + rl;
        const bool ok = r < (size_t)p.rows;
        const size_t at = (ok ? r : 0) * DV + 8 * co;
        float o[8], g[8], dy[8];
        {
            const floatx4 o0 = *reinterpret_cast<const floatx4*>(p.o + at);
            const floatx4 o1 = *reinterpret_cast<const floatx4*>(p.o + at + 4);
            const floatx4 y0 = *reinterpret_cast<const floatx4*>(p.dy + at);
            const floatx4 y1 = *reinterpret_cast<const floatx4*>(p.dy + at + 4);
            unpack8(*reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.g) + at), g);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                o[c] = ok ? o0[c] : 0.f;
                o[c + 4] = ok ? o1[c] : 0.f;
                dy[c] = ok ? y0[c] : 0.f;
                dy[c + 4] = ok ? y1[c] : 0.f;
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) ss += o[c] * o[c];
#pragma unroll
        for (int off = 1; off < LPT; off *= 2) ss += __shfl_xor(ss, off, 64);
        const float rr = rsqrtf(ss * (1.f / DV) + kEps);
        float dz[8], od = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float sg = silu(g[c]);
            dz[c] = dy[c] * wn[c] * sg;
            od += o[c] * dz[c];
            dwn[c] += dy[c] * o[c] * rr * sg;
        }
#pragma unroll
        for (int off = 1; off < LPT; off *= 2) od += __shfl_xor(od, off, 64);
        const float k3 = rr * rr * rr * od * (1.f / DV);
        float dov[8], dgv[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            dov[c] = rr * dz[c] - k3 * o[c];
            dgv[c] = dy[c] * o[c] * rr * wn[c] * silu_grad(g[c]);
        }
        if (ok) {
            *reinterpret_cast<floatx4*>(p.d_o + at) = floatx4{dov[0], dov[1], dov[2], dov[3]};
            *reinterpret_cast<floatx4*>(p.d_o + at + 4) = floatx4{dov[4], dov[5], dov[6], dov[7]};
            *reinterpret_cast<floatx4*>(p.dg + at) = floatx4{dgv[0], dgv[1], dgv[2], dgv[3]};
            *reinterpret_cast<floatx4*>(p.dg + at + 4) = floatx4{dgv[4], dgv[5], dgv[6], dgv[7]};
        }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) sW[rl][8 * co + c] = dwn[c];
    __syncthreads();
    for (int c = tid; c < DV; c += NT) {
        float acc = 0.f;
#pragma unroll 8
        for (int q = 0; q < RPP; ++q) acc += sW[q][c];
        p.part[(size_t)blockIdx.x * DV + c] = acc;
    }
}

// dnorm_weight[c]: one workgroup per channel over the per-workgroup partials
template <int DV>
__global__ __launch_bounds__(NT) void reduce_norm_kernel(EpilogueBwdParams p, int nblk) {
    const int c = blockIdx.x;
    floatx4 acc = zero4();
    for (int b = threadIdx.x; b < nblk; b += NT) acc[0] += p.part[(size_t)b * DV + c];
    acc = block_sum4(acc);
    if (threadIdx.x == 0) p.dnorm_weight[c] = acc[0];
}

}  // namespace mixer

bool mixer_supported(int d) { return d == 64 || d == 128; }

size_t mixer_prologue_bwd_workspace_bytes(int BH, int T, int dk, int dv) {
    const size_t ntile = (size_t)(T + mixer::BTILE - 1) / mixer::BTILE;
    // q and k partials take dk channels, v's dv; laid out as three dk-sized blocks
    const size_t d = dk > dv ? dk : dv;
    return 3 * (size_t)BH * ntile * d * kConvTaps * sizeof(float);
}

size_t mixer_epilogue_bwd_workspace_bytes(int dv) {
    return (size_t)kEpilogueBwdBlocks * dv * sizeof(float);
}

hipError_t launch_mixer_prologue_bwd(const MixerBwdParams& p, int dk, int dv, hipStream_t st) {
    if (p.T == 0) return hipErrorInvalidValue;
    const int ntile = (p.T + mixer::BTILE - 1) / mixer::BTILE;
    dim3 grid((unsigned)((size_t)p.BH * ntile), 3), block(mixer::NT);
    dim3 rgrid((unsigned)(p.H * (dk > dv ? dk : dv)), 3);
    if (dk == 128 && dv == 128) {
        hipLaunchKernelGGL((mixer::prologue_bwd_kernel<128, 128>), grid, block, 0, st, p);
        hipLaunchKernelGGL((mixer::reduce_taps_kernel<128, 128>), rgrid, block, 0, st, p);
    } else if (dk == 64 && dv == 64) {
        hipLaunchKernelGGL((mixer::prologue_bwd_kernel<64, 64>), grid, block, 0, st, p);
        hipLaunchKernelGGL((mixer::reduce_taps_kernel<64, 64>), rgrid, block, 0, st, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mixer_epilogue_bwd(const EpilogueBwdParams& p, int dv, hipStream_t st) {
    if (p.rows == 0) return hipErrorInvalidValue;
    dim3 grid(kEpilogueBwdBlocks), block(mixer::NT);
    if (dv == 128) {
        hipLaunchKernelGGL((mixer::epilogue_bwd_kernel<128>), grid, block, 0, st, p);
        hipLaunchKernelGGL((mixer::reduce_norm_kernel<128>), dim3(128), block, 0, st, p, kEpilogueBwdBlocks);
    } else if (dv == 64) {
        hipLaunchKernelGGL((mixer::epilogue_bwd_kernel<64>), grid, block, 0, st, p);
        hipLaunchKernelGGL((mixer::reduce_norm_kernel<64>), dim3(64), block, 0, st, p, kEpilogueBwdBlocks);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

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
