// Device-side helpers shared by the libgdr kernels (gfx950 / CDNA4 only).
//
// MFMA conventions used throughout (wave64):
//   every product is written  acc(16x16) += X[16 x K] · Y[16 x K]^T
//   with both operands stored "K-contiguous" in LDS (row r of X / Y holds
//   its K values contiguously).  Lane l supplies row (l & 15) of X and of Y
//   and a contiguous run of K values selected by (l >> 4); any fixed
//   assignment of K positions to lanes is valid as long as X and Y use the
//   same one, because K is summed over.
//   The accumulator (D) layout of the 16x16 fp32 result is:
//   acc[i] holds element (m = 4*(l >> 4) + i, n = l & 15).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
    return __uint_as_float(((uint32_t)u) << 16);
}

// round-to-nearest-even fp32 -> bf16 bits (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Gates given as logits (GDR_GATE_LOGITS and the token-mixer kernels): sigmoid
// and log-sigmoid in fp32.  The hardware reciprocal (1 ulp) replaces IEEE
// division, which costs about ten instructions per value.
__device__ __forceinline__ float gate_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float gate_sigmoid(float x) { return gate_rcp(1.f + __expf(-x)); }
// log(1 + e) for e in [0, 1] with relative accuracy for tiny e: with u = 1 + e
// rounded, log(u) * e / (u - 1) cancels the rounding of u (Goldberg, "What
// every computer scientist should know about floating-point arithmetic",
// 1991, Theorem 4); u == 1 means e is below half an ulp of 1, where log1p(e) = e.
__device__ __forceinline__ float gate_log1p_small(float e) {
    const float u = 1.f + e;
    return u == 1.f ? e : __logf(u) * e * gate_rcp(u - 1.f);
}
// log(sigmoid(z)) = min(z, 0) - log(1 + exp(-|z|)): no overflow for either sign,
// the tiny values for large z keep their relative accuracy, and z = +inf gives 0
__device__ __forceinline__ float gate_log_sigmoid(float z) {
    return fminf(z, 0.f) - gate_log1p_small(__expf(-fabsf(z)));
}

// Load 4 consecutive activations starting at element index `idx`.
template <bool F32>
__device__ __forceinline__ floatx4 load_act4(const void* base, size_t idx) {
    if constexpr (F32) {
        return *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(base) + idx);
    } else {
        uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + idx);
        floatx4 r;
        r[0] = __uint_as_float(u.x << 16);
        r[1] = __uint_as_float(u.x & 0xffff0000u);
        r[2] = __uint_as_float(u.y << 16);
        r[3] = __uint_as_float(u.y & 0xffff0000u);
        return r;
    }
}

template <bool F32>
__device__ __forceinline__ float load_act1(const void* base, size_t idx) {
    if constexpr (F32) return reinterpret_cast<const float*>(base)[idx];
    else return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
}

// Raw (unconverted) 4-element activation load, for register prefetching.
template <bool F32> struct Raw4;
template <> struct Raw4<false> { uint2 u; };
template <> struct Raw4<true> { floatx4 f; };

template <bool F32>
__device__ __forceinline__ Raw4<F32> load_raw4(const void* base, size_t idx) {
    Raw4<F32> r;
    if constexpr (F32) r.f = *reinterpret_cast<const floatx4*>(reinterpret_cast<const float*>(base) + idx);
    else r.u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + idx);
    return r;
}

template <bool F32>
__device__ __forceinline__ floatx4 cvt_raw4(const Raw4<F32>& r) {
    if constexpr (F32) {
        return r.f;
    } else {
        floatx4 f;
        f[0] = __uint_as_float(r.u.x << 16);
        f[1] = __uint_as_float(r.u.x & 0xffff0000u);
        f[2] = __uint_as_float(r.u.y << 16);
        f[3] = __uint_as_float(r.u.y & 0xffff0000u);
        return f;
    }
}

// ---------------------------------------------------------------------------
// MFMA tile products over LDS operands.
// ---------------------------------------------------------------------------

// acc += X[0:16, 0:K] · Y[0:16, 0:K]^T, f16 operands (K multiple of 16).
__device__ __forceinline__ void mma_f16(floatx4& acc, const _Float16* X, int ldx,
                                        const _Float16* Y, int ldy, int K, int lane) {
    const int row = lane & 15, kg = lane >> 4;
    const _Float16* xp = X + row * ldx;
    const _Float16* yp = Y + row * ldy;
    int k0 = 0;
    for (; k0 + 32 <= K; k0 += 32) {
        half8 a = *reinterpret_cast<const half8*>(xp + k0 + 8 * kg);
        half8 b = *reinterpret_cast<const half8*>(yp + k0 + 8 * kg);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
    if (k0 < K) {  // K % 32 == 16
        half4 a = *reinterpret_cast<const half4*>(xp + k0 + 4 * kg);
        half4 b = *reinterpret_cast<const half4*>(yp + k0 + 4 * kg);
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, acc, 0, 0, 0);
    }
}

// acc += X · Y^T with X stored fp32 (converted to f16 on load), Y f16.
__device__ __forceinline__ void mma_f16_xf32(floatx4& acc, const float* X, int ldx,
                                             const _Float16* Y, int ldy, int K, int lane) {
    const int row = lane & 15, kg = lane >> 4;
    const float* xp = X + row * ldx;
    const _Float16* yp = Y + row * ldy;
    int k0 = 0;
    for (; k0 + 32 <= K; k0 += 32) {
        floatx4 x0 = *reinterpret_cast<const floatx4*>(xp + k0 + 8 * kg);
        floatx4 x1 = *reinterpret_cast<const floatx4*>(xp + k0 + 8 * kg + 4);
        half8 a;
        a[0] = (_Float16)x0[0]; a[1] = (_Float16)x0[1]; a[2] = (_Float16)x0[2]; a[3] = (_Float16)x0[3];
        a[4] = (_Float16)x1[0]; a[5] = (_Float16)x1[1]; a[6] = (_Float16)x1[2]; a[7] = (_Float16)x1[3];
        half8 b = *reinterpret_cast<const half8*>(yp + k0 + 8 * kg);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
    if (k0 < K) {
        floatx4 x0 = *reinterpret_cast<const floatx4*>(xp + k0 + 4 * kg);
        half4 a;
        a[0] = (_Float16)x0[0]; a[1] = (_Float16)x0[1]; a[2] = (_Float16)x0[2]; a[3] = (_Float16)x0[3];
        half4 b = *reinterpret_cast<const half4*>(yp + k0 + 4 * kg);
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, acc, 0, 0, 0);
    }
}

// acc += X · Y^T, fp32 operands on fp32 MFMA (K multiple of 16).  For each
// 16-wide K block, lane group kg holds K positions 4*kg .. 4*kg+3 and the
// s-th of the four MFMAs consumes position 4*kg + s.
__device__ __forceinline__ void mma_f32(floatx4& acc, const float* X, int ldx,
                                        const float* Y, int ldy, int K, int lane) {
    const int row = lane & 15, kg = lane >> 4;
    const float* xp = X + row * ldx;
    const float* yp = Y + row * ldy;
    for (int k0 = 0; k0 < K; k0 += 16) {
        floatx4 a = *reinterpret_cast<const floatx4*>(xp + k0 + 4 * kg);
        floatx4 b = *reinterpret_cast<const floatx4*>(yp + k0 + 4 * kg);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    }
}

template <typename T> struct Mma;
template <> struct Mma<_Float16> {
    __device__ static __forceinline__ void run(floatx4& acc, const _Float16* X, int ldx,
                                               const _Float16* Y, int ldy, int K, int lane) {
        mma_f16(acc, X, ldx, Y, ldy, K, lane);
    }
    __device__ static __forceinline__ void run_xf32(floatx4& acc, const float* X, int ldx,
                                                    const _Float16* Y, int ldy, int K, int lane) {
        mma_f16_xf32(acc, X, ldx, Y, ldy, K, lane);
    }
};
template <> struct Mma<float> {
    __device__ static __forceinline__ void run(floatx4& acc, const float* X, int ldx,
                                               const float* Y, int ldy, int K, int lane) {
        mma_f32(acc, X, ldx, Y, ldy, K, lane);
    }
    __device__ static __forceinline__ void run_xf32(floatx4& acc, const float* X, int ldx,
                                                    const float* Y, int ldy, int K, int lane) {
        mma_f32(acc, X, ldx, Y, ldy, K, lane);
    }
};

// Workgroup barrier that orders LDS only: each wave waits for its own LDS
// operations, then all waves meet.  Unlike __syncthreads() it does not drain
// the wave's global loads and stores (vmcnt), so prefetches and output stores
// stay in flight across it.  Global memory written before it is not made
// visible to the other waves.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ floatx4 zero4() {
    floatx4 z;
    z[0] = z[1] = z[2] = z[3] = 0.f;
    return z;
}

// Map a linear workgroup index so that consecutive logical work items land
// on the same XCD.  Workgroups are dispatched round-robin over the 8 XCDs of
// an MI355X; logical items that share inputs (the value blocks of one head)
// then share that XCD's L2.  Identity when the count is not a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
    constexpr int NXCD = 8;
    if (nblk % NXCD != 0) return bid;
    return (bid % NXCD) * (nblk / NXCD) + bid / NXCD;
}

}  // namespace gdr
