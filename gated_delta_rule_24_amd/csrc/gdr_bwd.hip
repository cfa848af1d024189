// Gate-aware backward of the chunkwise forward (gdr_chunk_bwd).
//
// Loss L = <dO, o> + <dS_final, S_final>.  Per chunk, with S the chunk-start
// state, D the gradient of the chunk-end state and the forward quantities of
// the chunk kernels (S' = diag(e^{g_C}) S, R = X - E S', U = T R with
// T = (I + A)^-1, O = Qs S' + P U, S_next = S' + Kh^T U), reverse mode gives
//   dU  = Kh D + P^T dO            dR = T^T dU              dX = dR
//   dP  = lower(dO U^T)            dA = strict_lower(-dR U^T)
//   dQs = dO S'^T + dP Kh          dE = -dR S'^T + dA Kh
//   dKh = U D^T + dA^T E + dP^T Qs
//   dS' = D + Qs^T dO - E^T dR;    the chunk-start gradient is diag(e^{g_C}) dS'.
// E, Qs and Kh carry the in-chunk prefix g only as g_r - g_C, so with
//   dg_r = dE_r ⊙ E_r + dQs_r ⊙ Qs_r - dKh_r ⊙ Kh_r  and  Phi = rowsum(dS' ⊙ S'),
// the log-decay gradient of token i of the chunk is  Phi - sum_{r<i} dg_r.
// The erase gate and the write gate get separate gradients (the "gate-aware"
// accumulation of the Gated DeltaNet-2 Q&A page, Q4):
//   db = dE ⊙ k ⊙ e^{g-g_C}     dw = dX ⊙ v      dv = dX ⊙ w
//   dq = dQs ⊙ e^{g-g_C}        dk = dE ⊙ b ⊙ e^{g-g_C} + dKh ⊙ e^{g_C-g}
//
// Where the two-pass forward applies (bf16 activations, chunk 64), launch_bwd
// runs its WY pass, then its state chain (recording each chunk's S') beside the
// reverse chain of gdr_bwd_wy.hip on a second stream, then that file's
// per-chunk gradient kernel.  Otherwise (fp32 activations, chunks of 32, or the
// generic forward forced by flag), three launches on the caller's stream:
//   1. the generic forward recomputes every chunk-start state into the workspace;
//   2. dstate_kernel walks the chunks backwards carrying D (the columns of D
//      are independent; one workgroup per head and block of 32 value columns),
//      storing each chunk-end gradient and finally dS0;
//   3. grad_kernel computes the gradients of every chunk from its S and D, one
//      workgroup per (head, chunk), all chunks in parallel, with the value
//      dimension reduced in a fixed order (deterministic, no atomics).
// Dense products run on MFMA (f16 operands with bf16 activations, fp32
// operands with fp32 activations), accumulation and every element-wise step
// in fp32.  The chunk-local operands are built in LDS by prep_chunk, which
// both kernels share.
#include <mutex>

#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

namespace bwd {

// value columns per block: 32, or all of them for d_v = 16
template <int DV> constexpr int vb_of() { return DV < 32 ? DV : 32; }
constexpr float kF16DecayLimit = 10.0f;   // same operand range as the forward kernels
constexpr float kF32DecayLimit = 80.0f;

template <bool F32> struct Ty;
template <> struct Ty<false> { using T = _Float16; using F = half4; static constexpr int PAD = 8; };
template <> struct Ty<true> { using T = float; using F = floatx4; static constexpr int PAD = 4; };

__device__ __forceinline__ floatx4 splat(float x) {
    floatx4 f;
    f[0] = f[1] = f[2] = f[3] = x;
    return f;
}
__device__ __forceinline__ floatx4 expv(floatx4 x) {
    floatx4 r;
    r[0] = __expf(x[0]); r[1] = __expf(x[1]); r[2] = __expf(x[2]); r[3] = __expf(x[3]);
    return r;
}

template <typename T>
__device__ __forceinline__ void st4(T* p, floatx4 v) {
    if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<floatx4*>(p) = v;
    } else {
        half4 h;
        h[0] = (_Float16)v[0]; h[1] = (_Float16)v[1]; h[2] = (_Float16)v[2]; h[3] = (_Float16)v[3];
        *reinterpret_cast<half4*>(p) = h;
    }
}

// Four consecutive K values of one operand row: a vector load when K is the
// unit-stride axis (KC), else four strided scalar loads.
template <bool F32, bool KC>
__device__ __forceinline__ typename Ty<F32>::F frag(const typename Ty<F32>::T* p, int ks) {
    using F = typename Ty<F32>::F;
    if constexpr (KC) {
        return *reinterpret_cast<const F*>(p);
    } else {
        F f;
        f[0] = p[0]; f[1] = p[ks]; f[2] = p[2 * ks]; f[3] = p[3 * ks];
        return f;
    }
}

// One 16-wide K step.  f16: v_mfma_f32_16x16x16f16, lane group g supplies K
// positions 4g..4g+3.  fp32: four v_mfma_f32_16x16x4f32, the s-th consuming
// position 4g+s (the same permutation of K on both operands).
template <bool F32>
__device__ __forceinline__ floatx4 mma4(typename Ty<F32>::F a, typename Ty<F32>::F b, floatx4 acc) {
    if constexpr (F32) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
        return acc;
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, acc, 0, 0, 0);
    }
}

// acc(16x16) += X[16 rows, K in [k0, k1)] · Y[16 rows, same K]^T, where
// X(row, k) = X[row * xr + k * xk] and likewise Y; XK / YK state that the K
// stride is 1.  acc[i] is element (4*(lane>>4) + i, lane & 15).
template <bool F32, bool XK, bool YK>
__device__ __forceinline__ void mm(floatx4& acc, const typename Ty<F32>::T* X, int xr, int xk,
                                   const typename Ty<F32>::T* Y, int yr, int yk, int k0, int k1,
                                   int lane) {
    const int row = lane & 15, kq = 4 * (lane >> 4);
    const typename Ty<F32>::T* xp = X + row * xr;
    const typename Ty<F32>::T* yp = Y + row * yr;
    for (int k = k0; k < k1; k += 16) {
        const auto a = frag<F32, XK>(xp + (k + kq) * xk, xk);
        const auto b = frag<F32, YK>(yp + (k + kq) * yk, yk);
        acc = mma4<F32>(a, b, acc);
    }
}

// Shared LDS layout: the chunk operands (persistent across the phases of a
// chunk) followed by a region whose use changes from phase to phase.
template <int DK, int C, int NT, bool F32>
struct KeyLayout {
    using T = typename Ty<F32>::T;
    static constexpr int TS = (int)sizeof(T), PAD = Ty<F32>::PAD;
    static constexpr int LDE = DK + PAD;   // E, Qs, Kh  [C][LDE]
    static constexpr int LDT = C + PAD;    // T, P, A, dP, dA, Z  [C][LDT]
    static constexpr int LDA = C + 4;      // A fp32     [C][LDA]
    static constexpr int CQK = DK / 4;
    static constexpr int RGK = (NT / CQK < C) ? NT / CQK : C;
    static constexpr int RPK = C / RGK;
    static constexpr size_t oE = 0;
    static constexpr size_t oQ = oE + (size_t)C * LDE * TS;
    static constexpr size_t oK = oQ + (size_t)C * LDE * TS;
    static constexpr size_t oT = oK + (size_t)C * LDE * TS;
    static constexpr size_t oP = oT + (size_t)C * LDT * TS;
    static constexpr size_t oGam = oP + (size_t)C * LDT * TS;
    static constexpr size_t oEnd = oGam + (size_t)DK * 4;
    // prep scratch, placed by each kernel at offset `x` of its phase region
    static constexpr size_t pA = 0;
    static constexpr size_t pAh = pA + (size_t)C * LDA * 4;
    static constexpr size_t pZ = pAh + (size_t)C * LDT * TS;
    static constexpr size_t pTot = pZ + (size_t)(C / 2) * LDT * TS;
    static constexpr size_t pBytes = pTot + (size_t)RGK * DK * 4;
};

template <bool F32>
struct KeyBufs {
    using T = typename Ty<F32>::T;
    T* E; T* Q; T* K; T* Tm; T* P; float* gam;
    float* A; T* Ah; T* Z; float* tot;
};

template <int DK, int C, int NT, bool F32>
__device__ __forceinline__ KeyBufs<F32> key_bufs(unsigned char* smem, size_t x) {
    using L = KeyLayout<DK, C, NT, F32>;
    using T = typename Ty<F32>::T;
    KeyBufs<F32> s;
    s.E = reinterpret_cast<T*>(smem + L::oE);
    s.Q = reinterpret_cast<T*>(smem + L::oQ);
    s.K = reinterpret_cast<T*>(smem + L::oK);
    s.Tm = reinterpret_cast<T*>(smem + L::oT);
    s.P = reinterpret_cast<T*>(smem + L::oP);
    s.gam = reinterpret_cast<float*>(smem + L::oGam);
    s.A = reinterpret_cast<float*>(smem + x + L::pA);
    s.Ah = reinterpret_cast<T*>(smem + x + L::pAh);
    s.Z = reinterpret_cast<T*>(smem + x + L::pZ);
    s.tot = reinterpret_cast<float*>(smem + x + L::pTot);
    return s;
}

// The strictly upper 16x16 tiles of T and P are zero and never written by
// prep_chunk: clear them once per workgroup.
template <int C, bool F32>
__device__ __forceinline__ void clear_upper(typename Ty<F32>::T* Tm, typename Ty<F32>::T* P, int ldt) {
    using T = typename Ty<F32>::T;
    for (int idx = threadIdx.x; idx < C * C; idx += blockDim.x) {
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) {
            Tm[r * ldt + c] = (T)0.f;
            P[r * ldt + c] = (T)0.f;
        }
    }
}

// In-chunk prefix g of the log-decay (fp32) for this thread's rows, as in the
// forward: thread (cq, rg) holds channels 4cq..4cq+3 of rows rg*RPK.. ; returns
// g - g_C per row.  Uses `tot` ([RGK][DK] fp32) and two barriers.
template <int DK, int C, int NT>
__device__ __forceinline__ void chunk_prefix(const BwdParams& p, size_t tok0, float* tot,
                                             floatx4 (&gm)[KeyLayout<DK, C, NT, true>::RPK],
                                             floatx4& gC_out, floatx4& g0_out) {
    using L = KeyLayout<DK, C, NT, true>;
    constexpr int RPK = L::RPK, RGK = L::RGK, CQK = L::CQK;
    const int tid = threadIdx.x, cq = tid % CQK, rg = tid / CQK;
    const bool act = rg < RGK;
    const bool a_sc = (p.flags & GDR_ALPHA_SCALAR) != 0;
    floatx4 run = zero4();
    if (act) {
#pragma unroll
        for (int i = 0; i < RPK; ++i) {
            const size_t tok = tok0 + rg * RPK + i;
            run += a_sc ? splat(p.la[tok]) : *reinterpret_cast<const floatx4*>(p.la + tok * DK + 4 * cq);
            gm[i] = run;
        }
        *reinterpret_cast<floatx4*>(tot + rg * DK + 4 * cq) = run;
    }
    lds_barrier();
    if (act) {
        floatx4 off = zero4(), gC = zero4();
        for (int g = 0; g < RGK; ++g) {
            const floatx4 t = *reinterpret_cast<const floatx4*>(tot + g * DK + 4 * cq);
            if (g < rg) off += t;
            gC += t;
        }
#pragma unroll
        for (int i = 0; i < RPK; ++i) gm[i] = off + gm[i] - gC;
        gC_out = gC;
        g0_out = gm[0];
    }
    lds_barrier();
}

// Chunk operands in LDS: E, Qs, Kh (row-major), gamma = e^{g_C}, P (lower,
// with diagonal) and T = (I + A)^-1 (lower).  Returns nonzero, uniformly over
// the block, when the chunk's decay exceeds the operand range.
template <int DK, int C, int NT, bool F32>
__device__ int prep_chunk(const BwdParams& p, size_t tok0, const KeyBufs<F32>& s) {
    using L = KeyLayout<DK, C, NT, F32>;
    using T = typename Ty<F32>::T;
    constexpr int LDE = L::LDE, LDT = L::LDT, LDA = L::LDA;
    constexpr int CQK = L::CQK, RGK = L::RGK, RPK = L::RPK;
    constexpr int NB = C / 16, NW = NT / 64;
    constexpr float kLimit = F32 ? kF32DecayLimit : kF16DecayLimit;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, m_l = 4 * (lane >> 4);
    const int cq = tid % CQK, rg = tid / CQK;
    const bool act = rg < RGK;
    const bool b_sc = (p.flags & GDR_B_SCALAR) != 0;

    floatx4 q4[RPK], k4[RPK], b4[RPK];
    if (act) {
#pragma unroll
        for (int i = 0; i < RPK; ++i) {
            const size_t tok = tok0 + rg * RPK + i, ix = tok * DK + 4 * cq;
            q4[i] = load_act4<F32>(p.q, ix);
            k4[i] = load_act4<F32>(p.k, ix);
            b4[i] = b_sc ? splat(load_act1<F32>(p.b, tok)) : load_act4<F32>(p.b, ix);
        }
    }
    floatx4 gm[RPK], gC = zero4(), g0 = zero4();
    chunk_prefix<DK, C, NT>(p, tok0, s.tot, gm, gC, g0);
    int over = 0;
    if (act) {
        if (rg == 0) {
            *reinterpret_cast<floatx4*>(s.gam + 4 * cq) = expv(gC);
            over = !(g0[0] <= kLimit && g0[1] <= kLimit && g0[2] <= kLimit && g0[3] <= kLimit);
        }
#pragma unroll
        for (int i = 0; i < RPK; ++i) {
            const int r = rg * RPK + i;
            const floatx4 eg = expv(gm[i]), ek = expv(-gm[i]);
            st4<T>(s.E + r * LDE + 4 * cq, b4[i] * k4[i] * eg);
            st4<T>(s.Q + r * LDE + 4 * cq, q4[i] * eg);
            st4<T>(s.K + r * LDE + 4 * cq, k4[i] * ek);
        }
    }
    over = __syncthreads_or(over);

    // A = strict_lower(E Kh^T) (fp32 and operand copies), P = lower(Qs Kh^T)
    constexpr int NLT = NB * (NB + 1) / 2;
    for (int task = wave; task < 2 * NLT; task += NW) {
        const int which = task / NLT;
        int t = task % NLT, mt = 0;
        while (t > mt) { t -= mt + 1; ++mt; }
        const int nt = t;
        floatx4 acc = zero4();
        mm<F32, true, true>(acc, (which ? s.Q : s.E) + 16 * mt * LDE, LDE, 1, s.K + 16 * nt * LDE, LDE,
                            1, 0, DK, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * mt + m_l + i, col = 16 * nt + n_l;
            if (which == 0) {
                const float a = col < r ? acc[i] : 0.f;
                s.A[r * LDA + col] = a;
                s.Ah[r * LDT + col] = (T)a;
            } else {
                s.P[r * LDT + col] = (T)(col <= r ? acc[i] : 0.f);
            }
        }
    }
    lds_barrier();
    // diagonal 16x16 blocks of T by forward substitution (fp32), one lane per column
    if (wave == 0) {
        const int R = lane >> 4, j = lane & 15;
        if (R < NB) {
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == j) ? 1.f : 0.f;
                const float* arow = s.A + (16 * R + r) * LDA + 16 * R;
#pragma unroll
                for (int m = 0; m < r; ++m) acc -= arow[m] * x[m];
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) s.Tm[(16 * R + r) * LDT + 16 * R + j] = (T)x[r];
        }
    }
    lds_barrier();
    // off-diagonal blocks by doubling: T_BA = -T_BB (A_BA T_AA)
#pragma unroll
    for (int sz = 16; sz < C; sz *= 2) {
        const int nsub = sz / 16, ntask = (C / (2 * sz)) * nsub * nsub;
        for (int task = wave; task < ntask; task += NW) {
            const int pr = task / (nsub * nsub), mi = (task / nsub) % nsub, ni = task % nsub;
            const int a0 = 2 * sz * pr, b0 = a0 + sz;
            floatx4 acc = zero4();
            mm<F32, true, false>(acc, s.Ah + (b0 + 16 * mi) * LDT + a0, LDT, 1,
                                 s.Tm + a0 * LDT + a0 + 16 * ni, 1, LDT, 0, sz, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s.Z[(pr * sz + 16 * mi + m_l + i) * LDT + 16 * ni + n_l] = (T)acc[i];
        }
        lds_barrier();
        for (int task = wave; task < ntask; task += NW) {
            const int pr = task / (nsub * nsub), mi = (task / nsub) % nsub, ni = task % nsub;
            const int a0 = 2 * sz * pr, b0 = a0 + sz;
            floatx4 acc = zero4();
            mm<F32, true, false>(acc, s.Tm + (b0 + 16 * mi) * LDT + b0, LDT, 1,
                                 s.Z + pr * sz * LDT + 16 * ni, 1, LDT, 0, sz, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s.Tm[(b0 + 16 * mi + m_l + i) * LDT + a0 + 16 * ni + n_l] = (T)(-acc[i]);
        }
        lds_barrier();
    }
    return over;
}

// ---------------------------------------------------------------------------
// 2. chunk-end state gradients, backwards over the chunks
// ---------------------------------------------------------------------------
template <int DK, int DV, int C, bool F32>
struct DstateLayout {
    static constexpr int NT = 256;
    static constexpr int VB = vb_of<DV>();
    using K = KeyLayout<DK, C, NT, F32>;
    using T = typename Ty<F32>::T;
    static constexpr int TS = K::TS;
    static constexpr int LDV = VB + K::PAD;
    static constexpr size_t oX = (K::oEnd + 15) & ~size_t(15);
    static constexpr size_t wD = 0;                                   // [DK][LDV]
    static constexpr size_t wO = wD + (size_t)DK * LDV * TS;          // dO  [C][LDV]
    static constexpr size_t wZ = wO + (size_t)C * LDV * TS;           // Z   [C][LDV]
    static constexpr size_t wR = wZ + (size_t)C * LDV * TS;           // dR  [C][LDV]
    static constexpr size_t wBytes = wR + (size_t)C * LDV * TS;
    static constexpr size_t bytes = oX + (K::pBytes > wBytes ? K::pBytes : wBytes);
};

template <int DK, int DV, int C, bool F32>
__global__ __launch_bounds__(256, 1) void dstate_kernel(BwdParams p) {
    using L = DstateLayout<DK, DV, C, F32>;
    using K = typename L::K;
    using T = typename Ty<F32>::T;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    constexpr int NT = L::NT, NW = NT / 64;
    constexpr int LDE = K::LDE, LDT = K::LDT, LDV = L::LDV, VB = L::VB;
    constexpr int NVB = DV / VB, NB = C / 16, NNT = VB / 16, NMT = DK / 16;
    constexpr int NDT = NMT * NNT, NSW = (NDT + NW - 1) / NW;

    extern __shared__ __align__(16) unsigned char smem[];
    const KeyBufs<F32> kb = key_bufs<DK, C, NT, F32>(smem, L::oX);
    T* sD = reinterpret_cast<T*>(smem + L::oX + L::wD);
    T* sO = reinterpret_cast<T*>(smem + L::oX + L::wO);
    T* sZ = reinterpret_cast<T*>(smem + L::oX + L::wZ);
    T* sR = reinterpret_cast<T*>(smem + L::oX + L::wR);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, m_l = 4 * (lane >> 4);
    const int lid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int bh = lid / NVB, vb = lid % NVB;
    const int NC = p.T / C;
    const float qnan = __builtin_nanf("");

    clear_upper<C, F32>(kb.Tm, kb.P, LDT);
    floatx4 Dacc[NSW];
#pragma unroll
    for (int s = 0; s < NSW; ++s) {
        Dacc[s] = zero4();
        const int tile = wave + s * NW;
        if (tile < NDT && p.dSf) {
            const int mt = tile / NNT, nt = tile % NNT;
            const size_t base = ((size_t)bh * DK + 16 * mt + m_l) * DV + vb * VB + 16 * nt + n_l;
#pragma unroll
            for (int i = 0; i < 4; ++i) Dacc[s][i] = p.dSf[base + (size_t)i * DV];
        }
    }
    bool poisoned = false;

    for (int c = NC - 1; c >= 0; --c) {
        const size_t tok0 = (size_t)bh * p.T + (size_t)c * C;
        // the gradient of this chunk's end state, for the gradient kernel
#pragma unroll
        for (int s = 0; s < NSW; ++s) {
            const int tile = wave + s * NW;
            if (tile < NDT) {
                const int mt = tile / NNT, nt = tile % NNT;
                const size_t base = (((size_t)bh * NC + c) * DK + 16 * mt + m_l) * DV + vb * VB +
                                    16 * nt + n_l;
#pragma unroll
                for (int i = 0; i < 4; ++i) p.dstates[base + (size_t)i * DV] = poisoned ? qnan : Dacc[s][i];
            }
        }
        if (prep_chunk<DK, C, NT, F32>(p, tok0, kb)) poisoned = true;
        for (int idx = tid; idx < C * (VB / 4); idx += NT) {
            const int r = idx / (VB / 4), cq = idx % (VB / 4);
            st4<T>(sO + r * LDV + 4 * cq, load_act4<F32>(p.dO, (tok0 + r) * DV + vb * VB + 4 * cq));
        }
#pragma unroll
        for (int s = 0; s < NSW; ++s) {
            const int tile = wave + s * NW;
            if (tile < NDT) {
                const int mt = tile / NNT, nt = tile % NNT;
#pragma unroll
                for (int i = 0; i < 4; ++i) sD[(16 * mt + m_l + i) * LDV + 16 * nt + n_l] = (T)Dacc[s][i];
            }
        }
        lds_barrier();
        // Z = Kh D + P^T dO
        for (int task = wave; task < NB * NNT; task += NW) {
            const int mt = task / NNT, nt = task % NNT;
            floatx4 acc = zero4();
            mm<F32, true, false>(acc, kb.K + 16 * mt * LDE, LDE, 1, sD + 16 * nt, 1, LDV, 0, DK, lane);
            mm<F32, false, false>(acc, kb.P + 16 * mt, 1, LDT, sO + 16 * nt, 1, LDV, 16 * mt, C, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) sZ[(16 * mt + m_l + i) * LDV + 16 * nt + n_l] = (T)acc[i];
        }
        lds_barrier();
        // dR = T^T Z
        for (int task = wave; task < NB * NNT; task += NW) {
            const int mt = task / NNT, nt = task % NNT;
            floatx4 acc = zero4();
            mm<F32, false, false>(acc, kb.Tm + 16 * mt, 1, LDT, sZ + 16 * nt, 1, LDV, 16 * mt, C, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) sR[(16 * mt + m_l + i) * LDV + 16 * nt + n_l] = (T)acc[i];
        }
        lds_barrier();
        // D <- diag(gamma) (D + Qs^T dO - E^T dR)
#pragma unroll
        for (int s = 0; s < NSW; ++s) {
            const int tile = wave + s * NW;
            if (tile < NDT) {
                const int mt = tile / NNT, nt = tile % NNT;
                floatx4 a1 = zero4(), a2 = zero4();
                mm<F32, false, false>(a1, kb.Q + 16 * mt, 1, LDE, sO + 16 * nt, 1, LDV, 0, C, lane);
                mm<F32, false, false>(a2, kb.E + 16 * mt, 1, LDE, sR + 16 * nt, 1, LDV, 0, C, lane);
                const floatx4 gm = *reinterpret_cast<const floatx4*>(kb.gam + 16 * mt + m_l);
                Dacc[s] = gm * (Dacc[s] + a1 - a2);
            }
        }
        lds_barrier();
    }
    if (p.dS0) {
#pragma unroll
        for (int s = 0; s < NSW; ++s) {
            const int tile = wave + s * NW;
            if (tile < NDT) {
                const int mt = tile / NNT, nt = tile % NNT;
                const size_t base = ((size_t)bh * DK + 16 * mt + m_l) * DV + vb * VB + 16 * nt + n_l;
#pragma unroll
                for (int i = 0; i < 4; ++i) p.dS0[base + (size_t)i * DV] = poisoned ? qnan : Dacc[s][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 3. per-chunk gradients
// ---------------------------------------------------------------------------
template <int DK, int DV, int C, bool F32>
struct GradLayout {
    static constexpr int NT = 512;
    static constexpr int VB = vb_of<DV>();
    using K = KeyLayout<DK, C, NT, F32>;
    using T = typename Ty<F32>::T;
    static constexpr int TS = K::TS;
    static constexpr int LDV = VB + K::PAD;
    static constexpr int LDW = VB + 4;     // dw block, fp32
    static constexpr int LDG = DK + 4;     // g - g_C, then dg, fp32
    static constexpr int NCT = DK / 16;
    // row parts of the log-decay prefix (threads tid / DK >= NPART idle there)
    static constexpr int NPART = (NT / DK < C) ? NT / DK : C;
    // persistent small arrays after the key operands
    static constexpr size_t oPhi = K::oEnd;                          // [DK]
    static constexpr size_t oDWr = oPhi + (size_t)DK * 4;            // [C] dw row sums (scalar w)
    static constexpr size_t oRow = oDWr + (size_t)C * 4;             // [C] dg row sums (scalar alpha)
    static constexpr size_t oDBp = oRow + (size_t)C * 4;             // [NCT][C] db partials (scalar b)
    static constexpr size_t oMisc = oDBp + (size_t)NCT * C * 4;      // [4]
    static constexpr size_t oX = (oMisc + 16 + 15) & ~size_t(15);
    // value-block phase
    static constexpr size_t vS = 0;                                  // S'  [DK][LDV]
    static constexpr size_t vD = vS + (size_t)DK * LDV * TS;         // D   [DK][LDV]
    static constexpr size_t vO = vD + (size_t)DK * LDV * TS;         // dO  [C][LDV]
    static constexpr size_t vR = vO + (size_t)C * LDV * TS;          // R
    static constexpr size_t vU = vR + (size_t)C * LDV * TS;          // U
    static constexpr size_t vdU = vU + (size_t)C * LDV * TS;         // dU
    static constexpr size_t vdR = vdU + (size_t)C * LDV * TS;        // dR
    static constexpr size_t vW = vdR + (size_t)C * LDV * TS;         // dw block fp32 [C][LDW]
    static constexpr size_t vBytes = vW + (size_t)C * LDW * 4;
    // final phase
    static constexpr size_t fP = 0;                                  // dP [C][LDT]
    static constexpr size_t fA = fP + (size_t)C * K::LDT * TS;       // dA [C][LDT]
    static constexpr size_t fG = fA + (size_t)C * K::LDT * TS;       // [C][LDG] fp32
    static constexpr size_t fTot = fG + (size_t)C * LDG * 4;         // [max(RGK, NPART)][DK] fp32
    static constexpr int NTOT = K::RGK > NPART ? K::RGK : NPART;
    static constexpr size_t fBytes = fTot + (size_t)NTOT * DK * 4;
    static constexpr size_t xBytes = K::pBytes > vBytes ? (K::pBytes > fBytes ? K::pBytes : fBytes)
                                                        : (vBytes > fBytes ? vBytes : fBytes);
    static constexpr size_t bytes = oX + xBytes;
};

template <int DK, int DV, int C, bool F32>
__global__ __launch_bounds__(512, 1) void grad_kernel(BwdParams p) {
    using L = GradLayout<DK, DV, C, F32>;
    using K = typename L::K;
    using T = typename Ty<F32>::T;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    constexpr int NT = L::NT, NW = NT / 64;
    constexpr int LDE = K::LDE, LDT = K::LDT, LDV = L::LDV, LDW = L::LDW, LDG = L::LDG, VB = L::VB;
    constexpr int NVB = DV / VB, NB = C / 16, NNT = VB / 16, NCT = L::NCT;
    constexpr int NKT = NB * NCT, NKS = (NKT + NW - 1) / NW;      // C x DK tiles
    constexpr int NLT = NB * (NB + 1) / 2, NLS = (NLT + NW - 1) / NW;
    constexpr int NVT = NB * NNT;                                 // C x VB tiles
    static_assert(NCT <= NW, "one state row tile per wave");

    extern __shared__ __align__(16) unsigned char smem[];
    const KeyBufs<F32> kb = key_bufs<DK, C, NT, F32>(smem, L::oX);
    float* sPhi = reinterpret_cast<float*>(smem + L::oPhi);
    float* sDWr = reinterpret_cast<float*>(smem + L::oDWr);
    float* sRow = reinterpret_cast<float*>(smem + L::oRow);
    float* sDBp = reinterpret_cast<float*>(smem + L::oDBp);
    float* sMisc = reinterpret_cast<float*>(smem + L::oMisc);
    unsigned char* X = smem + L::oX;
    T* sS = reinterpret_cast<T*>(X + L::vS);
    T* sD = reinterpret_cast<T*>(X + L::vD);
    T* sO = reinterpret_cast<T*>(X + L::vO);
    T* sR = reinterpret_cast<T*>(X + L::vR);
    T* sU = reinterpret_cast<T*>(X + L::vU);
    T* sdU = reinterpret_cast<T*>(X + L::vdU);
    T* sdR = reinterpret_cast<T*>(X + L::vdR);
    float* sW = reinterpret_cast<float*>(X + L::vW);
    T* sdP = reinterpret_cast<T*>(X + L::fP);
    T* sdA = reinterpret_cast<T*>(X + L::fA);
    float* sG = reinterpret_cast<float*>(X + L::fG);
    float* sTot = reinterpret_cast<float*>(X + L::fTot);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_l = lane & 15, m_l = 4 * (lane >> 4);
    const int NC = p.T / C;
    const int bh = (int)blockIdx.x / NC, c = (int)blockIdx.x % NC;
    const size_t tok0 = (size_t)bh * p.T + (size_t)c * C;
    const size_t sbase = ((size_t)bh * NC + c) * DK * DV;        // this chunk's S and D
    const bool a_sc = (p.flags & GDR_ALPHA_SCALAR) != 0;
    const bool b_sc = (p.flags & GDR_B_SCALAR) != 0;
    const bool w_sc = (p.flags & GDR_W_SCALAR) != 0;

    clear_upper<C, F32>(kb.Tm, kb.P, LDT);
    for (int i = tid; i < C; i += NT) sDWr[i] = 0.f;
    const int over = prep_chunk<DK, C, NT, F32>(p, tok0, kb);
    const float poison = over ? __builtin_nanf("") : 0.f;

    floatx4 aQ[NKS], aE[NKS], aK[NKS], aP[NLS], aA[NLS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) aQ[s] = aE[s] = aK[s] = zero4();
#pragma unroll
    for (int s = 0; s < NLS; ++s) aP[s] = aA[s] = zero4();
    floatx4 phi = zero4();

    for (int vb = 0; vb < NVB; ++vb) {
        const int col0 = vb * VB;
        for (int idx = tid; idx < DK * (VB / 4); idx += NT) {
            const int r = idx / (VB / 4), cq = idx % (VB / 4);
            const size_t ix = sbase + (size_t)r * DV + col0 + 4 * cq;
            st4<T>(sS + r * LDV + 4 * cq, *reinterpret_cast<const floatx4*>(p.states + ix) * kb.gam[r]);
            st4<T>(sD + r * LDV + 4 * cq, *reinterpret_cast<const floatx4*>(p.dstates + ix));
        }
        for (int idx = tid; idx < C * (VB / 4); idx += NT) {
            const int r = idx / (VB / 4), cq = idx % (VB / 4);
            st4<T>(sO + r * LDV + 4 * cq, load_act4<F32>(p.dO, (tok0 + r) * DV + col0 + 4 * cq));
        }
        lds_barrier();
        // R = X - E S'  and  dU = Kh D + P^T dO
        for (int task = wave; task < 2 * NVT; task += NW) {
            const int which = task / NVT, t = task % NVT, mt = t / NNT, nt = t % NNT;
            floatx4 acc = zero4();
            if (which == 0) {
                mm<F32, true, false>(acc, kb.E + 16 * mt * LDE, LDE, 1, sS + 16 * nt, 1, LDV, 0, DK, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + m_l + i, col = col0 + 16 * nt + n_l;
                    const size_t tok = tok0 + r;
                    const float x = load_act1<F32>(p.v, tok * DV + col) *
                                    load_act1<F32>(p.w, w_sc ? tok : tok * DV + col);
                    sR[r * LDV + 16 * nt + n_l] = (T)(x - acc[i]);
                }
            } else {
                mm<F32, true, false>(acc, kb.K + 16 * mt * LDE, LDE, 1, sD + 16 * nt, 1, LDV, 0, DK, lane);
                mm<F32, false, false>(acc, kb.P + 16 * mt, 1, LDT, sO + 16 * nt, 1, LDV, 16 * mt, C, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) sdU[(16 * mt + m_l + i) * LDV + 16 * nt + n_l] = (T)acc[i];
            }
        }
        lds_barrier();
        // U = T R  and  dR = T^T dU; dv and dw from the fp32 dR
        for (int task = wave; task < 2 * NVT; task += NW) {
            const int which = task / NVT, t = task % NVT, mt = t / NNT, nt = t % NNT;
            floatx4 acc = zero4();
            if (which == 0) {
                mm<F32, true, false>(acc, kb.Tm + 16 * mt * LDT, LDT, 1, sR + 16 * nt, 1, LDV, 0,
                                     16 * (mt + 1), lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) sU[(16 * mt + m_l + i) * LDV + 16 * nt + n_l] = (T)acc[i];
            } else {
                mm<F32, false, false>(acc, kb.Tm + 16 * mt, 1, LDT, sdU + 16 * nt, 1, LDV, 16 * mt, C, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + m_l + i, col = col0 + 16 * nt + n_l;
                    const size_t tok = tok0 + r;
                    sdR[r * LDV + 16 * nt + n_l] = (T)acc[i];
                    const float wv = load_act1<F32>(p.w, w_sc ? tok : tok * DV + col);
                    const float vv = load_act1<F32>(p.v, tok * DV + col);
                    p.dv[tok * DV + col] = acc[i] * wv + poison;
                    if (w_sc) sW[r * LDW + 16 * nt + n_l] = acc[i] * vv;
                    else p.dw[tok * DV + col] = acc[i] * vv + poison;
                }
            }
        }
        lds_barrier();
        if (w_sc && tid < C) {
            float sum = 0.f;
            for (int j = 0; j < VB; ++j) sum += sW[tid * LDW + j];
            sDWr[tid] += sum;
        }
        // dP += dO U^T, (dR U^T) into aA, dQs += dO S'^T, (dR S'^T) into aE, dKh += U D^T
#pragma unroll
        for (int s = 0; s < NLS; ++s) {
            int t = wave + s * NW, mt = 0;
            if (t < NLT) {
                while (t > mt) { t -= mt + 1; ++mt; }
                const int nt = t;
                mm<F32, true, true>(aP[s], sO + 16 * mt * LDV, LDV, 1, sU + 16 * nt * LDV, LDV, 1, 0, VB, lane);
                mm<F32, true, true>(aA[s], sdR + 16 * mt * LDV, LDV, 1, sU + 16 * nt * LDV, LDV, 1, 0, VB, lane);
            }
        }
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const int t = wave + s * NW;
            if (t < NKT) {
                const int rt = t / NCT, ct = t % NCT;
                mm<F32, true, true>(aQ[s], sO + 16 * rt * LDV, LDV, 1, sS + 16 * ct * LDV, LDV, 1, 0, VB, lane);
                mm<F32, true, true>(aE[s], sdR + 16 * rt * LDV, LDV, 1, sS + 16 * ct * LDV, LDV, 1, 0, VB, lane);
                mm<F32, true, true>(aK[s], sU + 16 * rt * LDV, LDV, 1, sD + 16 * ct * LDV, LDV, 1, 0, VB, lane);
            }
        }
        // dS' = D + Qs^T dO - E^T dR on state rows 16*wave.. ; Phi += rowsum(dS' ⊙ S') (fp32 S, D)
        if (wave < NCT) {
            const int mt = wave;
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) {
                floatx4 a1 = zero4(), a2 = zero4();
                mm<F32, false, false>(a1, kb.Q + 16 * mt, 1, LDE, sO + 16 * nt, 1, LDV, 0, C, lane);
                mm<F32, false, false>(a2, kb.E + 16 * mt, 1, LDE, sdR + 16 * nt, 1, LDV, 0, C, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * mt + m_l + i;
                    const size_t ix = sbase + (size_t)row * DV + col0 + 16 * nt + n_l;
                    const float sp = p.states[ix] * kb.gam[row];
                    phi[i] += (p.dstates[ix] + a1[i] - a2[i]) * sp;
                }
            }
        }
        lds_barrier();
    }

    // Phi: sum over the 16 lanes of each row group (fixed butterfly order)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = phi[i];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        v += __shfl_xor(v, 8, 64);
        phi[i] = v;
    }
    if (wave < NCT && n_l == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sPhi[16 * wave + m_l + i] = phi[i];
    }
    // dP = lower(dO U^T), dA = strict_lower(-dR U^T) as operands
    for (int idx = tid; idx < C * C; idx += NT) {
        const int r = idx / C, cc = idx % C;
        if ((cc >> 4) > (r >> 4)) {
            sdP[r * LDT + cc] = (T)0.f;
            sdA[r * LDT + cc] = (T)0.f;
        }
    }
#pragma unroll
    for (int s = 0; s < NLS; ++s) {
        int t = wave + s * NW, mt = 0;
        if (t < NLT) {
            while (t > mt) { t -= mt + 1; ++mt; }
            const int nt = t;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + m_l + i, cc = 16 * nt + n_l;
                sdP[r * LDT + cc] = (T)(cc <= r ? aP[s][i] : 0.f);
                sdA[r * LDT + cc] = (T)(cc < r ? -aA[s][i] : 0.f);
            }
        }
    }
    lds_barrier();
    // dQs += dP Kh; dE = dA Kh - dR S'^T; dKh += dA^T E + dP^T Qs
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const int t = wave + s * NW;
        if (t < NKT) {
            const int rt = t / NCT, ct = t % NCT;
            mm<F32, true, false>(aQ[s], sdP + 16 * rt * LDT, LDT, 1, kb.K + 16 * ct, 1, LDE, 0, 16 * (rt + 1), lane);
            floatx4 t1 = zero4();
            mm<F32, true, false>(t1, sdA + 16 * rt * LDT, LDT, 1, kb.K + 16 * ct, 1, LDE, 0, 16 * (rt + 1), lane);
            aE[s] = t1 - aE[s];
            mm<F32, false, false>(aK[s], sdA + 16 * rt, 1, LDT, kb.E + 16 * ct, 1, LDE, 16 * rt, C, lane);
            mm<F32, false, false>(aK[s], sdP + 16 * rt, 1, LDT, kb.Q + 16 * ct, 1, LDE, 16 * rt, C, lane);
        }
    }
    // g - g_C again, in fp32, for the element-wise gradients
    {
        constexpr int RPK = K::RPK, CQK = K::CQK;
        floatx4 gm[RPK], gC = zero4(), g0 = zero4();
        chunk_prefix<DK, C, NT>(p, tok0, sTot, gm, gC, g0);
        const int cq = tid % CQK, rg = tid / CQK;
        if (rg < K::RGK) {
#pragma unroll
            for (int i = 0; i < RPK; ++i)
                *reinterpret_cast<floatx4*>(sG + (rg * RPK + i) * LDG + 4 * cq) = gm[i];
        }
    }
    lds_barrier();
    // element-wise gradients; dg replaces g - g_C in sG
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const int t = wave + s * NW;
        if (t < NKT) {
            const int rt = t / NCT, ct = t % NCT;
            floatx4 dbv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + m_l + i, ch = 16 * ct + n_l;
                const size_t tok = tok0 + r, ix = tok * DK + ch;
                const float gm = sG[r * LDG + ch];
                const float eg = __expf(gm), ek = __expf(-gm);
                const float qv = load_act1<F32>(p.q, ix), kv = load_act1<F32>(p.k, ix);
                const float bv = load_act1<F32>(p.b, b_sc ? tok : ix);
                const float dQs = aQ[s][i], dE = aE[s][i], dKh = aK[s][i];
                p.dq[ix] = dQs * eg + poison;
                p.dk[ix] = dE * bv * eg + dKh * ek + poison;
                dbv[i] = dE * kv * eg;
                if (!b_sc) p.db[ix] = dbv[i] + poison;
                sG[r * LDG + ch] = dE * (bv * kv * eg) + dQs * (qv * eg) - dKh * (kv * ek);
            }
            if (b_sc) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = dbv[i];
                    v += __shfl_xor(v, 1, 64);
                    v += __shfl_xor(v, 2, 64);
                    v += __shfl_xor(v, 4, 64);
                    v += __shfl_xor(v, 8, 64);
                    if (n_l == 0) sDBp[ct * C + 16 * rt + m_l + i] = v;
                }
            }
        }
    }
    lds_barrier();
    if (!a_sc) {
        // d log alpha_i = Phi - sum_{r<i} dg_r, per channel; NPART threads per channel
        constexpr int NPART = L::NPART, RPP = C / NPART;
        const int ch = tid % DK, part = tid / DK;
        const bool on = part < NPART;
        float sum = 0.f;
        if (on) {
            for (int r = 0; r < RPP; ++r) sum += sG[(part * RPP + r) * LDG + ch];
            sTot[part * DK + ch] = sum;
        }
        lds_barrier();
        float off = sPhi[ch];
        for (int q = 0; q < part && on; ++q) off -= sTot[q * DK + ch];
        for (int r = 0; r < RPP && on; ++r) {
            const int row = part * RPP + r;
            p.dla[(tok0 + row) * DK + ch] = off + poison;
            off -= sG[row * LDG + ch];
        }
    } else {
        // scalar decay: the channel sum of the above
        if (tid < C) {
            float sum = 0.f;
            for (int ch = 0; ch < DK; ++ch) sum += sG[tid * LDG + ch];
            sRow[tid] = sum;
        }
        if (tid == 64) {
            float sum = 0.f;
            for (int ch = 0; ch < DK; ++ch) sum += sPhi[ch];
            sMisc[0] = sum;
        }
        lds_barrier();
        if (wave == 0) {
            const float v = lane < C ? sRow[lane] : 0.f;
            float incl = v;
#pragma unroll
            for (int d = 1; d < 64; d *= 2) {
                const float u = __shfl_up(incl, d, 64);
                if (lane >= d) incl += u;
            }
            if (lane < C) p.dla[tok0 + lane] = sMisc[0] - (incl - v) + poison;
        }
    }
    if (b_sc && tid < C) {
        float sum = 0.f;
        for (int ct = 0; ct < NCT; ++ct) sum += sDBp[ct * C + tid];
        p.db[tok0 + tid] = sum + poison;
    }
    if (w_sc && tid < C) p.dw[tok0 + tid] = sDWr[tid] + poison;
}

// T == 0: dS0 = dS_final (or zero).  A kernel rather than a memset/memcpy so
// the call stays capturable.
__global__ void copy_or_zero(float* dst, const float* src, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

template <int DK, int DV, int C, bool F32>
static hipError_t launch_t(const BwdParams& p, hipStream_t st, bool with_dstate) {
    using LD = DstateLayout<DK, DV, C, F32>;
    using LG = GradLayout<DK, DV, C, F32>;
    auto kd = dstate_kernel<DK, DV, C, F32>;
    auto kg = grad_kernel<DK, DV, C, F32>;
    static std::atomic<unsigned long long> done_d{0}, done_g{0};
    hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(kd), (int)LD::bytes, done_d);
    if (e != hipSuccess) return e;
    e = ensure_dyn_lds(reinterpret_cast<const void*>(kg), (int)LG::bytes, done_g);
    if (e != hipSuccess) return e;
    const int NC = p.T / C;
    if (with_dstate) {
        hipLaunchKernelGGL(kd, dim3((unsigned)(p.BH * (DV / LD::VB))), dim3(LD::NT), LD::bytes, st, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kg, dim3((unsigned)(p.BH * NC)), dim3(LG::NT), LG::bytes, st, p);
    return hipGetLastError();
}

// the blocking the backward runs with: fp32 operands need chunks of at most 32
// to fit LDS
int bwd_chunk(int chunk, uint32_t flags) {
    if (flags & GDR_ACT_F32) return chunk < 32 ? chunk : 32;
    return chunk;
}

}  // namespace bwd

static bool head_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool bwd_supported(int dk, int dv, int chunk, uint32_t /*flags*/) {
    return head_ok(dk) && head_ok(dv) && (chunk == 16 || chunk == 32 || chunk == 64);
}

// The generic three-launch path for one head shape, blocked with chunks of cb.
template <int DK, int DV>
static hipError_t launch_generic(const BwdParams& p, hipStream_t st, int cb, bool f32) {
    if (f32) {
        if (cb == 32) return bwd::launch_t<DK, DV, 32, true>(p, st, true);
        if (cb == 16) return bwd::launch_t<DK, DV, 16, true>(p, st, true);
        return hipErrorInvalidValue;
    }
    if (cb == 64) return bwd::launch_t<DK, DV, 64, false>(p, st, true);
    if (cb == 32) return bwd::launch_t<DK, DV, 32, false>(p, st, true);
    if (cb == 16) return bwd::launch_t<DK, DV, 16, false>(p, st, true);
    return hipErrorInvalidValue;
}

template <int DK>
static hipError_t launch_generic_dv(const BwdParams& p, int dv, hipStream_t st, int cb, bool f32) {
    switch (dv) {
        case 16: return launch_generic<DK, 16>(p, st, cb, f32);
        case 32: return launch_generic<DK, 32>(p, st, cb, f32);
        case 64: return launch_generic<DK, 64>(p, st, cb, f32);
        case 128: return launch_generic<DK, 128>(p, st, cb, f32);
    }
    return hipErrorInvalidValue;
}

// A second stream per device, at the default priority, for the backward's
// reverse chain: it depends only on the WY records, so it runs beside the
// forward state chain (both are sequential over the chunks and leave most of
// each compute unit idle).  The fork and join go through events, so the
// caller's stream sees the usual ordering and the pattern stays capturable.
namespace {
struct SideStream {
    std::mutex m;
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;
SideStream& side_stream(int dev) {
    static SideStream sides[kMaxSideDevices];
    return sides[dev];
}
hipError_t side_init(SideStream& sd) {
    if (sd.s && sd.fork && sd.join) return hipSuccess;
    hipError_t e = hipSuccess;
    if (!sd.s) e = hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking);
    if (e == hipSuccess && !sd.fork) e = hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming);
    if (e == hipSuccess && !sd.join) e = hipEventCreateWithFlags(&sd.join, hipEventDisableTiming);
    return e;
}
}  // namespace

// The two chains of the two-pass backward: the reverse chain (dchain) on the
// side stream, forked from and joined back to st, beside the forward state
// chain (state_chain) on st; one after the other on st when no side stream
// can be made.
template <typename StateChain>
static hipError_t run_two_chains(const BwdParams& p, int dk, int dv, hipStream_t st, StateChain state_chain) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    SideStream* sd = (dev >= 0 && dev < kMaxSideDevices) ? &side_stream(dev) : nullptr;
    std::unique_lock<std::mutex> lk;
    if (sd) {
        lk = std::unique_lock<std::mutex>(sd->m);
        if (side_init(*sd) != hipSuccess) {
            // no second stream (e.g. first use inside a graph capture that forbids
            // creating one): the reverse chain runs after the state chain instead
            (void)hipGetLastError();
            sd = nullptr;
        }
    }
    if (sd) {
        e = hipEventRecord(sd->fork, st);
        if (e == hipSuccess) e = hipStreamWaitEvent(sd->s, sd->fork, 0);
        if (e == hipSuccess) e = launch_bwd_dchain(p, dk, dv, p.records, sd->s);
        if (e == hipSuccess) e = hipEventRecord(sd->join, sd->s);
        if (e == hipSuccess) e = state_chain();
        if (e == hipSuccess) e = hipStreamWaitEvent(st, sd->join, 0);
    } else {
        e = launch_bwd_dchain(p, dk, dv, p.records, st);
        if (e == hipSuccess) e = state_chain();
    }
    return e;
}

// the two-pass path keeps S' and the state gradients as f16 fragments, the
// generic path as fp32 rows
bool bwd_two_pass_supported(int dk, int dv, int chunk, uint32_t flags) {
    return dk == dv && fwd_wy_supported(dk, dv, bwd::bwd_chunk(chunk, flags), flags);
}

static bool bwd_two_pass(int dk, int dv, int T, int cb, uint32_t flags) {
    return T > 0 && dk == dv && fwd_wy_supported(dk, dv, cb, flags);
}

size_t bwd_states_bytes(int BH, int T, int dk, int dv, int chunk, uint32_t flags) {
    const int cb = bwd::bwd_chunk(chunk, flags);
    const size_t elem = bwd_two_pass(dk, dv, T, cb, flags) ? 2 : sizeof(float);
    return (size_t)BH * (size_t)(T / cb) * (size_t)dk * (size_t)dv * elem;
}

size_t bwd_workspace_bytes(int BH, int T, int dk, int dv, int chunk, uint32_t flags) {
    const int cb = bwd::bwd_chunk(chunk, flags);
    // chunk-start states, chunk-end state gradients, and (where the two-pass forward
    // recomputes the states) its per-chunk records
    size_t n = 2 * bwd_states_bytes(BH, T, dk, dv, chunk, flags);
    if (bwd_two_pass(dk, dv, T, cb, flags)) n += fwd_wy_workspace_bytes(BH, T, dk, dv, true);
    return n;
}

hipError_t launch_bwd(const BwdParams& p, int dk, int dv, int chunk, hipStream_t st) {
    if (!bwd_supported(dk, dv, chunk, p.flags)) return hipErrorInvalidValue;
    if (p.T == 0) {
        if (!p.dS0) return hipSuccess;
        const size_t n = (size_t)p.BH * dk * dv;
        hipLaunchKernelGGL(bwd::copy_or_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           p.dS0, p.dSf, n);
        return hipGetLastError();
    }
    const int cb = bwd::bwd_chunk(chunk, p.flags);
    if (p.T % cb != 0) return hipErrorInvalidValue;
    // 1. chunk-start states
    FwdParams f;
    f.q = p.q; f.k = p.k; f.v = p.v; f.la = p.la; f.b = p.b; f.w = p.w; f.S0 = p.S0;
    f.o = nullptr; f.Sf = nullptr; f.states = nullptr; f.state_frags = nullptr;
    f.cu_seqlens = nullptr; f.chunk_off = nullptr; f.chunk_tab = nullptr; f.seq_order = nullptr; f.nseq = 0;
    f.BH = p.BH; f.T = p.T; f.flags = p.flags & ~(uint32_t)GDR_OUT_BF16;
    hipError_t e;
    if (bwd_two_pass(dk, dv, p.T, cb, p.flags)) {
        if (!p.records || !p.state_frags || !p.dstate_frags) return hipErrorInvalidValue;
        // two-pass forward (its records keep the operands the reverse passes need,
        // its chain the decayed chunk-start states), the reverse chain over those
        // records, then every chunk's gradients
        f.state_frags = p.state_frags;
        e = launch_fwd_wy(f, dk, dv, p.records, st, true, kWyPass);
        if (e != hipSuccess) return e;
        e = run_two_chains(p, dk, dv, st, [&] { return launch_fwd_wy(f, dk, dv, p.records, st, true, kChainPass); });
        if (e != hipSuccess) return e;
        return launch_bwd_wgrad(p, dk, dv, p.records, st);
    }
    f.states = p.states;
    int used = 0;
    e = launch_fwd(f, dk, dv, cb, st, &used);
    if (e != hipSuccess) return e;
    if (used != cb) return hipErrorInvalidValue;
    // 2 and 3
    const bool f32 = (p.flags & GDR_ACT_F32) != 0;
    switch (dk) {
        case 16: return launch_generic_dv<16>(p, dv, st, cb, f32);
        case 32: return launch_generic_dv<32>(p, dv, st, cb, f32);
        case 64: return launch_generic_dv<64>(p, dv, st, cb, f32);
        case 128: return launch_generic_dv<128>(p, dv, st, cb, f32);
    }
    return hipErrorInvalidValue;
}

// Packed sequences: the same three steps over the packed records, S' and D
// fragments (numbered head * chunk count + chunk), after the prep step.
static size_t packed_rec_bytes(int dk, int dv) { return fwd_wy_workspace_bytes(1, 64, dk, dv, true); }

size_t bwd_varlen_workspace_bytes(int H, long long T, int nseq, int dk, int dv) {
    if (H < 1 || nseq < 1 || T < 0 || dk != dv || !(dk == 64 || dk == 128)) return 0;
    const size_t per_chunk = packed_rec_bytes(dk, dv) + 2 * (size_t)dk * dv * 2;
    return (size_t)H * packed_max_chunks(T, nseq) * per_chunk + packed_prep_bytes(T, nseq);
}

hipError_t launch_bwd_varlen(const BwdParams& p0, int dk, int dv, void* ws, size_t ws_bytes, hipStream_t st) {
    const size_t need = bwd_varlen_workspace_bytes(p0.BH, p0.T, p0.nseq, dk, dv);
    if (need == 0 || ws_bytes < need || !p0.cu_seqlens || !fwd_wy_supported(dk, dv, 64, p0.flags))
        return hipErrorInvalidValue;
    BwdParams p = p0;
    const size_t n = (size_t)p.BH * packed_max_chunks(p.T, p.nseq);
    const size_t recb = n * packed_rec_bytes(dk, dv), fragb = n * (size_t)dk * dv * 2;
    unsigned char* base = reinterpret_cast<unsigned char*>(ws);
    p.records = base;
    p.state_frags = base + recb;
    p.dstate_frags = base + recb + fragb;
    int *off = nullptr, *tab = nullptr, *ord = nullptr;
    hipError_t e = launch_packed_prep(p.cu_seqlens, p.nseq, p.T, base + recb + 2 * fragb, &off, &tab, &ord, st);
    if (e != hipSuccess) return e;
    p.chunk_off = off;
    p.chunk_tab = tab;
    p.seq_order = ord;
    FwdParams f;
    f.q = p.q; f.k = p.k; f.v = p.v; f.la = p.la; f.b = p.b; f.w = p.w; f.S0 = p.S0;
    f.o = nullptr; f.Sf = nullptr; f.states = nullptr; f.state_frags = p.state_frags;
    f.cu_seqlens = p.cu_seqlens; f.chunk_off = off; f.chunk_tab = tab; f.seq_order = ord; f.nseq = p.nseq;
    f.BH = p.BH; f.T = p.T; f.flags = p.flags & ~(uint32_t)GDR_OUT_BF16;
    e = launch_fwd_wy_packed(f, dk, dv, p.records, st, true, kWyPass);
    if (e != hipSuccess) return e;
    e = run_two_chains(p, dk, dv, st, [&] { return launch_fwd_wy_packed(f, dk, dv, p.records, st, true, kChainPass); });
    if (e != hipSuccess) return e;
    return launch_bwd_wgrad(p, dk, dv, p.records, st);
}

}  // namespace gdr
