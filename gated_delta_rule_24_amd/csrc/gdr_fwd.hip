// Chunkwise-parallel forward of the gated delta rule, fused into one kernel.
//
// Method (Gated DeltaNet-2 Q&A page, Q4; "Gated DeltaNet-2 Review" §3-2
// item 5): the in-chunk cumulative channel decay is absorbed into the
// rank-one erase factor, which turns each chunk into a decay-free asymmetric
// delta recurrence with a WY (UT) solution; only the state crosses chunks.
//
// Per (batch·head) and chunk of C tokens, with g_r the in-chunk inclusive
// cumulative log-decay (fp32) and g_C its value at the last token:
//   E  = b ⊙ k ⊙ exp(g - g_C)    Qs = q ⊙ exp(g - g_C)    Kh = k ⊙ exp(g_C - g)
//   X  = w ⊙ v
//   A  = strict_lower(E Kh^T)    P = lower(Qs Kh^T)        T = (I + A)^-1
//   S' = diag(exp(g_C)) S        (state pre-scaled to the chunk end)
//   U  = T (X - E S')            (rows are the per-token gated prediction errors)
//   O  = Qs S' + P U             (read-out after each token's write)
//   S  = S' + Kh^T U             (carried to the next chunk)
// Every factor exp(g_r - g_i) with i <= r is split as exp(g_r - g_C) ·
// exp(g_C - g_i).  With f16 operands the large factor stays representable
// while the decay accumulated inside one chunk is at most kF16DecayLimit nats
// on every channel (kF32DecayLimit with fp32 operands).  A chunk beyond the
// limit is detected and poisons the outputs of its head with NaN from that
// chunk on, instead of returning silently wrong values.
//
// Mapping: one workgroup (4 waves) per (batch·head, block of VB value
// columns).  Columns of the state are independent (every operator acts on S
// from the left), so value blocks of one head run in parallel and only the
// key-side work (gate prep, A, P, T) is repeated per block.  The fp32 state
// block lives in MFMA accumulator registers for the whole sequence.  Global
// loads for chunk c+1 are issued before the MFMA work of chunk c.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

template <bool F32> struct Cfg;
template <> struct Cfg<false> { using T = _Float16; static constexpr int PAD = 8; };
template <> struct Cfg<true> { using T = float; static constexpr int PAD = 4; };

template <int DK, int DV, int C, int VB, bool F32>
struct FwdLayout {
    using T = typename Cfg<F32>::T;
    static constexpr int PAD = Cfg<F32>::PAD;
    static constexpr int NT = 256, NW = 4;
    static constexpr int TS = (int)sizeof(T);
    // key-side load mapping: 4 channels x RPK consecutive rows per thread
    static constexpr int CQK = DK / 4;
    static constexpr int RGK = (NT / CQK < C) ? NT / CQK : C;
    static constexpr int RPK = C / RGK;
    // value-side load mapping
    static constexpr int CQV = VB / 4;
    static constexpr int RGV = (NT / CQV < C) ? NT / CQV : C;
    static constexpr int RPV = C / RGV;
    // LDS row strides (elements)
    static constexpr int LDE = DK + PAD;   // E, Qs, Kh       [C][LDE]
    static constexpr int LDC = C + PAD;    // KhT [DK], Th/TT/P [C], RT/UT [VB]
    static constexpr int LDX = VB + 4;     // X fp32          [C][LDX]
    static constexpr int LDA = C + 4;      // A fp32          [C][LDA]
    static constexpr int LDZ = C / 2 + PAD;  // Z^T           [C/2][LDZ]
    static constexpr int LDS_ = DK + PAD;  // S'^T            [VB][LDS_]
    // byte offsets
    static constexpr size_t oE = 0;
    static constexpr size_t oQ = oE + (size_t)C * LDE * TS;
    static constexpr size_t oK = oQ + (size_t)C * LDE * TS;
    static constexpr size_t oKT = oK + (size_t)C * LDE * TS;
    static constexpr size_t oX = oKT + (size_t)DK * LDC * TS;
    static constexpr size_t oG = oX + (size_t)C * LDX * 4;
    static constexpr size_t oTot = oG + (size_t)DK * 4;
    static constexpr size_t oA = oTot + (size_t)RGK * DK * 4;
    static constexpr size_t oTh = oA + (size_t)C * LDA * 4;
    static constexpr size_t oTT = oTh + (size_t)C * LDC * TS;
    static constexpr size_t oP = oTT + (size_t)C * LDC * TS;
    static constexpr size_t oZ = oP + (size_t)C * LDC * TS;
    static constexpr size_t oST = oZ + (size_t)(C / 2) * LDZ * TS;
    static constexpr size_t oRT = oST + (size_t)VB * LDS_ * TS;
    static constexpr size_t oUT = oRT + (size_t)VB * LDC * TS;
    static constexpr size_t bytes = oUT + (size_t)VB * LDC * TS;
};

constexpr size_t kMaxLds = 160 * 1024;
constexpr float kF16DecayLimit = 10.0f;   // e^10 * |b k| stays far below the f16 max
constexpr float kF32DecayLimit = 80.0f;

template <typename T>
__device__ __forceinline__ void st4(T* p, floatx4 v);
template <>
__device__ __forceinline__ void st4<_Float16>(_Float16* p, floatx4 v) {
    half4 h;
    h[0] = (_Float16)v[0]; h[1] = (_Float16)v[1]; h[2] = (_Float16)v[2]; h[3] = (_Float16)v[3];
    *reinterpret_cast<half4*>(p) = h;
}
template <>
__device__ __forceinline__ void st4<float>(float* p, floatx4 v) {
    *reinterpret_cast<floatx4*>(p) = v;
}

// Gate/decay loads that are either 4 channels or one per-token scalar.
template <bool F32>
__device__ __forceinline__ Raw4<F32> load_gate(const void* base, size_t idx4, size_t idx1, bool scalar) {
    if (!scalar) return load_raw4<F32>(base, idx4);
    // only element 0 is defined in scalar mode (cvt_gate broadcasts it); leaving the
    // rest unwritten keeps VALU writes out of registers with loads in flight
    Raw4<F32> r;
    if constexpr (F32) r.f[0] = reinterpret_cast<const float*>(base)[idx1];
    else r.u.x = reinterpret_cast<const uint16_t*>(base)[idx1];
    return r;
}
template <bool F32>
__device__ __forceinline__ floatx4 cvt_gate(const Raw4<F32>& r, bool scalar) {
    if (!scalar) return cvt_raw4<F32>(r);
    float x;
    if constexpr (F32) x = r.f[0];
    else x = __uint_as_float(r.u.x << 16);
    floatx4 f;
    f[0] = f[1] = f[2] = f[3] = x;
    return f;
}

__device__ __forceinline__ floatx4 exp4(floatx4 x) {
    floatx4 r;
    r[0] = __expf(x[0]); r[1] = __expf(x[1]); r[2] = __expf(x[2]); r[3] = __expf(x[3]);
    return r;
}

template <int DK, int DV, int C, int VB, bool F32>
__global__ __launch_bounds__(256, 1) void fwd_kernel(FwdParams p) {
    using L = FwdLayout<DK, DV, C, VB, F32>;
    using T = typename L::T;
    static_assert(L::bytes <= kMaxLds, "LDS budget");
    constexpr int NT = L::NT, NW = L::NW;
    constexpr int LDE = L::LDE, LDC = L::LDC, LDX = L::LDX, LDA = L::LDA, LDZ = L::LDZ,
                  LDS_ = L::LDS_;
    constexpr int NVB = DV / VB;
    constexpr int NB = C / 16;                         // 16-row blocks per chunk
    constexpr int NLT = NB * (NB + 1) / 2;             // lower 16x16 tiles
    constexpr int NNT = VB / 16;                       // 16-col tiles per value block
    constexpr int NST = (DK / 16) * NNT;               // state tiles
    constexpr int NSW = (NST + NW - 1) / NW;           // state tiles per wave
    constexpr int NWK = NW - 1;                        // "worker" waves for Y / O
    constexpr int NQT = NB * NNT;                      // output tiles per chunk
    constexpr int NQW = (NQT + NWK - 1) / NWK;
    constexpr int RPK = L::RPK, RGK = L::RGK, CQK = L::CQK;
    constexpr int RPV = L::RPV, RGV = L::RGV, CQV = L::CQV;

    extern __shared__ __align__(16) unsigned char smem[];
    T* sE = reinterpret_cast<T*>(smem + L::oE);
    T* sQ = reinterpret_cast<T*>(smem + L::oQ);
    T* sK = reinterpret_cast<T*>(smem + L::oK);
    T* sKT = reinterpret_cast<T*>(smem + L::oKT);
    float* sX = reinterpret_cast<float*>(smem + L::oX);
    float* sGam = reinterpret_cast<float*>(smem + L::oG);
    float* sTot = reinterpret_cast<float*>(smem + L::oTot);
    float* sA = reinterpret_cast<float*>(smem + L::oA);
    T* sTh = reinterpret_cast<T*>(smem + L::oTh);
    T* sTT = reinterpret_cast<T*>(smem + L::oTT);
    T* sP = reinterpret_cast<T*>(smem + L::oP);
    T* sZ = reinterpret_cast<T*>(smem + L::oZ);
    T* sST = reinterpret_cast<T*>(smem + L::oST);
    T* sRT = reinterpret_cast<T*>(smem + L::oRT);
    T* sUT = reinterpret_cast<T*>(smem + L::oUT);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int bh = lid / NVB, vb = lid % NVB;
    const int Tn = p.T, NC = Tn / C;
    const bool a_sc = (p.flags & GDR_ALPHA_SCALAR) != 0;
    const bool b_sc = (p.flags & GDR_B_SCALAR) != 0;
    const bool w_sc = (p.flags & GDR_W_SCALAR) != 0;
    const bool out_bf16 = (p.flags & GDR_OUT_BF16) != 0;
    const int n_l = lane & 15, m_l = 4 * (lane >> 4);
    constexpr float kDecayLimit = F32 ? kF32DecayLimit : kF16DecayLimit;
    bool poisoned = false;   // block-uniform

    // The strictly upper 16x16 tiles of T and P are zero and never written:
    // clear them once (in T^T they are the strictly lower tiles).
    for (int idx = tid; idx < C * C; idx += NT) {
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) {
            sTh[r * LDC + c] = (T)0.f;
            sP[r * LDC + c] = (T)0.f;
            sTT[c * LDC + r] = (T)0.f;
        }
    }

    // ---- state block in accumulators: tile s of this wave = (mt, nt)
    floatx4 Sacc[NSW];
#pragma unroll
    for (int s = 0; s < NSW; ++s) {
        Sacc[s] = zero4();
        const int tile = wave + s * NW;
        if (tile < NST && p.S0) {
            const int mt = tile / NNT, nt = tile % NNT;
            const size_t base = ((size_t)bh * DK + 16 * mt + m_l) * DV + vb * VB + 16 * nt + n_l;
#pragma unroll
            for (int i = 0; i < 4; ++i) Sacc[s][i] = p.S0[base + (size_t)i * DV];
        }
    }

    // ---- register prefetch of one chunk's inputs
    const int cq = tid % CQK, rg = tid / CQK;
    const bool kact = rg < RGK;
    const int cqv = tid % CQV, rgv = tid / CQV;
    const bool vact = rgv < RGV;
    Raw4<F32> rq[RPK], rk[RPK], rb[RPK];
    Raw4<true> rla[RPK];
    Raw4<F32> rv[RPV], rw[RPV];

    auto issue_loads = [&](int c) {
        if (kact) {
#pragma unroll
            for (int i = 0; i < RPK; ++i) {
                const size_t tok = (size_t)bh * Tn + (size_t)c * C + rg * RPK + i;
                const size_t ix = tok * DK + 4 * cq;
                rq[i] = load_raw4<F32>(p.q, ix);
                rk[i] = load_raw4<F32>(p.k, ix);
                rb[i] = load_gate<F32>(p.b, ix, tok, b_sc);
                rla[i] = load_gate<true>(p.la, ix, tok, a_sc);
            }
        }
        if (vact) {
#pragma unroll
            for (int i = 0; i < RPV; ++i) {
                const size_t tok = (size_t)bh * Tn + (size_t)c * C + rgv * RPV + i;
                const size_t ix = tok * DV + vb * VB + 4 * cqv;
                rv[i] = load_raw4<F32>(p.v, ix);
                rw[i] = load_gate<F32>(p.w, ix, tok, w_sc);
            }
        }
    };

    if (NC > 0) issue_loads(0);

    for (int c = 0; c < NC; ++c) {
        // ================= gate prep (fp32) =================
        floatx4 gl[RPK];
        if (kact) {
            floatx4 run = zero4();
#pragma unroll
            for (int i = 0; i < RPK; ++i) {
                run += cvt_gate<true>(rla[i], a_sc);
                gl[i] = run;
            }
            *reinterpret_cast<floatx4*>(sTot + rg * DK + 4 * cq) = run;
        }
        if (p.states) {  // chunk-start state snapshot for the backward pass
#pragma unroll
            for (int s = 0; s < NSW; ++s) {
                const int tile = wave + s * NW;
                if (tile < NST) {
                    const int mt = tile / NNT, nt = tile % NNT;
                    const size_t base = (((size_t)bh * NC + c) * DK + 16 * mt + m_l) * DV + vb * VB +
                                        16 * nt + n_l;
#pragma unroll
                    for (int i = 0; i < 4; ++i) p.states[base + (size_t)i * DV] = Sacc[s][i];
                }
            }
        }
        __syncthreads();
        int over = 0;
        if (kact) {
            floatx4 off = zero4(), gC = zero4();
#pragma unroll
            for (int g = 0; g < RGK; ++g) {
                const floatx4 t = *reinterpret_cast<const floatx4*>(sTot + g * DK + 4 * cq);
                if (g < rg) off += t;
                gC += t;
            }
            if (rg == 0) {
                *reinterpret_cast<floatx4*>(sGam + 4 * cq) = exp4(gC);
                const floatx4 span = gl[0] - gC;   // largest exponent g_0 - g_C of the chunk
                over = !(span[0] <= kDecayLimit && span[1] <= kDecayLimit &&
                         span[2] <= kDecayLimit && span[3] <= kDecayLimit);
            }
            T kt[4][RPK];
#pragma unroll
            for (int i = 0; i < RPK; ++i) {
                const int r = rg * RPK + i;
                const floatx4 g = off + gl[i];
                const floatx4 eg = exp4(g - gC);
                const floatx4 ek = exp4(gC - g);
                const floatx4 q4 = cvt_raw4<F32>(rq[i]);
                const floatx4 k4 = cvt_raw4<F32>(rk[i]);
                const floatx4 b4 = cvt_gate<F32>(rb[i], b_sc);
                const floatx4 kh = k4 * ek;
                st4<T>(sE + r * LDE + 4 * cq, b4 * k4 * eg);
                st4<T>(sQ + r * LDE + 4 * cq, q4 * eg);
                st4<T>(sK + r * LDE + 4 * cq, kh);
#pragma unroll
                for (int j = 0; j < 4; ++j) kt[j][i] = (T)kh[j];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < RPK; ++i) sKT[(4 * cq + j) * LDC + rg * RPK + i] = kt[j][i];
        }
        if (vact) {
#pragma unroll
            for (int i = 0; i < RPV; ++i) {
                const int r = rgv * RPV + i;
                const floatx4 x = cvt_gate<F32>(rw[i], w_sc) * cvt_raw4<F32>(rv[i]);
                *reinterpret_cast<floatx4*>(sX + r * LDX + 4 * cqv) = x;
            }
        }
        issue_loads(c + 1 < NC ? c + 1 : c);   // unconditional: loads land in the carried registers
        if (__syncthreads_or(over)) poisoned = true;

        // ================= A, P (MFMA) and S' =================
        for (int task = wave; task < 2 * NLT; task += NW) {
            const int which = task / NLT;
            int t = task % NLT, mt = 0;
            while (t > mt) { t -= mt + 1; ++mt; }
            const int nt = t;
            floatx4 acc = zero4();
            Mma<T>::run(acc, (which == 0 ? sE : sQ) + 16 * mt * LDE, LDE, sK + 16 * nt * LDE, LDE,
                        DK, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + m_l + i, col = 16 * nt + n_l;
                if (which == 0) sA[r * LDA + col] = (col < r) ? acc[i] : 0.f;
                else sP[r * LDC + col] = (T)((col <= r) ? acc[i] : 0.f);
            }
        }
#pragma unroll
        for (int s = 0; s < NSW; ++s) {
            const int tile = wave + s * NW;
            if (tile < NST) {
                const int mt = tile / NNT, nt = tile % NNT;
                const floatx4 gm = *reinterpret_cast<const floatx4*>(sGam + 16 * mt + m_l);
                Sacc[s] = Sacc[s] * gm;
                st4<T>(sST + (16 * nt + n_l) * LDS_ + 16 * mt + m_l, Sacc[s]);
            }
        }
        __syncthreads();

        // ====== diagonal blocks of T (wave 0)  ||  Y = [E; Qs] S' (other waves)
        floatx4 Yq[NQW];
        if (wave == 0) {
            const int R = lane >> 4, j = lane & 15;
            if (R < NB) {
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float s = (r == j) ? 1.f : 0.f;
                    const float* arow = sA + (16 * R + r) * LDA + 16 * R;
#pragma unroll
                    for (int m = 0; m < r; ++m) s -= arow[m] * x[m];
                    x[r] = s;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) sTh[(16 * R + r) * LDC + 16 * R + j] = (T)x[r];
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    floatx4 v;
                    v[0] = x[r]; v[1] = x[r + 1]; v[2] = x[r + 2]; v[3] = x[r + 3];
                    st4<T>(sTT + (16 * R + j) * LDC + 16 * R + r, v);
                }
            }
        } else {
            const int wk = wave - 1;
#pragma unroll
            for (int s = 0; s < NQW; ++s) {
                const int qt = wk + s * NWK;
                Yq[s] = zero4();
                if (qt < NQT) {
                    const int mt = qt / NNT, nt = qt % NNT;
                    // E part -> R = X - E S'  (stored transposed)
                    floatx4 acc = zero4();
                    Mma<T>::run(acc, sE + 16 * mt * LDE, LDE, sST + 16 * nt * LDS_, LDS_, DK, lane);
                    floatx4 rr;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        rr[i] = sX[(16 * mt + m_l + i) * LDX + 16 * nt + n_l] - acc[i];
                    st4<T>(sRT + (16 * nt + n_l) * LDC + 16 * mt + m_l, rr);
                    // Qs part, kept for the output
                    Mma<T>::run(Yq[s], sQ + 16 * mt * LDE, LDE, sST + 16 * nt * LDS_, LDS_, DK, lane);
                }
            }
        }
        __syncthreads();

        // ====== off-diagonal blocks of T by doubling: T_BA = -T_BB (A_BA T_AA)
#pragma unroll
        for (int s = 16; s < C; s *= 2) {
            const int nsub = s / 16;
            const int ntask = (C / (2 * s)) * nsub * nsub;
            for (int task = wave; task < ntask; task += NW) {
                const int pr = task / (nsub * nsub), mi = (task / nsub) % nsub, ni = task % nsub;
                const int a0 = 2 * s * pr, b0 = a0 + s;
                floatx4 acc = zero4();
                Mma<T>::run_xf32(acc, sA + (b0 + 16 * mi) * LDA + a0, LDA,
                                 sTT + (a0 + 16 * ni) * LDC + a0, LDC, s, lane);
                T* z = sZ + pr * s * LDZ;
                st4<T>(z + (16 * ni + n_l) * LDZ + 16 * mi + m_l, acc);
            }
            __syncthreads();
            for (int task = wave; task < ntask; task += NW) {
                const int pr = task / (nsub * nsub), mi = (task / nsub) % nsub, ni = task % nsub;
                const int a0 = 2 * s * pr, b0 = a0 + s;
                const T* z = sZ + pr * s * LDZ;
                floatx4 acc = zero4();
                Mma<T>::run(acc, sTh + (b0 + 16 * mi) * LDC + b0, LDC, z + 16 * ni * LDZ, LDZ, s, lane);
                acc = -acc;
                const int r0 = b0 + 16 * mi + m_l, cc = a0 + 16 * ni + n_l;
#pragma unroll
                for (int i = 0; i < 4; ++i) sTh[(r0 + i) * LDC + cc] = (T)acc[i];
                st4<T>(sTT + cc * LDC + r0, acc);
            }
            __syncthreads();
        }

        // ================= U = T R =================
        for (int task = wave; task < NQT; task += NW) {
            const int mt = task / NNT, nt = task % NNT;
            floatx4 acc = zero4();
            Mma<T>::run(acc, sTh + 16 * mt * LDC, LDC, sRT + 16 * nt * LDC, LDC, 16 * (mt + 1), lane);
            st4<T>(sUT + (16 * nt + n_l) * LDC + 16 * mt + m_l, acc);
        }
        __syncthreads();

        // ================= O = Qs S' + P U ;  S = S' + Kh^T U =================
        if (wave > 0 && p.o) {
            const int wk = wave - 1;
#pragma unroll
            for (int s = 0; s < NQW; ++s) {
                const int qt = wk + s * NWK;
                if (qt < NQT) {
                    const int mt = qt / NNT, nt = qt % NNT;
                    floatx4 acc = Yq[s];
                    Mma<T>::run(acc, sP + 16 * mt * LDC, LDC, sUT + 16 * nt * LDC, LDC, 16 * (mt + 1),
                                lane);
                    if (poisoned) acc[0] = acc[1] = acc[2] = acc[3] = __builtin_nanf("");
                    const size_t base = ((size_t)bh * Tn + (size_t)c * C + 16 * mt + m_l) * DV +
                                        vb * VB + 16 * nt + n_l;
                    if (out_bf16) {
                        uint16_t* o = reinterpret_cast<uint16_t*>(p.o);
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[base + (size_t)i * DV] = f32_to_bf16(acc[i]);
                    } else {
                        float* o = reinterpret_cast<float*>(p.o);
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[base + (size_t)i * DV] = acc[i];
                    }
                }
            }
        }
#pragma unroll
        for (int s = 0; s < NSW; ++s) {
            const int tile = wave + s * NW;
            if (tile < NST) {
                const int mt = tile / NNT, nt = tile % NNT;
                Mma<T>::run(Sacc[s], sKT + 16 * mt * LDC, LDC, sUT + 16 * nt * LDC, LDC, C, lane);
            }
        }
    }

    if (p.Sf) {
#pragma unroll
        for (int s = 0; s < NSW; ++s) {
            const int tile = wave + s * NW;
            if (tile < NST) {
                const int mt = tile / NNT, nt = tile % NNT;
                const size_t base = ((size_t)bh * DK + 16 * mt + m_l) * DV + vb * VB + 16 * nt + n_l;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.Sf[base + (size_t)i * DV] = poisoned ? __builtin_nanf("") : Sacc[s][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------

template <int DK, int DV, int C, bool F32>
constexpr int pick_vb() {
    return DV < 32 ? DV : 32;
}

template <int DK, int DV, int C, bool F32>
constexpr bool fits() {
    return FwdLayout<DK, DV, C, pick_vb<DK, DV, C, F32>(), F32>::bytes <= kMaxLds;
}

template <int DK, int DV, int C, bool F32>
static hipError_t launch_one(const FwdParams& p, hipStream_t st) {
    constexpr int VB = pick_vb<DK, DV, C, F32>();
    using L = FwdLayout<DK, DV, C, VB, F32>;
    auto kern = fwd_kernel<DK, DV, C, VB, F32>;
    static std::atomic<unsigned long long> done{0};
    const hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(kern), (int)L::bytes, done);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(p.BH * (DV / VB))), block(256);
    hipLaunchKernelGGL(kern, grid, block, L::bytes, st, p);
    return hipGetLastError();
}

// Chunk actually used: the requested one if its tiles fit in LDS, else the
// largest smaller one that does (fp32 operands at d_k >= 64 block with 32).
template <int DK, int DV, bool F32>
static int chunk_for(int chunk) {
    if (chunk >= 64 && fits<DK, DV, 64, F32>()) return 64;
    if (chunk >= 32 && fits<DK, DV, 32, F32>()) return 32;
    return 16;
}

template <int DK, int DV, bool F32>
static hipError_t launch_c(const FwdParams& p, int chunk, hipStream_t st, int* used) {
    const int c = chunk_for<DK, DV, F32>(chunk);
    if (used) *used = c;
    if (c == 64) {
        if constexpr (fits<DK, DV, 64, F32>()) return launch_one<DK, DV, 64, F32>(p, st);
    } else if (c == 32) {
        if constexpr (fits<DK, DV, 32, F32>()) return launch_one<DK, DV, 32, F32>(p, st);
    } else {
        return launch_one<DK, DV, 16, F32>(p, st);
    }
    return hipErrorInvalidValue;
}

template <int DK, int DV>
static hipError_t launch_d(const FwdParams& p, int chunk, hipStream_t st, int* used) {
    if (p.flags & GDR_ACT_F32) return launch_c<DK, DV, true>(p, chunk, st, used);
    return launch_c<DK, DV, false>(p, chunk, st, used);
}

static bool head_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool fwd_supported(int dk, int dv, int chunk, uint32_t flags) {
    (void)flags;
    return (chunk == 16 || chunk == 32 || chunk == 64) && head_ok(dk) && head_ok(dv);
}

template <int DK>
static hipError_t launch_dv(const FwdParams& p, int dv, int chunk, hipStream_t st, int* used) {
    switch (dv) {
        case 16: return launch_d<DK, 16>(p, chunk, st, used);
        case 32: return launch_d<DK, 32>(p, chunk, st, used);
        case 64: return launch_d<DK, 64>(p, chunk, st, used);
        case 128: return launch_d<DK, 128>(p, chunk, st, used);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdParams& p, int dk, int dv, int chunk, hipStream_t st, int* used) {
    if (!(p.flags & GDR_FWD_GENERIC) && fwd_pipe_supported(dk, dv, chunk, p.flags)) {
        if (used) *used = chunk;
        return launch_fwd_pipe(p, dk, dv, st);
    }
    switch (dk) {
        case 16: return launch_dv<16>(p, dv, chunk, st, used);
        case 32: return launch_dv<32>(p, dv, chunk, st, used);
        case 64: return launch_dv<64>(p, dv, chunk, st, used);
        case 128: return launch_dv<128>(p, dv, chunk, st, used);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
