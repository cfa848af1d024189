// Backward passes over the two-pass forward's records (bf16 activations,
// chunk 64, d_k = d_v in {64, 128}): the reverse chain that carries the
// gradient of the state backwards through the chunks, and the per-chunk
// gradients with separate erase and write gate gradients (the gate-aware
// accumulation of the Gated DeltaNet-2 Q&A page, Q4).  The reverse-mode
// formulas per chunk are those written out at the top of gdr_bwd.hip; here the
// triangular factors come from the forward's records instead of being rebuilt.
#include "gdr_device.h"
#include "gdr_launch.h"
#include "gdr_wy.h"

namespace gdr {

namespace wy {

// Reverse chain of the backward.  With the forward's chunk operands, the
// gradient of the chunk-start state follows from the gradient D of the
// chunk-end state as
//   diag(e^{g_C}) (D + Q̃^T dO - W^T (Kh D)),
// because the triangular solve of the reverse mode folds into W and Q̃
// (E^T T^T = W^T and Qs - P W = Q̃).  One workgroup of two waves per (head,
// 16-column strip): wave 0 carries D (Z = Kh D, D += F - W^T Z, D *= gamma)
// and stores every chunk-end gradient; wave 1 computes F = Q̃^T dO one chunk
// ahead (nothing on the chain depends on it) and publishes it in LDS.  Both
// prefetch their operands two chunks ahead.
template <int DK, int NK2>
struct DFrags {
    half8 kw[DK / 32][C / 16], wt[DK / 16][NK2];
    floatx4 gm[DK / 16];
    int flag;
};
template <int DK, int NK2>
struct FFrags {
    half8 qt[DK / 16][NK2];
    uint32_t dob[NK2][8];       // raw bf16 dO values (K = tokens)
};

template <int DK, int DV, bool VL>
__global__ __launch_bounds__(128, 1) void dchain_kernel(BwdParams p, const unsigned char* ws) {
    using R = Rec<DK, DV>;
    constexpr size_t RB = R::bwd_bytes;
    constexpr int NST = DV / 16, NKT = DK / 16, NKK = DK / 32, NB = C / 16, NK2 = C / 32;
    __shared__ __align__(16) floatx4 sF[2][NKT][64];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // chain bh (packed sequences: sequence bh / H of head bh % H, the longest
    // first) and its 16-column strip nt
    int bh, nt, NC, seq_len;
    size_t tok_base, chunk0;
    if constexpr (VL) {
        bh = packed_chain(p.seq_order, p.BH, NST, (int)blockIdx.x, (int)gridDim.x, nt);
        const PackedSpan sp = packed_span(p.cu_seqlens, p.chunk_off, p.nseq, p.BH, p.T, bh);
        NC = sp.NC;
        seq_len = sp.len;
        tok_base = sp.tok0;
        chunk0 = sp.chunk0;
    } else {
        const int lid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
        bh = lid / NST;
        nt = lid % NST;
        NC = p.T / C;
        seq_len = p.T;
        tok_base = (size_t)bh * p.T;
        chunk0 = (size_t)bh * NC;
    }
    const unsigned char* rec0 = ws + chunk0 * RB;
    const int n_l = lane & 15, g4 = 4 * (lane >> 4), col = 16 * nt + n_l;
    auto frag = [&](const unsigned char* rec, size_t off) __attribute__((always_inline)) {
        return *reinterpret_cast<const half8*>(rec + off + (size_t)lane * 16);
    };
    auto recp = [&](int c) __attribute__((always_inline)) {
        return rec0 + (size_t)(c < 0 ? 0 : c) * RB;
    };

    if (wave == 1) {
        // ------------------------------------------------ F = Q̃^T dO, one chunk ahead
        using F = FFrags<DK, NK2>;
        const uint16_t* dO = reinterpret_cast<const uint16_t*>(p.dO);
        auto fetch = [&](int c, F& f) __attribute__((always_inline)) {
            const int cc = c < 0 ? 0 : c;
            const unsigned char* rec = recp(cc);
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
                for (int kk = 0; kk < NK2; ++kk) f.qt[mt][kk] = frag(rec, R::QT + (size_t)(mt * NK2 + kk) * 1024);
            const size_t tok0 = tok_base + (size_t)cc * C;
#pragma unroll
            for (int kk = 0; kk < NK2; ++kk)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    // (packed sequences: rows past the sequence's end read as zero)
                    const int t = 32 * kk + (j < 4 ? g4 + j : 16 + g4 + j - 4);
                    const bool ok = !VL || cc * C + t < seq_len;
                    f.dob[kk][j] = dO[(tok0 + (ok ? t : 0)) * DV + col];
                    if (!ok) f.dob[kk][j] = 0;
                }
        };
        auto compute = [&](F& f, int buf) __attribute__((always_inline)) {
            half8 dof[NK2];
#pragma unroll
            for (int kk = 0; kk < NK2; ++kk)
#pragma unroll
                for (int j = 0; j < 8; ++j) dof[kk][j] = (_Float16)__uint_as_float(f.dob[kk][j] << 16);
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt) {
                floatx4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < NK2; ++kk) acc = mfma32(f.qt[mt][kk], dof[kk], acc);
                sF[buf][mt][lane] = acc;
            }
        };
        F fa, fb;
        if (NC > 0) {
            fetch(NC - 1, fa);
            fetch(NC - 2, fb);
            compute(fa, 0);
            fetch(NC - 3, fa);
        }
        // iteration j (chunk NC-1-j on wave 0) prepares chunk NC-2-j
        auto step = [&](int j, F& f) __attribute__((always_inline)) {
            lds_barrier();
            const int c = NC - 2 - j;
            if (c >= 0) {
                compute(f, (j + 1) & 1);
                fetch(c - 2, f);
            }
        };
        for (int j = 0; j < NC; j += 2) {
            step(j, fb);
            if (j + 1 < NC) step(j + 1, fa);
        }
        return;
    }

    // ---------------------------------------------------- wave 0: D, backwards
    using F = DFrags<DK, NK2>;
    floatx4 D[NKT];
#pragma unroll
    for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            D[mt][i] = p.dSf ? p.dSf[((size_t)bh * DK + 16 * mt + g4 + i) * DV + col] : 0.f;
    auto fetch_kg = [&](int c, F& f) __attribute__((always_inline)) {
        const unsigned char* rec = recp(c);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) f.kw[kk][rt] = frag(rec, R::KW + (size_t)(rt * NKK + kk) * 1024);
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt) f.gm[mt] = *reinterpret_cast<const floatx4*>(rec + R::G + (16 * mt + g4) * 4);
        f.flag = *reinterpret_cast<const int*>(rec + R::G + DK * 4);
    };
    auto fetch_w = [&](int c, F& f) __attribute__((always_inline)) {
        const unsigned char* rec = recp(c);
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
            for (int kk = 0; kk < NK2; ++kk) f.wt[mt][kk] = frag(rec, R::WT + (size_t)(mt * NK2 + kk) * 1024);
    };
    F fa, fb;
    if (NC > 0) {
        fetch_kg(NC - 1, fa); fetch_w(NC - 1, fa);
        fetch_kg(NC - 2, fb); fetch_w(NC - 2, fb);
    }
    bool poisoned = false;
    const float qnan = __builtin_nanf("");
    half8 nan8;
#pragma unroll
    for (int e = 0; e < 8; ++e) nan8[e] = (_Float16)qnan;
    auto step = [&](int j, F& f) __attribute__((always_inline)) {
        const int c = NC - 1 - j;
        // Z = Kh D; the f16 fragments of D are also the gradient kernel's copy of
        // this chunk's end-state gradient
        half8 df[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) df[kk] = cat8(to_h4(D[2 * kk]), to_h4(D[2 * kk + 1]));
        {
            using SFB = StateFrag<DK, DV>;
            unsigned char* dst = reinterpret_cast<unsigned char*>(p.dstate_frags) + (chunk0 + c) * SFB::bytes;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                *reinterpret_cast<half8*>(dst + SFB::block(nt, kk) + (size_t)lane * 16) = poisoned ? nan8 : df[kk];
        }
        if (f.flag) poisoned = true;
        floatx4 Z[NB];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) Z[rt] = zero4();
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) Z[rt] = mfma32(f.kw[kk][rt], df[kk], Z[rt]);
        lds_barrier();                                   // F of chunk c is published
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt) D[mt] += sF[j & 1][mt][lane];
        // D += -W^T Z, then D = diag(gamma) D
        half8 zf[NK2];
#pragma unroll
        for (int kk = 0; kk < NK2; ++kk) zf[kk] = cat8(to_h4(-Z[2 * kk]), to_h4(-Z[2 * kk + 1]));
#pragma unroll
        for (int kk = 0; kk < NK2; ++kk)
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt) D[mt] = mfma32(f.wt[mt][kk], zf[kk], D[mt]);
        const floatx4* gm = f.gm;
        floatx4 g2[NKT];
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt) g2[mt] = gm[mt];
        fetch_kg(c - 2, f);
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt) D[mt] = D[mt] * g2[mt];
        fetch_w(c - 2, f);
    };
    for (int j = 0; j < NC; j += 2) {
        step(j, fa);
        if (j + 1 < NC) step(j + 1, fb);
    }
    if (p.dS0) {
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p.dS0[((size_t)bh * DK + 16 * mt + g4 + i) * DV + col] = poisoned ? qnan : D[mt][i];
    }
}

template <int DK, int DV>
static hipError_t launch_dchain(const BwdParams& p, const void* ws, hipStream_t st) {
    const unsigned char* rec = reinterpret_cast<const unsigned char*>(ws);
    if (p.cu_seqlens) {
        hipLaunchKernelGGL((dchain_kernel<DK, DV, true>), dim3((unsigned)(p.nseq * p.BH * (DV / 16))), dim3(128), 0,
                           st, p, rec);
    } else {
        hipLaunchKernelGGL((dchain_kernel<DK, DV, false>), dim3((unsigned)(p.BH * (DV / 16))), dim3(128), 0, st, p,
                           rec);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-chunk gradients
// ---------------------------------------------------------------------------
// One workgroup of d/16 waves per chunk, all chunks in parallel.  Inputs: the
// chunk's record, its decayed start state S' and its end-state gradient D (f16
// fragments), dO and the activations.  With U = Ũ - W S', dU = Kh D + P^T dO and
// dR = T^T dU (the reverse of the triangular solve):
//   dP  = lower(dO U^T),        dA  = strict_lower(-dR U^T),
//   dQs = dO S'^T + dP Kh,       dE  = -dR S'^T + dA Kh,
//   dKh = U D^T + dA^T E + dP^T Qs,
// and the log-decay gradient dlog_alpha_t = Phi - sum_{r<t} dg_r with
// dg = dE ⊙ E + dQs ⊙ Qs - dKh ⊙ Kh and, per channel,
//   Phi = rowsum(dS' ⊙ S'),  dS' = D + Qs^T dO - E^T dR,
// computed as rowsum(D ⊙ S') + colsum(Qs ⊙ dO S'^T) - colsum(E ⊙ dR S'^T), so
// that dS' itself is never formed.
// Phase A gives each wave one 16-column value tile: U, dU, dR, and from dR the
// value-side gradients dv = dR ⊙ w, dw = dR ⊙ v.  The record fragments every
// wave reads there (W, Kh, P^T, T^T) are copied to LDS once per workgroup.  U,
// dR and dO go to LDS with tokens as rows.  Phases B and C give each wave one
// 16-channel tile: phase B the value reductions S' dO^T, S' dR^T and D U^T
// (channel x token accumulators), Phi, and the small dP and dA; phase C the
// token reductions and the element-wise gradients of q, k, b and log alpha.
// Register tiles change orientation on the MFMA unit (product with the
// identity), so no operand is gathered from LDS with strided scalar reads.
template <int D>
struct WgradLayout {
    static constexpr int LDX = D + 8;      // U, dR, dO: [C][LDX] f16, rows = tokens
    static constexpr int LDP = C + 8;      // dP, dA, their transposes: [C][LDP] f16
    static constexpr size_t oU = 0;
    static constexpr size_t oR = oU + (size_t)C * LDX * 2;
    static constexpr size_t oO = oR + (size_t)C * LDX * 2;
    static constexpr size_t endB = oO + (size_t)C * LDX * 2;
    static constexpr size_t oP = 0;                               // after phase B
    static constexpr size_t oA = oP + (size_t)C * LDP * 2;
    static constexpr size_t oPT = oA + (size_t)C * LDP * 2;
    static constexpr size_t oAT = oPT + (size_t)C * LDP * 2;
    static constexpr size_t endC = oAT + (size_t)C * LDP * 2;
    static constexpr int NW = D / 16;      // waves: one 16-column value tile (phase A) and
                                           // one 16-channel tile (phases B, C) each
    // the record's fragments every wave of phase A reads, copied once: W, Kh
    // (rows, K = channels), then P^T and T^T (rows, K = tokens)
    static constexpr size_t oFW = endB > endC ? endB : endC;
    static constexpr size_t oFK = oFW + (size_t)C * D * 2;
    static constexpr size_t oFT = oFK + (size_t)C * D * 2;        // P^T blocks, then T^T blocks
    static constexpr size_t endF = oFT + (size_t)2 * C * C * 2;
    // after phase A the same space holds S' and D with channels as rows (phase B's
    // operands, K = value columns): [D][LDS] f16 each
    static constexpr int LDS = D + 8;
    static constexpr size_t oSr = oFW;
    static constexpr size_t oDr = oSr + (size_t)D * LDS * 2;
    static constexpr size_t endS = oDr + (size_t)D * LDS * 2;
    static constexpr size_t oRed = endF > endS ? endF : endS;     // [3][NW][C] fp32
    static constexpr size_t oPhi = oRed + (size_t)3 * NW * C * 4; // [NW] fp32
    static constexpr size_t bytes = oPhi + (size_t)NW * 4;
};

__device__ __forceinline__ half4 bf16x4_to_h4(uint2 u) {
    half4 h;
    h[0] = (_Float16)__uint_as_float(u.x << 16);
    h[1] = (_Float16)__uint_as_float(u.x & 0xffff0000u);
    h[2] = (_Float16)__uint_as_float(u.y << 16);
    h[3] = (_Float16)__uint_as_float(u.y & 0xffff0000u);
    return h;
}
__device__ __forceinline__ float hsum4(floatx4 v) { return (v[0] + v[1]) + (v[2] + v[3]); }
__device__ __forceinline__ floatx4 splat4(float x) {
    floatx4 f;
    f[0] = f[1] = f[2] = f[3] = x;
    return f;
}
// Cross-lane moves within the 16-lane rows of a wave (DPP; lanes whose source
// falls outside the row read 0).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// inclusive prefix sum over the 16 lanes of each row (lane & 15 order)
__device__ __forceinline__ floatx4 scan16(floatx4 x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = x[i];
        v += dpp<0x111>(v);     // row_shr:1
        v += dpp<0x112>(v);     // row_shr:2
        v += dpp<0x114>(v);     // row_shr:4
        v += dpp<0x118>(v);     // row_shr:8
        x[i] = v;
    }
    return x;
}
// sum over the 16 lanes of each row, the same bits in every lane
__device__ __forceinline__ floatx4 rowsum16(floatx4 x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float v = x[i];
        v += dpp<0xB1>(v);      // quad_perm [1,0,3,2]
        v += dpp<0x4E>(v);      // quad_perm [2,3,0,1]
        v += dpp<0x141>(v);     // row_half_mirror
        v += dpp<0x140>(v);     // row_mirror
        x[i] = v;
    }
    return x;
}
__device__ __forceinline__ floatx4 expv4(floatx4 x) {
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __expf(x[i]);
    return r;
}

// g - g_C for the four channels 4g..4g+3 of a 16-channel tile (or the scalar
// decay) at tokens 16 tt + r, tt < 4, from log alpha at those positions: the
// in-chunk prefix over the lanes of each row and across the four token tiles
__device__ __forceinline__ void chunk_decay(const floatx4 (&la)[4], floatx4 (&gm)[4]) {
    floatx4 carry = zero4();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        gm[tt] = scan16(la[tt]) + carry;
        carry += rowsum16(la[tt]);
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) gm[tt] -= carry;
}

template <int D, bool AS, bool BS, bool WS, bool VL, bool LG>
__global__ __launch_bounds__(D * 4, 1) void wgrad_kernel(BwdParams p, const unsigned char* ws) {
    using R = Rec<D, D>;
    using SFB = StateFrag<D, D>;
    using L = WgradLayout<D>;
    constexpr size_t RB = R::bwd_bytes;
    constexpr int NW = L::NW, NKK = D / 32, NB = C / 16, NK2 = C / 32;
    constexpr int LDX = L::LDX, LDP = L::LDP;
    static_assert(NW * 16 == D && L::bytes <= 160 * 1024, "layout");
    extern __shared__ __align__(16) unsigned char smem[];
    _Float16* sU = reinterpret_cast<_Float16*>(smem + L::oU);
    _Float16* sR = reinterpret_cast<_Float16*>(smem + L::oR);
    _Float16* sO = reinterpret_cast<_Float16*>(smem + L::oO);
    _Float16* sP = reinterpret_cast<_Float16*>(smem + L::oP);
    _Float16* sA = reinterpret_cast<_Float16*>(smem + L::oA);
    _Float16* sPT = reinterpret_cast<_Float16*>(smem + L::oPT);
    _Float16* sAT = reinterpret_cast<_Float16*>(smem + L::oAT);
    float* sRed = reinterpret_cast<float*>(smem + L::oRed);
    float* sPhi = reinterpret_cast<float*>(smem + L::oPhi);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = 4 * (lane >> 4);
    // this workgroup's chunk: its record/fragment index, first token and length
    // (packed sequences: chunk r of head h from the chunk table; rows past the
    // sequence's end load as zeros and store nothing)
    size_t chunk, tok0;
    int len;
    if constexpr (VL) {
        const int CN = p.chunk_off[p.nseq];
        const int idx = (int)blockIdx.x;
        if (idx >= p.BH * CN) return;                // grid sized for the largest chunk count
        const int h = idx / CN, r = idx - h * CN;
        const int2 e = reinterpret_cast<const int2*>(p.chunk_tab)[r];
        chunk = (size_t)h * CN + r;
        tok0 = (size_t)h * p.T + (size_t)e.x;
        len = e.y;
    } else {
        const int NC = p.T / C;
        const int bh = (int)blockIdx.x / NC, c = (int)blockIdx.x % NC;
        chunk = (size_t)bh * NC + c;
        tok0 = (size_t)bh * p.T + (size_t)c * C;
        len = C;
    }
    const unsigned char* rec = ws + chunk * RB;
    const unsigned char* sfr = reinterpret_cast<const unsigned char*>(p.state_frags) + chunk * SFB::bytes;
    const unsigned char* dfr = reinterpret_cast<const unsigned char*>(p.dstate_frags) + chunk * SFB::bytes;
    // chunk bases (uniform) and 32-bit lane offsets keep the addresses in scalar registers
    const size_t ea = tok0 * D;                                  // element offset, [T][D] tensors
    const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q) + ea;
    const uint16_t* kg = reinterpret_cast<const uint16_t*>(p.k) + ea;
    const uint16_t* bg = reinterpret_cast<const uint16_t*>(p.b) + (BS ? tok0 : ea);
    const uint16_t* vg = reinterpret_cast<const uint16_t*>(p.v) + ea;
    const uint16_t* wg = reinterpret_cast<const uint16_t*>(p.w) + (WS ? tok0 : ea);
    const uint16_t* og = reinterpret_cast<const uint16_t*>(p.dO) + ea;
    const float* lag = p.la + (AS ? tok0 : ea);
    float* dqg = p.dq + ea;
    float* dkg = p.dk + ea;
    float* dvg = p.dv + ea;
    float* dbg = p.db + (BS ? tok0 : ea);
    float* dwg = p.dw + (WS ? tok0 : ea);
    float* dlag = p.dla + (AS ? tok0 : ea);
    const half4 id = ident4(lane);
    const int lo16 = lane * 16;
    auto frag = [&](const unsigned char* base, size_t off) __attribute__((always_inline)) {
        return *reinterpret_cast<const half8*>(base + off + lo16);
    };
    const float poison = *reinterpret_cast<const int*>(rec + R::G + D * 4) ? __builtin_nanf("") : 0.f;
    // gates given as logits (LG, GDR_GATE_LOGITS): the values are sigmoid / log
    // sigmoid of the inputs, the gate gradients are those of the logits (absent
    // tokens: decay logit +inf)
    constexpr bool lg = LG;
    auto gate4 = [&](floatx4 x) __attribute__((always_inline)) {
        if (lg) {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = gate_sigmoid(x[i]);
        }
        return x;
    };

    // ================= phase A: value columns 16 vt .. 16 vt + 15 (vt = wave), all tokens
    const int vt = wave, ct = wave;
    // Every load of the phase is issued before the first wait: the shared
    // fragments (copied into LDS, 16-byte pieces in record order) first, so
    // that waiting for them leaves the later loads in flight.
    constexpr int PW = C * D * 2 / 16, PT2 = 2 * C * C * 2 / 16, NPC = 2 * PW + PT2;
    constexpr int PER = (NPC + 64 * NW - 1) / (64 * NW);
    uint4 cp[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int pc = min(tid + 64 * NW * m, NPC - 1);
        const size_t src = pc < PW ? R::W + (size_t)pc * 16
                         : pc < 2 * PW ? R::KW + (size_t)(pc - PW) * 16 : R::PT + (size_t)(pc - 2 * PW) * 16;
        cp[m] = *reinterpret_cast<const uint4*>(rec + src);
    }
    // inputs needed late in this phase: v and w for dv, dw; dO
    uint2 vr[NB], wr[NB], dor[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
        const int t0 = 16 * rt + r16;
        const bool ok = !VL || t0 < len;
        const int t = ok ? t0 : 0, ix = t * D + 16 * vt + g4;
        vr[rt] = *reinterpret_cast<const uint2*>(vg + ix);
        if constexpr (WS) wr[rt].x = wg[t];
        else wr[rt] = *reinterpret_cast<const uint2*>(wg + ix);
        dor[rt] = *reinterpret_cast<const uint2*>(og + ix);
        if (!ok) vr[rt] = wr[rt] = dor[rt] = make_uint2(0u, 0u);
    }
    // Ũ (this wave's value tile) and the state fragments of the channel loop
    half8 fur[NK2], fsa[NKK], fda[NKK];
#pragma unroll
    for (int kk = 0; kk < NK2; ++kk) fur[kk] = frag(rec, R::U + (size_t)(vt * NK2 + kk) * 1024);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        fsa[kk] = frag(sfr, SFB::block(vt, kk));
        fda[kk] = frag(dfr, SFB::block(vt, kk));
    }
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int pc = tid + 64 * NW * m;
        if (NPC % (64 * NW) == 0 || pc < NPC) *reinterpret_cast<uint4*>(smem + L::oFW + (size_t)pc * 16) = cp[m];
    }
    auto lfrag = [&](size_t off) __attribute__((always_inline)) {
        return *reinterpret_cast<const half8*>(smem + off + lo16);
    };
    lds_barrier();
    // Y = W S' and Z = Kh D over the channels
    floatx4 Y[NB], Z[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) Y[rt] = Z[rt] = zero4();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
            Y[rt] = mfma32(lfrag(L::oFW + (size_t)(rt * NKK + kk) * 1024), fsa[kk], Y[rt]);
            Z[rt] = mfma32(lfrag(L::oFK + (size_t)(rt * NKK + kk) * 1024), fda[kk], Z[rt]);
        }
    }
    // dO: rows to LDS, and columns (K = tokens) for P^T dO
    half8 dov[NK2];
    {
        floatx4 tq[NB];
#pragma unroll
        for (int st = 0; st < NB; ++st) {
            const half4 h = bf16x4_to_h4(dor[st]);
            *reinterpret_cast<half4*>(sO + (16 * st + r16) * LDX + 16 * vt + g4) = h;
            tq[st] = swap16(h, id);
        }
#pragma unroll
        for (int kk = 0; kk < NK2; ++kk) dov[kk] = cat8(to_h4(tq[2 * kk]), to_h4(tq[2 * kk + 1]));
    }
    // dU = Kh D + P^T dO  (P^T blocks left of the diagonal pair are zero)
#pragma unroll
    for (int rt = 0; rt < NB; ++rt)
#pragma unroll
        for (int kk = rt / 2; kk < NK2; ++kk)
            Z[rt] = mfma32(lfrag(L::oFT + (size_t)(rt * NK2 + kk) * 1024), dov[kk], Z[rt]);
    // dR = T^T dU
    half8 duf[NK2];
#pragma unroll
    for (int kk = 0; kk < NK2; ++kk) duf[kk] = cat8(to_h4(Z[2 * kk]), to_h4(Z[2 * kk + 1]));
    floatx4 dR[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
        dR[rt] = zero4();
#pragma unroll
        for (int kk = rt / 2; kk < NK2; ++kk)
            dR[rt] = mfma32(lfrag(L::oFT + (size_t)(NB * NK2 + rt * NK2 + kk) * 1024), duf[kk], dR[rt]);
    }
    // U = Ũ - W S'  -> LDS rows (tokens)
#pragma unroll
    for (int kk = 0; kk < NK2; ++kk) {
        const half8 ur = fur[kk];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int rt = 2 * kk + h;
            const floatx4 u = f4(h ? hi4(ur) : lo4(ur)) - Y[rt];
            *reinterpret_cast<half4*>(sU + (16 * rt + r16) * LDX + 16 * vt + g4) = to_h4(swap16(to_h4(u), id));
        }
    }
    // dR -> LDS rows; dv = dR ⊙ w and dw = dR ⊙ v from the row layout (fp32:
    // the transposed f16 value plus the transposed f16 remainder)
    float dwp[NB];
#pragma unroll
    for (int rt = 0; rt < NB; ++rt) {
        const half4 hi = to_h4(dR[rt]);
        const floatx4 t1 = swap16(hi, id);
        *reinterpret_cast<half4*>(sR + (16 * rt + r16) * LDX + 16 * vt + g4) = to_h4(t1);
        const floatx4 x = mfma16(to_h4(dR[rt] - f4(hi)), id, t1);
        const int ix = (16 * rt + r16) * D + 16 * vt + g4;
        const bool ok = !VL || 16 * rt + r16 < len;
        const floatx4 v4 = cvt_raw4<false>(Raw4<false>{vr[rt]});
        const floatx4 w4 = gate4(WS ? splat4(bf16_to_f32((uint16_t)wr[rt].x)) : cvt_raw4<false>(Raw4<false>{wr[rt]}));
        if (ok) *reinterpret_cast<floatx4*>(dvg + ix) = x * w4 + poison;
        if constexpr (WS) dwp[rt] = hsum4(x * v4);
        else if (ok) *reinterpret_cast<floatx4*>(dwg + ix) = x * v4 * (lg ? w4 * (1.f - w4) : splat4(1.f)) + poison;
    }
    if constexpr (WS) {
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
            float v = dwp[rt];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if (g4 == 0) sRed[(0 * NW + wave) * C + 16 * rt + r16] = v;
        }
    }
    // the element-wise inputs of this wave's channels (16 ct .. 16 ct + 15), loaded
    // now and kept to the end
    floatx4 lar[NB];
    uint2 qr[NB], kr[NB], brw[NB];
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
        const int t0 = 16 * tt + r16;
        const bool ok = !VL || t0 < len;
        const int t = ok ? t0 : 0, ix = t * D + 16 * ct + g4;
        lar[tt] = AS ? splat4(lag[t]) : *reinterpret_cast<const floatx4*>(lag + ix);
        qr[tt] = *reinterpret_cast<const uint2*>(qg + ix);
        kr[tt] = *reinterpret_cast<const uint2*>(kg + ix);
        if constexpr (BS) brw[tt].x = bg[t];
        else brw[tt] = *reinterpret_cast<const uint2*>(bg + ix);
        if (!ok) {
            lar[tt] = splat4(lg ? __builtin_inff() : 0.f);
            qr[tt] = kr[tt] = brw[tt] = make_uint2(0u, 0u);
        }
    }
    lds_barrier();
    // S' and D (this wave's value tile, all channels) into LDS with channels as
    // rows, for phase B's value reductions (the shared fragments are dead now)
    {
        _Float16* sSr = reinterpret_cast<_Float16*>(smem + L::oSr);
        _Float16* sDr = reinterpret_cast<_Float16*>(smem + L::oDr);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int off = (32 * kk + 16 * h + r16) * L::LDS + 16 * vt + g4;
                *reinterpret_cast<half4*>(sSr + off) = to_h4(swap16(h ? hi4(fsa[kk]) : lo4(fsa[kk]), id));
                *reinterpret_cast<half4*>(sDr + off) = to_h4(swap16(h ? hi4(fda[kk]) : lo4(fda[kk]), id));
            }
    }
    lds_barrier();

    // ================= phase B: channels 16 ct .. 16 ct + 15, all tokens
    // Per 32-column step kv: S' and D with K = value columns (their rows, from
    // LDS), rowsum(D ⊙ S'), and
    // A1 = S' dO^T, A2 = S' dR^T, A3 = D U^T  (rows = channels, columns = tokens)
    floatx4 A1[NB], A2[NB], A3[NB];
    float phd = 0.f;
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) A1[tt] = A2[tt] = A3[tt] = zero4();
    {
        const _Float16* sSr = reinterpret_cast<const _Float16*>(smem + L::oSr) + (16 * ct + r16) * L::LDS + g4;
        const _Float16* sDr = reinterpret_cast<const _Float16*>(smem + L::oDr) + (16 * ct + r16) * L::LDS + g4;
#pragma unroll
        for (int kv = 0; kv < NKK; ++kv) {
            // S'[16ct + r][32kv + 4g + i] and [.. + 16 + ..], likewise D
            const half8 sc = cat8(ld_h4(sSr + 32 * kv), ld_h4(sSr + 32 * kv + 16));
            const half8 dc = cat8(ld_h4(sDr + 32 * kv), ld_h4(sDr + 32 * kv + 16));
#pragma unroll
            for (int e = 0; e < 8; ++e) phd += (float)sc[e] * (float)dc[e];
#pragma unroll
            for (int tt = 0; tt < NB; ++tt) {
                const int off = (16 * tt + r16) * LDX + 32 * kv + g4;
                A1[tt] = mfma32(sc, cat8(ld_h4(sO + off), ld_h4(sO + off + 16)), A1[tt]);
                A2[tt] = mfma32(sc, cat8(ld_h4(sR + off), ld_h4(sR + off + 16)), A2[tt]);
                A3[tt] = mfma32(dc, cat8(ld_h4(sU + off), ld_h4(sU + off + 16)), A3[tt]);
            }
        }
    }
    // dP^T and dA^T tiles (s-tile st <= t-tile tt): Res[s][t] = sum_v U[s][v] X[t][v]
    // with X = dO (dP) or dR (-dA); twenty tiles over the waves
    constexpr int NPA = 2 * NB * (NB + 1) / 2, PAW = (NPA + NW - 1) / NW;
    auto pa_tile = [&](int it, int& kind, int& st, int& tt) __attribute__((always_inline)) {
        kind = it / (NPA / 2);
        int t = it % (NPA / 2);
        tt = 0;
        while (t > tt) { t -= tt + 1; ++tt; }
        st = t;
    };
    floatx4 pa[PAW];
#pragma unroll
    for (int m = 0; m < PAW; ++m) {
        pa[m] = zero4();
        const int it = wave + NW * m;
        if (it >= NPA) break;
        int kind, st, tt;
        pa_tile(it, kind, st, tt);
        const _Float16* xs = kind ? sR : sO;
#pragma unroll
        for (int kv = 0; kv < NKK; ++kv) {
            const int ou = (16 * st + r16) * LDX + 32 * kv + g4, ox = (16 * tt + r16) * LDX + 32 * kv + g4;
            pa[m] = mfma32(cat8(ld_h4(sU + ou), ld_h4(sU + ou + 16)), cat8(ld_h4(xs + ox), ld_h4(xs + ox + 16)), pa[m]);
        }
    }
    lds_barrier();          // U, dR, dO are no longer read: their space takes dP and dA

    // dP, dA (rows = t) and their transposes (rows = s); strict/inclusive masks on
    // the diagonal tiles; tiles beyond the diagonal are zero
#pragma unroll
    for (int m = 0; m < PAW; ++m) {
        const int it = wave + NW * m;
        if (it >= NPA) break;
        int kind, st, tt;
        pa_tile(it, kind, st, tt);
        floatx4 v = pa[m];
        if (st == tt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool keep = kind ? (g4 + i < r16) : (g4 + i <= r16);
                v[i] = keep ? v[i] : 0.f;
            }
        }
        const half4 hv = to_h4(v);
        _Float16* rows = kind ? sA : sP;
        _Float16* cols = kind ? sAT : sPT;
        *reinterpret_cast<half4*>(rows + (16 * tt + r16) * LDP + 16 * st + g4) = hv;
        *reinterpret_cast<half4*>(cols + (16 * st + r16) * LDP + 16 * tt + g4) = to_h4(swap16(hv, id));
    }
    {
        const half4 z4 = to_h4(zero4());
        for (int idx = tid; idx < 6 * 16 * 4 * 4; idx += 64 * NW) {
            const int mtx = idx & 3, q = (idx >> 2) & 3, row = (idx >> 4) & 15, pr = idx >> 8;
            const int a = pr < 3 ? 0 : (pr < 5 ? 1 : 2);
            const int b = pr < 3 ? pr + 1 : (pr < 5 ? pr - 1 : 3);
            _Float16* base = mtx == 0 ? sP : mtx == 1 ? sA : mtx == 2 ? sPT : sAT;
            const int rt = mtx < 2 ? a : b, cb = mtx < 2 ? b : a;
            *reinterpret_cast<half4*>(base + (16 * rt + row) * LDP + 16 * cb + 4 * q) = z4;
        }
    }
    // element-wise part, lane (r, g): token 16 tt + r, channels 16 ct + 4g .. +3:
    // g - g_C, E, Qs, Kh, Phi, and the channel-row fragments of -E, Qs and Kh (K = tokens)
    floatx4 gm[NB];
    if (lg) {
        // decay logits -> log alpha (kept: the chain rule below needs it)
#pragma unroll
        for (int tt = 0; tt < NB; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) lar[tt][i] = gate_log_sigmoid(lar[tt][i]);
    }
    chunk_decay(lar, gm);
    half8 ef[NK2], qf[NK2], kf[NK2];
    floatx4 phi;
    {
        floatx4 p2 = zero4(), eT[NB], qT[NB], kT[NB];
#pragma unroll
        for (int tt = 0; tt < NB; ++tt) {
            const floatx4 eg = expv4(gm[tt]);
            const floatx4 q4 = cvt_raw4<false>(Raw4<false>{qr[tt]}), k4 = cvt_raw4<false>(Raw4<false>{kr[tt]});
            const floatx4 b4 = gate4(BS ? splat4(bf16_to_f32((uint16_t)brw[tt].x)) : cvt_raw4<false>(Raw4<false>{brw[tt]}));
            const floatx4 E = b4 * k4 * eg, Qs = q4 * eg, Kh = k4 * expv4(-gm[tt]);
            p2 += Qs * A1[tt] - E * A2[tt];
            eT[tt] = swap16(to_h4(-E), id);     // -E: the dA tiles hold -dA
            qT[tt] = swap16(to_h4(Qs), id);
            kT[tt] = swap16(to_h4(Kh), id);
        }
#pragma unroll
        for (int kk = 0; kk < NK2; ++kk) {
            ef[kk] = cat8(to_h4(eT[2 * kk]), to_h4(eT[2 * kk + 1]));
            qf[kk] = cat8(to_h4(qT[2 * kk]), to_h4(qT[2 * kk + 1]));
            kf[kk] = cat8(to_h4(kT[2 * kk]), to_h4(kT[2 * kk + 1]));
        }
        // Phi: the token sum over the lanes of a row, plus rowsum(D ⊙ S') (per
        // channel r in every lane group after the cross-group sum)
        p2 = rowsum16(p2);
        float pd = phd;
        pd += __shfl_xor(pd, 16, 64);
        pd += __shfl_xor(pd, 32, 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) phi[i] = p2[i] + __shfl(pd, g4 + i, 64);
    }
    lds_barrier();

    // ================= phase C: token reductions
    //   A1 += Kh^T-rows dP,   A2 += Kh^T-rows (-dA)   (so dE = -A2),
    //   A3 += (-E) (-dA)^T + Qs dP^T   (dKh)
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
        const int row = (16 * tt + r16) * LDP + g4;
#pragma unroll
        for (int kk = 0; kk < NK2; ++kk) {
            if (2 * kk <= tt) {
                A1[tt] = mfma32(kf[kk], cat8(ld_h4(sP + row + 32 * kk), ld_h4(sP + row + 32 * kk + 16)), A1[tt]);
                A2[tt] = mfma32(kf[kk], cat8(ld_h4(sA + row + 32 * kk), ld_h4(sA + row + 32 * kk + 16)), A2[tt]);
            }
            if (2 * kk + 1 >= tt) {
                A3[tt] = mfma32(ef[kk], cat8(ld_h4(sAT + row + 32 * kk), ld_h4(sAT + row + 32 * kk + 16)), A3[tt]);
                A3[tt] = mfma32(qf[kk], cat8(ld_h4(sPT + row + 32 * kk), ld_h4(sPT + row + 32 * kk + 16)), A3[tt]);
            }
        }
    }

    // element-wise gradients; lane (r, g): token 16 tt + r, channels 16 ct + 4g .. +3
    float dbs[NB], dgs[NB];
    floatx4 carry = zero4();
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
        const int ix = (16 * tt + r16) * D + 16 * ct + g4;
        const bool ok = !VL || 16 * tt + r16 < len;
        const floatx4 eg = expv4(gm[tt]), ek = expv4(-gm[tt]);
        const floatx4 q4 = cvt_raw4<false>(Raw4<false>{qr[tt]}), k4 = cvt_raw4<false>(Raw4<false>{kr[tt]});
        const floatx4 b4 = gate4(BS ? splat4(bf16_to_f32((uint16_t)brw[tt].x)) : cvt_raw4<false>(Raw4<false>{brw[tt]}));
        const floatx4 dQs = A1[tt], dE = -A2[tt], dKh = A3[tt];
        if (ok) {
            *reinterpret_cast<floatx4*>(dqg + ix) = dQs * eg + poison;
            *reinterpret_cast<floatx4*>(dkg + ix) = dE * b4 * eg + dKh * ek + poison;
        }
        const floatx4 dbv = dE * k4 * eg;
        if constexpr (BS) dbs[tt] = hsum4(dbv);
        else if (ok) *reinterpret_cast<floatx4*>(dbg + ix) = dbv * (lg ? b4 * (1.f - b4) : splat4(1.f)) + poison;
        const floatx4 dg = dE * (b4 * k4 * eg) + dQs * (q4 * eg) - dKh * (k4 * ek);
        if constexpr (AS) {
            dgs[tt] = hsum4(dg);
        } else {
            // d log alpha = Phi - (exclusive prefix of dg over the tokens)
            floatx4 dla = phi - (carry + (scan16(dg) - dg)) + poison;
            if (lg) {
                // d/da log sigmoid(a) = sigmoid(-a) = 1 - alpha = -expm1(log alpha)
#pragma unroll
                for (int i = 0; i < 4; ++i) dla[i] *= -expm1f(lar[tt][i]);
            }
            if (ok) *reinterpret_cast<floatx4*>(dlag + ix) = dla;
            carry += rowsum16(dg);
        }
    }
    if constexpr (AS || BS) {
#pragma unroll
        for (int tt = 0; tt < NB; ++tt) {
            float vb = BS ? dbs[tt] : 0.f, vg2 = AS ? dgs[tt] : 0.f;
            vb += __shfl_xor(vb, 16, 64);
            vb += __shfl_xor(vb, 32, 64);
            vg2 += __shfl_xor(vg2, 16, 64);
            vg2 += __shfl_xor(vg2, 32, 64);
            if (g4 == 0) {
                sRed[(1 * NW + wave) * C + 16 * tt + r16] = vb;
                sRed[(2 * NW + wave) * C + 16 * tt + r16] = vg2;
            }
        }
        // Phi summed over this wave's channels (each lane group holds the same sums)
        if constexpr (AS) {
            float v = hsum4(phi);
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if (lane == 0) sPhi[wave] = v;
        }
    }
    if constexpr (AS || BS || WS) {
        lds_barrier();
        if (wave == 0) {
            const int t = lane;      // C == 64 tokens, one per lane
            auto wsum = [&](int which) __attribute__((always_inline)) {
                float a = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) a += sRed[(which * NW + w) * C + t];
                return a;
            };
            const bool ok = !VL || t < len;
            // logits: the per-token gate's own value for the chain rule (absent
            // tokens are not stored; their index is clamped into the chunk)
            auto dsig = [&](const uint16_t* g) __attribute__((always_inline)) {
                if (!lg) return 1.f;
                const float x = gate_sigmoid(bf16_to_f32(g[ok ? t : 0]));
                return x * (1.f - x);
            };
            if constexpr (WS) {
                const float v = wsum(0) * dsig(wg) + poison;
                if (ok) dwg[t] = v;
            }
            if constexpr (BS) {
                const float v = wsum(1) * dsig(bg) + poison;
                if (ok) dbg[t] = v;
            }
            if constexpr (AS) {
                const float dg = wsum(2);
                float incl = dg;
#pragma unroll
                for (int d = 1; d < 64; d *= 2) {
                    const float u = __shfl_up(incl, d, 64);
                    if (t >= d) incl += u;
                }
                float ptot = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) ptot += sPhi[w];
                float f = 1.f;
                if (lg) f = -expm1f(gate_log_sigmoid(lag[ok ? t : 0]));
                if (ok) dlag[t] = (ptot - (incl - dg)) * f + poison;
            }
        }
    }
}

template <int D, bool AS, bool BS, bool WS, bool VL, bool LG>
static hipError_t launch_wgrad_v(const BwdParams& p, const void* ws, hipStream_t st) {
    auto k = wgrad_kernel<D, AS, BS, WS, VL, LG>;
    static std::atomic<unsigned long long> done{0};
    const hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(k), (int)WgradLayout<D>::bytes, done);
    if (e != hipSuccess) return e;
    // packed sequences: the chunk count is on the device; the grid covers the
    // largest possible count and the workgroups past the real one return at once
    const size_t items = VL ? (size_t)p.BH * packed_max_chunks(p.T, p.nseq) : (size_t)p.BH * (p.T / C);
    hipLaunchKernelGGL(k, dim3((unsigned)items), dim3(D * 4), WgradLayout<D>::bytes, st, p,
                       reinterpret_cast<const unsigned char*>(ws));
    return hipGetLastError();
}

template <int D, bool AS, bool BS, bool WS, bool LG>
static hipError_t launch_wgrad_l(const BwdParams& p, const void* ws, hipStream_t st) {
    return p.cu_seqlens ? launch_wgrad_v<D, AS, BS, WS, true, LG>(p, ws, st)
                        : launch_wgrad_v<D, AS, BS, WS, false, LG>(p, ws, st);
}

template <int D, bool AS, bool BS, bool WS>
static hipError_t launch_wgrad_t(const BwdParams& p, const void* ws, hipStream_t st) {
    return (p.flags & GDR_GATE_LOGITS) ? launch_wgrad_l<D, AS, BS, WS, true>(p, ws, st)
                                       : launch_wgrad_l<D, AS, BS, WS, false>(p, ws, st);
}

template <int D>
static hipError_t launch_wgrad(const BwdParams& p, const void* ws, hipStream_t st) {
    const int m = ((p.flags & GDR_ALPHA_SCALAR) ? 4 : 0) | ((p.flags & GDR_B_SCALAR) ? 2 : 0) |
                  ((p.flags & GDR_W_SCALAR) ? 1 : 0);
    switch (m) {
        case 0: return launch_wgrad_t<D, false, false, false>(p, ws, st);
        case 1: return launch_wgrad_t<D, false, false, true>(p, ws, st);
        case 2: return launch_wgrad_t<D, false, true, false>(p, ws, st);
        case 3: return launch_wgrad_t<D, false, true, true>(p, ws, st);
        case 4: return launch_wgrad_t<D, true, false, false>(p, ws, st);
        case 5: return launch_wgrad_t<D, true, false, true>(p, ws, st);
        case 6: return launch_wgrad_t<D, true, true, false>(p, ws, st);
        default: return launch_wgrad_t<D, true, true, true>(p, ws, st);
    }
}

}  // namespace wy

hipError_t launch_bwd_dchain(const BwdParams& p, int dk, int dv, const void* records, hipStream_t st) {
    if (dk == 128 && dv == 128) return wy::launch_dchain<128, 128>(p, records, st);
    if (dk == 64 && dv == 64) return wy::launch_dchain<64, 64>(p, records, st);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_wgrad(const BwdParams& p, int dk, int dv, const void* records, hipStream_t st) {
    if (dk == 128 && dv == 128) return wy::launch_wgrad<128>(p, records, st);
    if (dk == 64 && dv == 64) return wy::launch_wgrad<64>(p, records, st);
    return hipErrorInvalidValue;
}

}  // namespace gdr
