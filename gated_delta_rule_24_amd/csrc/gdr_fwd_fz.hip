// Chunkwise forward of the gated delta rule, two roles (bf16 activations,
// chunk 64, d_k and d_v in {64, 128}): a producer that builds every chunk's
// state-independent WY operands, and a state chain that consumes them.
//
// The chunk form (Gated DeltaNet-2 Q&A page, Q4; "Gated DeltaNet-2 Review"
// §3-2 item 5: the cumulative decay is absorbed into the rank-one erase
// factor, which leaves an asymmetric delta recurrence that a WY form solves).
// Per chunk of C tokens with local index r, g_r the in-chunk inclusive prefix
// of log alpha (fp32, per channel; "Gated DeltaNet-2 Review" §3-2 item 2) and
// g_C the chunk total:
//   E_s = b⊙k⊙e^{g}          (decay from the chunk start: every factor <= 1)
//   Q_s = q⊙e^{g}
//   Kh  = k⊙e^{g_C - g}      (decay to the chunk end: <= 1)
//   X   = w⊙v
//   A_ri = sum_c b_r k_r k_i e^{g_r - g_i}  (i < r),   P_ri = sum_c q_r k_i e^{g_r - g_i}  (i <= r)
//   T = (I + A)^-1,  W = T E_s,  U' = T X
// and, with S the chunk-start state,
//   U = U' - W S,   O = Q_s S + P U,   S <- diag(e^{g_C}) S + Kh^T U.
// Every operand above is bounded by its raw input: the factors e^{g},
// e^{g_C - g} and e^{g_r - g_i} (i <= r) never exceed 1, so strong decay only
// makes them underflow where the true contribution is negligible.
//
// A and P are formed on MFMA from operands scaled per 16-token block (a
// block's tokens are one wave's in the element-wise mapping):
//   row operands  b⊙k⊙e^{g_r - rr_R},  q⊙e^{g_r - rr_R}      (r in block R)
//   col operands  k⊙e^{cr_I - g_i}                            (i in block I)
// and a tile (R, I), R > I, rescales the col operand by e^{rr_R - cr_I}.
// A block whose tokens all lie within kMidLimit of the chunk's middle token
// (g at token C/2 - 1) takes that token as both references; blocks of this
// kind share one reference, so their tiles need no rescaling (the usual case:
// a chunk's whole decay is a few nats).  Otherwise a block whose in-block
// decay is moderate takes its own middle token as both references (rr = cr =
// g at token 7 of the block; every factor within e^{±kMidLimit}), so its
// diagonal tile needs no rescaling.  A block with stronger decay references
// its ends (rr = g before its first token, cr = g at its last token; every
// factor <= 1) and forms its diagonal tile from the exact per-element factors
// e^{g_r - g_i} in fp32.  With log alpha <= 0 (g never increases) a rescaled
// col operand k_i e^{rr_R - g_i} stays within e^{kMidLimit} of k_i: the
// factor exceeds 1 only when R takes the chunk's middle and I (< R) its own,
// and then every token of R, so every earlier token, lies above
// rr_R - kMidLimit.
//
// The producer writes each chunk's record (W, Kh^T, U', Q_s, P as MFMA
// fragments, then e^{g_C}) to the workspace; the chain keeps the state in
// MFMA accumulators, one workgroup per 64 value columns of a head, and copies
// each chunk's record into LDS once per workgroup with direct global-to-LDS
// loads.
#include "gdr_device.h"
#include "gdr_launch.h"
#include "gdr_wy.h"

namespace gdr {

namespace fz {

using wy::C;
using wy::cat8;
using wy::f4;
using wy::hi4;
using wy::ld_col4;
using wy::ld_h4;
using wy::ld_h4w;
using wy::ld_h8;
using wy::lo4;
using wy::mfma16;
using wy::mfma32;
using wy::to_h4;

constexpr float kLog2e = 1.4426950408889634f;
// a block takes the middle-token reference when all of its tokens lie within
// this many nats of the block's middle (factors within e^{±6} keep f16 normal
// for inputs down to about 0.01)
constexpr float kMidLimit = 6.0f * kLog2e;   // in log2 units
// a 16-token block's reference for its A and P operands (see Producer::chunk)
constexpr int kRefBlock = 0, kRefEnds = 1, kRefChunk = 2;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Per-chunk record (bytes).  Fragment blocks are 64 lanes x 16 bytes; lane
// l = r + 16 g holds, for a 32-wide K step kk, the K positions 32kk + 4g..+3
// followed by 32kk + 16 + 4g..+3.
//   W    block (rt, kk): row t = 16 rt + r of W, K = channels
//   Kh^T block (mt, kk): channel 16 mt + r of Kh^T, K = tokens
//   U'   strip nt, block kk: column 16 nt + r of U', K = tokens
//   Q_s  block (rt, kk): row 16 rt + r of Q_s, K = channels
//   P    block (rt, kk): row 16 rt + r of P, K = tokens
//   G    e^{g_C} per channel (fp32), in a 1 KiB slot
template <int DK, int DV>
struct RecF {
    static constexpr size_t W = 0;
    static constexpr size_t K = W + (size_t)C * DK * 2;
    static constexpr size_t U = K + (size_t)DK * C * 2;
    static constexpr size_t Q = U + (size_t)C * DV * 2;
    static constexpr size_t P = Q + (size_t)C * DK * 2;
    static constexpr size_t G = P + (size_t)C * C * 2;
    static constexpr size_t bytes = G + 1024;
    static_assert(DK * 4 <= 1024, "G slot");
};

// ---------------------------------------------------------------------------
// producer
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct ProdLayout {
    static constexpr int NT = 256, NW = NT / 64;
    static constexpr int LDE = DK + 8;      // row operands, col operand  [C][LDE]  f16
    static constexpr int LDT = C + 8;       // T, P, Z rows               [*][LDT]  f16
    static constexpr int LDT2 = C + 2;      // E_s^T and X^T rows (odd dword stride)
    static constexpr int LDA = C + 4;       // A                          [C][LDA]  fp32
    static constexpr int LDD = 20;          // diagonal blocks of A, transposed
    static constexpr int CO = DK / 8;       // channel groups of 8 (key side)
    static constexpr int NPART = NT / CO;   // token parts
    static constexpr int TPP = C / NPART;   // tokens per part
    static constexpr int PW = 64 / CO;      // parts per wave: a wave holds one 16-token block
    static constexpr int VO = DV / 8;
    static constexpr int XPART = NT / VO;
    static constexpr int XTP = C / XPART;
    static constexpr size_t oE = 0;
    static constexpr size_t oQ = oE + (size_t)C * LDE * 2;
    static constexpr size_t oK = oQ + (size_t)C * LDE * 2;
    static constexpr size_t oEt = oK + (size_t)C * LDE * 2;      // E_s^T [DK][LDT2]
    static constexpr size_t oXt = oEt + (size_t)DK * LDT2 * 2;   // X^T   [DV][LDT2]
    static constexpr size_t oKt = oXt + (size_t)DV * LDT2 * 2;   // Kh^T  [DK][LDT2]
    static constexpr size_t oT = (oKt + (size_t)DK * LDT2 * 2 + 15) & ~size_t(15);
    static constexpr size_t oP = oT + (size_t)C * LDT * 2;
    static constexpr size_t oZ = oP + (size_t)C * LDT * 2;       // Z^T [C/2][LDT]
    static constexpr size_t oA = oZ + (size_t)(C / 2) * LDT * 2;
    static constexpr size_t oTot = oA + (size_t)C * LDA * 4;     // [NW][DK] fp32 wave totals
    static constexpr size_t oRef = oTot + (size_t)NW * DK * 4;   // [3][4][DK] fp32 (log2 units)
    static constexpr size_t oAd = oRef + (size_t)3 * 4 * DK * 4; // [C/16][16][LDD] fp32
    static constexpr size_t oFl = oAd + (size_t)(C / 16) * 16 * LDD * 4;   // [NW] int
    static constexpr size_t bytes = oFl + (size_t)NW * 4;
    static_assert(PW * TPP == 16, "a wave holds one block");
    static_assert(TPP % 2 == 0 && XTP % 2 == 0, "per-token gates are loaded two tokens at a time");
};

// the channel of slot i (0..7) of channel group co: two runs of four, in the
// fragment K order (32 kk + 4 g .. +3, then 32 kk + 16 + 4 g .. +3)
__device__ __forceinline__ int grp_ch(int co, int i) {
    return 32 * (co >> 2) + 4 * (co & 3) + (i & 3) + (i >= 4 ? 16 : 0);
}

struct NextItem {
    bool has;
    size_t tok0;
    int len;           // tokens of the chunk (C but for a packed sequence's last chunk)
};

// VL: packed variable-length sequences; a chunk may hold fewer than C tokens
// (a sequence's last one).  Its missing rows are loaded from its last token (in
// bounds) and then zeroed (q, k, v) or given no decay (log alpha), so they add
// nothing to A, P, W, U' or the chunk's decay.
template <int DK, int DV, bool AS, bool LG, bool VL = false>
struct Producer {
    using L = ProdLayout<DK, DV>;
    using R = RecF<DK, DV>;
    static constexpr int NT = L::NT, NW = L::NW;
    static constexpr int LDE = L::LDE, LDT = L::LDT, LDT2 = L::LDT2, LDA = L::LDA, LDD = L::LDD;
    static constexpr int CO = L::CO, TPP = L::TPP, PW = L::PW, VO = L::VO, XTP = L::XTP;
    static constexpr int NB = C / 16, NKK = DK / 32, NST = DV / 16;

    unsigned char* smem;
    int tid, lane, wave, r16, g4, co, part, vo, xpart;
    bool BS, WS;            // b, w one value per token (GDR_B_SCALAR, GDR_W_SCALAR)
    // raw inputs of one chunk (issued one chunk ahead, in three groups)
    uint2 rq[TPP][2], rk[TPP][2], rb[TPP][2];
    uint32_t rbs[TPP / 2], rws[XTP / 2];   // b, w of one value per token: two tokens' bf16 per word
    uint32_t rbv[VL ? TPP : 1], rwv[VL ? XTP : 1];   // VL: the same, one token per word
    floatx4 rla[TPP][2];
    u32x4 rv[XTP], rw[XTP];

    __device__ __forceinline__ _Float16* sE() { return reinterpret_cast<_Float16*>(smem + L::oE); }
    __device__ __forceinline__ _Float16* sQ() { return reinterpret_cast<_Float16*>(smem + L::oQ); }
    __device__ __forceinline__ _Float16* sK() { return reinterpret_cast<_Float16*>(smem + L::oK); }
    __device__ __forceinline__ _Float16* sEt() { return reinterpret_cast<_Float16*>(smem + L::oEt); }
    __device__ __forceinline__ _Float16* sXt() { return reinterpret_cast<_Float16*>(smem + L::oXt); }
    __device__ __forceinline__ _Float16* sKt() { return reinterpret_cast<_Float16*>(smem + L::oKt); }
    __device__ __forceinline__ _Float16* sT() { return reinterpret_cast<_Float16*>(smem + L::oT); }
    __device__ __forceinline__ _Float16* sP() { return reinterpret_cast<_Float16*>(smem + L::oP); }
    __device__ __forceinline__ _Float16* sZ() { return reinterpret_cast<_Float16*>(smem + L::oZ); }
    __device__ __forceinline__ float* sA() { return reinterpret_cast<float*>(smem + L::oA); }
    __device__ __forceinline__ float* sTot() { return reinterpret_cast<float*>(smem + L::oTot); }
    __device__ __forceinline__ float* sRef() { return reinterpret_cast<float*>(smem + L::oRef); }
    __device__ __forceinline__ float* sAd() { return reinterpret_cast<float*>(smem + L::oAd); }
    __device__ __forceinline__ int* sFl() { return reinterpret_cast<int*>(smem + L::oFl); }

    __device__ __forceinline__ void init(unsigned char* s, uint32_t flags) {
        smem = s;
        BS = (flags & GDR_B_SCALAR) != 0;
        WS = (flags & GDR_W_SCALAR) != 0;
        tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        r16 = lane & 15;
        g4 = 4 * (lane >> 4);
        co = tid % CO;
        part = tid / CO;
        vo = tid % VO;
        xpart = tid / VO;
        // upper tiles of T and P stay zero (only lower tiles are written per chunk)
        for (int idx = tid; idx < C * C; idx += NT) {
            const int r = idx / C, c = idx % C;
            if ((c >> 4) > (r >> 4)) {
                sT()[r * LDT + c] = (_Float16)0.f;
                sP()[r * LDT + c] = (_Float16)0.f;
            }
        }
    }

    // the loads of a chunk's inputs, group 0 (q, k), 1 (b, log alpha), 2 (v, w).
    // Both forms of b and w are loaded whatever the gate mode: the per-token
    // value (in bounds in either layout) and eight channels, which with one
    // value per token come from k or v instead (same shape, never used).  The
    // loads then take no branch, so no loaded register is copied (a copy would
    // wait for every load in flight).
    __device__ __forceinline__ void issue(const FwdParams& p, size_t tok0, int group, int len = C) {
        const size_t tlast = tok0 + (size_t)(len - 1);     // VL: rows past it read this token
        const uint16_t* bg = reinterpret_cast<const uint16_t*>(p.b);
        const uint16_t* bv = BS ? reinterpret_cast<const uint16_t*>(p.k) : bg;
        if (group < 2) {
            const int c0 = grp_ch(co, 0), c1 = grp_ch(co, 4);
#pragma unroll
            for (int j = 0; j < TPP; ++j) {
                size_t t = tok0 + part * TPP + j;
                if (VL) t = t < tlast ? t : tlast;
                const size_t ix = t * DK;
                if (group == 0) {
                    const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q) + ix;
                    const uint16_t* kg = reinterpret_cast<const uint16_t*>(p.k) + ix;
                    rq[j][0] = *reinterpret_cast<const uint2*>(qg + c0);
                    rq[j][1] = *reinterpret_cast<const uint2*>(qg + c1);
                    rk[j][0] = *reinterpret_cast<const uint2*>(kg + c0);
                    rk[j][1] = *reinterpret_cast<const uint2*>(kg + c1);
                } else {
                    if constexpr (VL) rbv[j] = bg[t];
                    else if (j % 2 == 0) rbs[j / 2] = *reinterpret_cast<const uint32_t*>(bg + t);
                    rb[j][0] = *reinterpret_cast<const uint2*>(bv + ix + c0);
                    rb[j][1] = *reinterpret_cast<const uint2*>(bv + ix + c1);
                    if constexpr (AS) {
                        rla[j][0][0] = p.la[t];
                    } else {
                        rla[j][0] = *reinterpret_cast<const floatx4*>(p.la + ix + c0);
                        rla[j][1] = *reinterpret_cast<const floatx4*>(p.la + ix + c1);
                    }
                }
            }
        } else {
            const uint16_t* vg = reinterpret_cast<const uint16_t*>(p.v);
            const uint16_t* wg = reinterpret_cast<const uint16_t*>(p.w);
            const uint16_t* wv = WS ? vg : wg;
#pragma unroll
            for (int j = 0; j < XTP; ++j) {
                size_t t = tok0 + xpart * XTP + j;
                if (VL) t = t < tlast ? t : tlast;
                const size_t ix = t * DV + 8 * vo;
                rv[j] = *reinterpret_cast<const u32x4*>(vg + ix);
                rw[j] = *reinterpret_cast<const u32x4*>(wv + ix);
                if constexpr (VL) rwv[j] = wg[t];
                else if (j % 2 == 0) rws[j / 2] = *reinterpret_cast<const uint32_t*>(wg + t);
            }
        }
    }

    // the 8 values of slot order (see grp_ch) of a packed pair of uint2 (bf16)
    __device__ static __forceinline__ void unpack(const uint2 (&u)[2], float (&f)[8]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f[4 * h + 0] = __uint_as_float(u[h].x << 16);
            f[4 * h + 1] = __uint_as_float(u[h].x & 0xffff0000u);
            f[4 * h + 2] = __uint_as_float(u[h].y << 16);
            f[4 * h + 3] = __uint_as_float(u[h].y & 0xffff0000u);
        }
    }
    __device__ __forceinline__ void gate_b(int j, float (&b8)[8]) const {
        if (BS) {
            float bs = VL ? __uint_as_float(rbv[j] << 16)
                          : __uint_as_float(j % 2 == 0 ? rbs[j / 2] << 16 : rbs[j / 2] & 0xffff0000u);
            if (LG) bs = gate_sigmoid(bs);
#pragma unroll
            for (int i = 0; i < 8; ++i) b8[i] = bs;
        } else {
            unpack(rb[j], b8);
            if (LG) {
#pragma unroll
                for (int i = 0; i < 8; ++i) b8[i] = gate_sigmoid(b8[i]);
            }
        }
    }

    // One chunk: the element-wise gate work, A and P, T = (I + A)^-1, then W,
    // U', P and Kh^T fragments into `rec`; the next chunk's inputs are issued
    // during the phases.  `hook` runs around the first barrier:
    // hook.before() just before it, hook.after() just after it, returning the
    // next chunk (has, tok0).  Ends with an LDS barrier.
    template <typename Hook>
    __device__ __forceinline__ void chunk(const FwdParams& p, unsigned char* rec, Hook& hook, int len = C) {
        float* tot = sTot();
        float* ref = sRef();
        if constexpr (VL) {
            // rows past the chunk's tokens: q, k zero (v where it is used, log
            // alpha below)
#pragma unroll
            for (int j = 0; j < TPP; ++j) {
                const bool in = part * TPP + j < len;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    rq[j][h] = in ? rq[j][h] : make_uint2(0u, 0u);
                    rk[j][h] = in ? rk[j][h] : make_uint2(0u, 0u);
                }
            }
        }
        // ---------------- in-chunk prefix of log alpha, per channel (log2 units)
        if (LG) {
#pragma unroll
            for (int j = 0; j < TPP; ++j)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!AS || (hh == 0 && i == 0)) rla[j][hh][i] = gate_log_sigmoid(rla[j][hh][i]);
        }
        if constexpr (VL) {
#pragma unroll
            for (int j = 0; j < TPP; ++j) {
                const bool in = part * TPP + j < len;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int i = 0; i < 4; ++i) rla[j][hh][i] = in ? rla[j][hh][i] : 0.f;
            }
        }
        float gl[TPP][8];     // prefix within the part, then the chunk-relative prefix
        float run[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) run[i] = 0.f;
#pragma unroll
        for (int j = 0; j < TPP; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                run[i] += (AS ? rla[j][0][0] : rla[j][i >> 2][i & 3]) * kLog2e;
                gl[j][i] = run[i];
            }
        float excl[8];
        {
            float inc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) inc[i] = run[i];
#pragma unroll
            for (int sh = CO; sh < 64; sh *= 2)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float t = __shfl_up(inc[i], sh);
                    if (lane >= sh) inc[i] += t;
                }
#pragma unroll
            for (int i = 0; i < 8; ++i) excl[i] = inc[i] - run[i];
            if (lane >= 64 - CO) {
#pragma unroll
                for (int i = 0; i < 8; ++i) tot[wave * DK + grp_ch(co, i)] = inc[i];
            }
        }
        hook.before();
        lds_barrier();
        const NextItem nx = hook.after();
        const bool has_next = nx.has;
        const size_t ntok0 = nx.tok0;
        float base[8], wtot[8], gC[8], mid[8], gM[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            base[i] = 0.f;
            gC[i] = 0.f;
            gM[i] = 0.f;
        }
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float t = tot[w2 * DK + grp_ch(co, i)];
                if (w2 < wave) base[i] += t;
                if (w2 == wave) wtot[i] = t;
                if (w2 < NW / 2) gM[i] += t;          // g at the chunk's middle token (C/2 - 1)
                gC[i] += t;
            }
        // g at every token, and at token 7 of this wave's block (the lane of the
        // part holding it, same channels)
        {
            constexpr int PM = 7 / TPP;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float last = excl[i] + gl[TPP - 1][i];
                mid[i] = base[i] + __shfl(last, PM * CO + (lane % CO));
            }
#pragma unroll
            for (int j = 0; j < TPP; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i) gl[j][i] += base[i] + excl[i];
        }
        // the block's reference (its mode, kept in sFl for the tile phase):
        //   kRefChunk  the chunk's middle token, when every token of the block lies
        //              within kMidLimit of it (blocks of this mode share one
        //              reference, so their off-diagonal tiles need no rescaling);
        //   kRefBlock  else the block's middle token, under the same bound;
        //   kRefEnds   else the block's two ends (its diagonal tile exact).
        bool farB = false, farC = false;
#pragma unroll
        for (int j = 0; j < TPP; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                farB |= !(fabsf(gl[j][i] - mid[i]) <= kMidLimit);
                farC |= !(fabsf(gl[j][i] - gM[i]) <= kMidLimit);
            }
        const int mode = __any(farC) == 0 ? kRefChunk : (__any(farB) == 0 ? kRefBlock : kRefEnds);
        const bool slow = mode == kRefEnds;
        float rr[8], cr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float m = mode == kRefChunk ? gM[i] : mid[i];
            rr[i] = slow ? base[i] : m;
            cr[i] = slow ? base[i] + wtot[i] : m;
        }
        if (lane < CO) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int ch = grp_ch(co, i);
                ref[(0 * 4 + wave) * DK + ch] = rr[i];
                ref[(1 * 4 + wave) * DK + ch] = cr[i];
                if (wave == 0) ref[(2 * 4) * DK + ch] = gC[i];
            }
            if (wave == 0) {
                floatx4 e0, e1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e0[i] = __builtin_amdgcn_exp2f(gC[i]);
                    e1[i] = __builtin_amdgcn_exp2f(gC[4 + i]);
                }
                *reinterpret_cast<floatx4*>(rec + R::G + 4 * grp_ch(co, 0)) = e0;
                *reinterpret_cast<floatx4*>(rec + R::G + 4 * grp_ch(co, 4)) = e1;
            }
        }
        if (lane == 0) sFl()[wave] = mode;
        // ---------------- operands: A/P rows and cols, E_s^T, Kh^T, Q_s fragments, X^T
        {
            typedef _Float16 h2 __attribute__((ext_vector_type(2)));
            // Kh = k e^{g_C - g} = (k e^{cr - g}) e^{g_C - cr}: both factors <= 1 or
            // within e^{kMidLimit}, their product <= 1
            float fK[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) fK[i] = __builtin_amdgcn_exp2f(gC[i] - cr[i]);
            h2 et[8], kt[8];   // E_s^T and Kh^T of a token pair, stored once both are formed
            const int kq = co >> 2, gq = co & 3;
#pragma unroll
            for (int j = 0; j < TPP; ++j) {
                const int t = part * TPP + j;
                float q8[8], k8[8], b8[8];
                unpack(rq[j], q8);
                unpack(rk[j], k8);
                gate_b(j, b8);
                half4 e[2], qq[2], kk[2];
                half8 qs;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float d = gl[j][i];
                    const float er = __builtin_amdgcn_exp2f(d - rr[i]);
                    const float ec = __builtin_amdgcn_exp2f(cr[i] - d);
                    const float es = __builtin_amdgcn_exp2f(d);
                    const float bk = b8[i] * k8[i];
                    e[i >> 2][i & 3] = (_Float16)(bk * er);
                    qq[i >> 2][i & 3] = (_Float16)(q8[i] * er);
                    kk[i >> 2][i & 3] = (_Float16)(k8[i] * ec);
                    qs[i] = (_Float16)(q8[i] * es);
                    et[i][j & 1] = (_Float16)(bk * es);
                    kt[i][j & 1] = (_Float16)(k8[i] * (ec * fK[i]));
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int ch = grp_ch(co, 4 * h);
                    *reinterpret_cast<half4*>(sE() + t * LDE + ch) = e[h];
                    *reinterpret_cast<half4*>(sQ() + t * LDE + ch) = qq[h];
                    *reinterpret_cast<half4*>(sK() + t * LDE + ch) = kk[h];
                }
                // Q_s straight to its fragment: row t, K step kq, lane (t & 15) + 16 gq
                *reinterpret_cast<half8*>(rec + R::Q + ((size_t)((t >> 4) * NKK + kq) * 64 + (t & 15) + 16 * gq) * 16) = qs;
                if (j & 1) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        *reinterpret_cast<h2*>(sEt() + grp_ch(co, i) * LDT2 + t - 1) = et[i];
                        *reinterpret_cast<h2*>(sKt() + grp_ch(co, i) * LDT2 + t - 1) = kt[i];
                    }
                }
            }
            _Float16 xt[8][XTP];
#pragma unroll
            for (int j = 0; j < XTP; ++j) {
                float v8[8], w8[8];
                const bool vin = !VL || xpart * XTP + j < len;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t u = vin ? rv[j][i] : 0u;
                    v8[2 * i] = __uint_as_float(u << 16);
                    v8[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
                }
                if (WS) {
                    float wsv = VL ? __uint_as_float(rwv[j] << 16)
                                   : __uint_as_float(j % 2 == 0 ? rws[j / 2] << 16 : rws[j / 2] & 0xffff0000u);
                    if (LG) wsv = gate_sigmoid(wsv);
#pragma unroll
                    for (int i = 0; i < 8; ++i) w8[i] = wsv;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        w8[2 * i] = __uint_as_float(rw[j][i] << 16);
                        w8[2 * i + 1] = __uint_as_float(rw[j][i] & 0xffff0000u);
                    }
                    if (LG) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) w8[i] = gate_sigmoid(w8[i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) xt[i][j] = (_Float16)(v8[i] * w8[i]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < XTP; j += 2) {
                    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                    h2 v;
                    v[0] = xt[i][j];
                    v[1] = xt[i][j + 1];
                    *reinterpret_cast<h2*>(sXt() + (8 * vo + i) * LDT2 + xpart * XTP + j) = v;
                }
        }
        if (slow) diag_exact(gl);
        // the next chunk's q and k load while this one is processed
        if (has_next) issue(p, ntok0, 0, nx.len);
        lds_barrier();

        // ---------------- A = strict_lower(E K^T) (fp32), P = lower(Q K^T) (f16)
        // One lower tile (mt, nt) per task gives both its A and its P tile; a
        // tile below the diagonal rescales its col operand by e^{rr_mt - cr_nt}
        // (<= 1); a diagonal tile of an end-referenced block was formed exactly.
        {
            const int* fl = sFl();
            constexpr int NLT = NB * (NB + 1) / 2;
#pragma unroll
            for (int s2 = 0; s2 < (NLT + NW - 1) / NW; ++s2) {
                const int task = wave + NW * s2;
                if (task >= NLT) break;
                int t = task, mt = 0;
                while (t > mt) { t -= mt + 1; ++mt; }
                const int nt = t;
                if (mt == nt && fl[mt] == kRefEnds) continue;
                const _Float16* xe = sE() + (16 * mt + r16) * LDE + 2 * g4;
                const _Float16* xq = sQ() + (16 * mt + r16) * LDE + 2 * g4;
                const _Float16* xk = sK() + (16 * nt + r16) * LDE + 2 * g4;
                half8 fe[NKK], fq[NKK], fk[NKK];
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    fe[kk] = ld_h8(xe + 32 * kk);
                    fk[kk] = ld_h8(xk + 32 * kk);
                    fq[kk] = ld_h8(xq + 32 * kk);
                }
                if (mt != nt && !(fl[mt] == kRefChunk && fl[nt] == kRefChunk)) {
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) {
                        const int ch = 32 * kk + 2 * g4;
                        const floatx4 a0 = *reinterpret_cast<const floatx4*>(ref + (0 * 4 + mt) * DK + ch);
                        const floatx4 a1 = *reinterpret_cast<const floatx4*>(ref + (0 * 4 + mt) * DK + ch + 4);
                        const floatx4 b0 = *reinterpret_cast<const floatx4*>(ref + (1 * 4 + nt) * DK + ch);
                        const floatx4 b1 = *reinterpret_cast<const floatx4*>(ref + (1 * 4 + nt) * DK + ch + 4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            fk[kk][i] = (_Float16)((float)fk[kk][i] * __builtin_amdgcn_exp2f(a0[i] - b0[i]));
                            fk[kk][4 + i] = (_Float16)((float)fk[kk][4 + i] * __builtin_amdgcn_exp2f(a1[i] - b1[i]));
                        }
                    }
                }
                floatx4 acc = zero4(), acp = zero4();
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    acc = mfma32(fe[kk], fk[kk], acc);
                    acp = mfma32(fk[kk], fq[kk], acp);
                }
                {
                    floatx4 a;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 16 * mt + g4 + i, c = 16 * nt + r16;
                        a[i] = c < r ? acc[i] : 0.f;
                        sA()[r * LDA + c] = a[i];
                    }
                    if (mt == nt) *reinterpret_cast<floatx4*>(sAd() + (mt * 16 + r16) * LDD + g4) = a;
                }
                {
                    // lane holds P[16 mt + r16][16 nt + g4 + i]
                    const int tr = 16 * mt + r16;
                    floatx4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (16 * nt + g4 + i <= tr) ? acp[i] : 0.f;
                    *reinterpret_cast<half4*>(sP() + tr * LDT + 16 * nt + g4) = to_h4(v);
                }
            }
        }
        lds_barrier();
        if (has_next) issue(p, ntok0, 1, nx.len);
        {
            // diagonal block `wave` of T = (I + A)^-1 by forward substitution in fp32:
            // lane (column jc, rows 4 rg .. 4 rg + 3) holds its rows' values of the
            // column, and A's column m (rows 4 rg ..) comes from the transposed copy;
            // step m takes x_m from the lane group holding row m and subtracts
            // A[:, m] x_m (A is zero on and above the diagonal, so row m keeps x_m)
            static_assert(NB == NW, "one diagonal block per wave");
            const int jc = lane & 15, rg = lane >> 4;
            const float* ad = sAd() + wave * 16 * LDD + 4 * rg;
            floatx4 acol[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) acol[m] = *reinterpret_cast<const floatx4*>(ad + m * LDD);
            floatx4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (4 * rg + i == jc) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                const float xm = __shfl(x[m & 3], jc + 16 * (m >> 2));
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] -= acol[m][i] * xm;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sT()[(16 * wave + 4 * rg + i) * LDT + 16 * wave + jc] = (_Float16)x[i];
        }
        {
            // fragments of P and Kh^T (both K = tokens) from their LDS rows
            constexpr int NPB = NB * (C / 32), NKB = (DK / 16) * (C / 32);
            for (int task = wave; task < NPB + NKB; task += NW) {
                if (task < NPB) {
                    const int rt = task / (C / 32), kk = task % (C / 32);
                    const _Float16* src = sP() + (16 * rt + r16) * LDT + 32 * kk + g4;
                    *reinterpret_cast<half8*>(rec + R::P + ((size_t)(rt * (C / 32) + kk) * 64 + lane) * 16) =
                        cat8(ld_h4(src), ld_h4(src + 16));
                } else {
                    const int tk = task - NPB, mt = tk / (C / 32), kk = tk % (C / 32);
                    const _Float16* src = sKt() + (16 * mt + r16) * LDT2 + 32 * kk + g4;
                    *reinterpret_cast<half8*>(rec + R::K + ((size_t)(mt * (C / 32) + kk) * 64 + lane) * 16) =
                        cat8(ld_h4w(src), ld_h4w(src + 16));
                }
            }
        }
        lds_barrier();
        // ---------------- off-diagonal blocks of T by doubling: T_BA = -T_BB (A_BA T_AA)
#pragma unroll
        for (int sz = 16; sz < C; sz *= 2) {
            const int nsub = sz / 16, ntask = (C / (2 * sz)) * nsub * nsub;
            for (int task = wave; task < ntask; task += NW) {
                const int pr = task / (nsub * nsub), mi = (task / nsub) % nsub, ni = task % nsub;
                const int a0 = 2 * sz * pr, b0 = a0 + sz;
                floatx4 acc = zero4();
#pragma unroll
                for (int k = 0; k < sz; k += 16) {
                    const floatx4 av = *reinterpret_cast<const floatx4*>(sA() + (b0 + 16 * mi + r16) * LDA + a0 + k + g4);
                    acc = mfma16(to_h4(av), ld_col4(sT() + (a0 + k + g4) * LDT + a0 + 16 * ni + r16, LDT), acc);
                }
                *reinterpret_cast<half4*>(sZ() + (pr * sz + 16 * ni + r16) * LDT + 16 * mi + g4) = to_h4(acc);
            }
            lds_barrier();
            for (int task = wave; task < ntask; task += NW) {
                const int pr = task / (nsub * nsub), mi = (task / nsub) % nsub, ni = task % nsub;
                const int a0 = 2 * sz * pr, b0 = a0 + sz;
                floatx4 acc = zero4();
#pragma unroll
                for (int k = 0; k < sz; k += 16)
                    acc = mfma16(ld_h4(sT() + (b0 + 16 * mi + r16) * LDT + b0 + k + g4),
                                 ld_h4(sZ() + (pr * sz + 16 * ni + r16) * LDT + k + g4), acc);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sT()[(b0 + 16 * mi + g4 + i) * LDT + a0 + 16 * ni + r16] = (_Float16)(-acc[i]);
            }
            lds_barrier();
        }
        // ---------------- W = T E_s (fragments: W^T = E_s^T T^T) and U' = T X.
        // T's upper tiles are zero, so every product runs over the full K = C;
        // pairs of 16-token blocks form the 32-deep MFMA operands.
        static_assert((NB * NKK) % NW == 0 && (NST * (C / 32)) % NW == 0, "tasks per wave");
#pragma unroll
        for (int s2 = 0; s2 < NB * NKK / NW; ++s2) {
            const int task = wave + NW * s2;
            const int rt = task / NKK, kk = task % NKK;
            half4 fx[2][NB], fy[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                fy[k] = ld_h4(sT() + (16 * rt + r16) * LDT + 16 * k + g4);
#pragma unroll
                for (int h = 0; h < 2; ++h) fx[h][k] = ld_h4w(sEt() + (32 * kk + 16 * h + r16) * LDT2 + 16 * k + g4);
            }
            floatx4 acc[2] = {zero4(), zero4()};
#pragma unroll
            for (int k = 0; k < NB; k += 2)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    acc[h] = mfma32(cat8(fx[h][k], fx[h][k + 1]), cat8(fy[k], fy[k + 1]), acc[h]);
            *reinterpret_cast<half8*>(rec + R::W + ((size_t)(rt * NKK + kk) * 64 + lane) * 16) =
                cat8(to_h4(acc[0]), to_h4(acc[1]));
        }
#pragma unroll
        for (int s2 = 0; s2 < NST * (C / 32) / NW; ++s2) {
            const int task = wave + NW * s2;
            const int nt = task / (C / 32), kk = task % (C / 32);
            half4 fx[2][NB], fy[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                fy[k] = ld_h4w(sXt() + (16 * nt + r16) * LDT2 + 16 * k + g4);
#pragma unroll
                for (int h = 0; h < 2; ++h) fx[h][k] = ld_h4(sT() + (16 * (2 * kk + h) + r16) * LDT + 16 * k + g4);
            }
            floatx4 acc[2] = {zero4(), zero4()};
#pragma unroll
            for (int k = 0; k < NB; k += 2)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    acc[h] = mfma32(cat8(fx[h][k], fx[h][k + 1]), cat8(fy[k], fy[k + 1]), acc[h]);
            *reinterpret_cast<half8*>(rec + R::U + ((size_t)(nt * (C / 32) + kk) * 64 + lane) * 16) =
                cat8(to_h4(acc[0]), to_h4(acc[1]));
        }
        if (has_next) issue(p, ntok0, 2, nx.len);
        lds_barrier();
    }

    // Diagonal A and P tiles of this wave's block from the exact per-element
    // factors e^{g_r - g_i} (fp32).  For each part s of the block, every lane
    // forms its 8 channels' share of the (row of its part, column of part s)
    // pairs; the shares are summed over the CO lanes of the part (a butterfly),
    // and lane co writes the pairs e = co, co + CO, ... of the TPP x TPP sums.
    // gl holds the chunk-relative prefix g (log2 units) of this lane's tokens;
    // the raw inputs in the registers are still those of this chunk.
    __device__ __forceinline__ void diag_exact(const float (&gl)[TPP][8]) {
        const int pw = lane / CO, cl = lane % CO;
        float q8[TPP][8], bk8[TPP][8];
#pragma unroll
        for (int j = 0; j < TPP; ++j) {
            float k8[8], b8[8];
            unpack(rq[j], q8[j]);
            unpack(rk[j], k8);
            gate_b(j, b8);
#pragma unroll
            for (int i = 0; i < 8; ++i) bk8[j][i] = b8[i] * k8[i];
        }
        float* A = sA();
        float* Ad = sAd();
        _Float16* P = sP();
#pragma unroll
        for (int s = 0; s < PW; ++s) {
            const int src = s * CO + cl;
            float pa[TPP][TPP], pp[TPP][TPP];
#pragma unroll
            for (int jj = 0; jj < TPP; ++jj) {
                uint2 ku[2];
                ku[0].x = __shfl(rk[jj][0].x, src);
                ku[0].y = __shfl(rk[jj][0].y, src);
                ku[1].x = __shfl(rk[jj][1].x, src);
                ku[1].y = __shfl(rk[jj][1].y, src);
                float ks[8], gs[8];
                unpack(ku, ks);
#pragma unroll
                for (int i = 0; i < 8; ++i) gs[i] = __shfl(gl[jj][i], src);
#pragma unroll
                for (int j = 0; j < TPP; ++j) {
                    float a = 0.f, q = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float e = ks[i] * __builtin_amdgcn_exp2f(gl[j][i] - gs[i]);
                        a += bk8[j][i] * e;
                        q += q8[j][i] * e;
                    }
                    pa[j][jj] = a;
                    pp[j][jj] = q;
                }
            }
#pragma unroll
            for (int m = 1; m < CO; m *= 2)
#pragma unroll
                for (int j = 0; j < TPP; ++j)
#pragma unroll
                    for (int jj = 0; jj < TPP; ++jj) {
                        pa[j][jj] += __shfl_xor(pa[j][jj], m);
                        pp[j][jj] += __shfl_xor(pp[j][jj], m);
                    }
#pragma unroll
            for (int e = 0; e < TPP * TPP; ++e) {
                if (e % CO != cl) continue;
                const int j = e / TPP, jj = e % TPP;
                const int row = pw * TPP + j, col = s * TPP + jj;   // within the block
                const float a = col < row ? pa[j][jj] : 0.f;
                const float q = col <= row ? pp[j][jj] : 0.f;
                const int r = 16 * wave + row;
                A[r * LDA + 16 * wave + col] = a;
                Ad[(wave * 16 + col) * LDD + row] = a;
                P[r * LDT + 16 * wave + col] = (_Float16)q;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// state chain
// ---------------------------------------------------------------------------
// A head's DV value columns are split into DV/64 blocks of 64, and each block
// is one workgroup of four waves: two compute waves, each owning 32 of the
// block's columns (their fp32 state in MFMA accumulators), and two copy waves
// that move each chunk's record into LDS (direct global-to-LDS loads, one
// chunk ahead, two stages) and watch the records' readiness.  The compute
// waves read every fragment from LDS and touch global memory only to store
// the output.  Every compute wave reads the chunk's full W, Kh^T, Q_s and P,
// so LDS traffic grows with the number of compute waves: two waves per 64
// columns measured faster than four waves per 64 or per 128 columns.
constexpr int kChainCols = 64;
constexpr int kComputeWaves = 2;

template <int DK, int DV>
struct ChainLayout {
    using R = RecF<DK, DV>;
    static constexpr int SPW = kChainCols / (16 * kComputeWaves);   // strips per compute wave
    static constexpr int WPH = DV / kChainCols;              // workgroups per head
    static constexpr size_t stage = R::bytes;                // one whole record
    static constexpr size_t oOk = 2 * stage;                 // int[2]: a record is ready
    static constexpr size_t bytes = oOk + 16;
    static constexpr int NLOAD = (int)(stage / 1024);        // 1 KiB copies per chunk
    static_assert(stage % 1024 == 0, "record in 1 KiB pieces");
};

// a 1 KiB global-to-LDS copy by one wave: lane l moves bytes 16 l .. 16 l + 15
__device__ __forceinline__ void copy_1k(const unsigned char* src, unsigned char* lds_dst, int lane) {
    typedef __attribute__((address_space(3))) void* lds_ptr;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + 16 * lane),
                                     (lds_ptr)lds_dst, 16, 0, 0);
}

// wait until at most n of this wave's vector memory operations are in flight
// (they complete in issue order)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int DK, int DV>
struct Chain {
    using L = ChainLayout<DK, DV>;
    using R = RecF<DK, DV>;
    static constexpr int NKT = DK / 16, NKK = DK / 32, NB = C / 16, NK2 = C / 32, SPW = L::SPW;

    unsigned char* smem;
    int lane, wave, n_l, g4;

    __device__ __forceinline__ void init(unsigned char* s) {
        smem = s;
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        n_l = lane & 15;
        g4 = 4 * (lane >> 4);
    }

    // a copy wave's share of the copies of chunk record `rec` into stage st
    __device__ __forceinline__ void fetch(const unsigned char* rec, int st) {
        unsigned char* dst = smem + (size_t)st * L::stage;
        for (int i = wave - kComputeWaves; i < L::NLOAD; i += 4 - kComputeWaves)
            copy_1k(rec + (size_t)i * 1024, dst + (size_t)i * 1024, lane);
    }

    // The chain of sequence bh over NC chunks whose records start at rec0 (RB
    // bytes apart).  A record's readiness is asked by the first copy wave only,
    // through rd:
    //   rd.poll(c)  starts looking at chunk c (no wait),
    //   rd.wait(c)  returns once chunk c's record may be read; false if it never
    //               became ready (the chain then stops and writes NaN state),
    // and reaches the other waves through LDS (one slot per chunk parity).  One
    // workgroup barrier per chunk: past it, chunk c's copies are in LDS, every
    // wave is done with chunk c - 1 (so its stage takes chunk c + 1's copies),
    // and chunk c + 1's readiness is in its slot.  Chunk c + 2's readiness is
    // awaited while the compute waves work on chunk c.  bh indexes the state
    // (S0, S_final); the last chunk stores its first last_rows output rows only;
    // with NC = 0 the state passes through.
    template <typename Ready>
    __device__ __forceinline__ void run(const FwdParams& p, const unsigned char* rec0, size_t RB, int NC, int bh,
                                        size_t tok_base, int colbase, Ready& rd, int last_rows = C) {
        int* s_ok = reinterpret_cast<int*>(smem + L::oOk);   // [2]: chunk x's readiness in slot x & 1
        bool ok = true;
        if (NC > 0) {
            if (wave == kComputeWaves) {
                rd.poll(0);
                const bool r0 = rd.wait(0);
                bool r1 = true;
                if (NC > 1) {
                    rd.poll(1);
                    r1 = rd.wait(1);
                }
                if (lane == 0) {
                    s_ok[0] = r0 ? 1 : 0;
                    s_ok[1] = r1 ? 1 : 0;
                }
            }
            lds_barrier();
            ok = s_ok[0] != 0;
        }
        if (wave < kComputeWaves) compute(p, rec0, NC, bh, tok_base, colbase, ok, last_rows);
        else copy(rec0, RB, NC, ok, rd);
        lds_barrier();                                         // LDS free for the next chain
    }

    template <typename Ready>
    __device__ __forceinline__ void copy(const unsigned char* rec0, size_t RB, int NC, bool ok, Ready& rd) {
        int* s_ok = reinterpret_cast<int*>(smem + L::oOk);
        if (ok && NC > 0) fetch(rec0, 0);
        for (int c = 0; c < NC && ok; ++c) {
            wait_vm<0>();                                      // this wave's copies of chunk c
            lds_barrier();
            if (c + 1 < NC && s_ok[(c + 1) & 1] == 0) {
                ok = false;
                break;
            }
            if (c + 1 < NC) fetch(rec0 + (size_t)(c + 1) * RB, (c + 1) & 1);
            // chunk c + 2's readiness into slot c & 1 (read after the next barrier;
            // its previous readers, past the barrier of chunk c - 1, are past this one)
            if (wave == kComputeWaves && c + 2 < NC) {
                rd.poll(c + 2);
                const bool r = rd.wait(c + 2);
                if (lane == 0) s_ok[c & 1] = r ? 1 : 0;
            }
        }
    }

    __device__ __forceinline__ void compute(const FwdParams& p, const unsigned char* rec0, int NC, int bh,
                                            size_t tok_base, int colbase, bool ok, int last_rows) {
        (void)rec0;
        const int col0 = colbase + 16 * SPW * wave;          // this wave's first column
        int* s_ok = reinterpret_cast<int*>(smem + L::oOk);
        floatx4 S[SPW][NKT];
#pragma unroll
        for (int s = 0; s < SPW; ++s)
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[s][mt][i] = p.S0 ? p.S0[((size_t)bh * DK + 16 * mt + g4 + i) * DV + col0 + 16 * s + n_l] : 0.f;
        const bool out_bf16 = (p.flags & GDR_OUT_BF16) != 0;
        for (int c = 0; c < NC && ok; ++c) {
            lds_barrier();
            if (c + 1 < NC && s_ok[(c + 1) & 1] == 0) {
                ok = false;
                break;
            }
            const unsigned char* st = smem + (size_t)(c & 1) * L::stage;
            auto frag = [&](size_t off) __attribute__((always_inline)) {
                return *reinterpret_cast<const half8*>(st + off + (size_t)lane * 16);
            };
            // The fragments of each phase are read from LDS into registers during the
            // previous phase's MFMAs (W right after the barrier; K, U', e^{g_C}
            // while Y runs; Q_s and P while the state update runs), one LDS read
            // placed after each MFMA, so that LDS reads and products overlap.
            half8 wf[NB][NKK];
#pragma unroll
            for (int rt = 0; rt < NB; ++rt)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) wf[rt][kk] = frag(R::W + (size_t)(rt * NKK + kk) * 1024);
            // the state as f16 fragments (lane: column n_l, K = channels)
            half8 sf[SPW][NKK];
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) sf[s][kk] = cat8(to_h4(S[s][2 * kk]), to_h4(S[s][2 * kk + 1]));
            __builtin_amdgcn_sched_barrier(0);
            // phase A: Y = W S, with the reads of phase B's operands in between
            half8 kf[NKT][NK2], uq[SPW][NK2];
            floatx4 gm[NKT];
            const float* G = reinterpret_cast<const float*>(st + R::G);
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
                for (int kk = 0; kk < NK2; ++kk) kf[mt][kk] = frag(R::K + (size_t)(mt * NK2 + kk) * 1024);
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int kk = 0; kk < NK2; ++kk) uq[s][kk] = frag(R::U + (size_t)((col0 / 16 + s) * NK2 + kk) * 1024);
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt) gm[mt] = *reinterpret_cast<const floatx4*>(G + 16 * mt + g4);
            floatx4 Y[SPW][NB];
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int rt = 0; rt < NB; ++rt) Y[s][rt] = zero4();
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int rt = 0; rt < NB; ++rt)
#pragma unroll
                    for (int s = 0; s < SPW; ++s) Y[s][rt] = mfma32(wf[rt][kk], sf[s][kk], Y[s][rt]);
            {
                constexpr int NRD = NKT * NK2 + SPW * NK2 + NKT, NMF = NKK * NB * SPW;
                constexpr int NPAIR = NRD < NMF ? NRD : NMF;
#pragma unroll
                for (int i = 0; i < NPAIR; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, NMF - NPAIR, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, NRD - NPAIR, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            // U = U' - Y as fragments (lane: column n_l, K = tokens)
            half8 uf[SPW][NK2];
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int kk = 0; kk < NK2; ++kk)
                    uf[s][kk] = cat8(to_h4(f4(lo4(uq[s][kk])) - Y[s][2 * kk]), to_h4(f4(hi4(uq[s][kk])) - Y[s][2 * kk + 1]));
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
                for (int s = 0; s < SPW; ++s) S[s][mt] = S[s][mt] * gm[mt];
            __builtin_amdgcn_sched_barrier(0);
            // phase B: S = diag(e^{g_C}) S + Kh^T U, with the reads of Q_s and P in between
            half8 qf[NB][NKK], pf[NB][NK2];
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) qf[rt][kk] = frag(R::Q + (size_t)(rt * NKK + kk) * 1024);
#pragma unroll
                for (int kk = 0; kk <= rt / 2; ++kk) pf[rt][kk] = frag(R::P + (size_t)(rt * NK2 + kk) * 1024);
            }
#pragma unroll
            for (int kk = 0; kk < NK2; ++kk)
#pragma unroll
                for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
                    for (int s = 0; s < SPW; ++s) S[s][mt] = mfma32(kf[mt][kk], uf[s][kk], S[s][mt]);
            {
                constexpr int NRD = NB * NKK + (NB / 2) * (NB / 2 + 1), NMF = NK2 * NKT * SPW;
                constexpr int NPAIR = NRD < NMF ? NRD : NMF;
#pragma unroll
                for (int i = 0; i < NPAIR; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, NMF - NPAIR, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, NRD - NPAIR, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            // phase C: O^T = S^T Q_s^T + U^T P^T (S the chunk-start state): a lane
            // ends with four consecutive columns of one token's output row
            floatx4 O[SPW][NB];
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int rt = 0; rt < NB; ++rt) O[s][rt] = zero4();
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int rt = 0; rt < NB; ++rt)
#pragma unroll
                    for (int s = 0; s < SPW; ++s) O[s][rt] = mfma32(sf[s][kk], qf[rt][kk], O[s][rt]);
#pragma unroll
            for (int rt = 0; rt < NB; ++rt)
#pragma unroll
                for (int kk = 0; kk <= rt / 2; ++kk)
#pragma unroll
                    for (int s = 0; s < SPW; ++s) O[s][rt] = mfma32(uf[s][kk], pf[rt][kk], O[s][rt]);
            // lane holds O[token 16 rt + n_l][columns 16 s + g4 .. + 3]
            const size_t tok0 = tok_base + (size_t)c * C;
            const int rows = c + 1 < NC ? C : last_rows;
#pragma unroll
            for (int rt = 0; rt < NB; ++rt)
#pragma unroll
                for (int s = 0; s < SPW; ++s) {
                    if (16 * rt + n_l >= rows) continue;
                    const size_t base = (tok0 + 16 * rt + n_l) * DV + col0 + 16 * s + g4;
                    const floatx4 o = O[s][rt];
                    if (out_bf16) {
                        uint2 u;
                        u.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
                        u.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
                        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.o) + base) = u;
                    } else {
                        *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(p.o) + base) = o;
                    }
                }
        }
        if (p.Sf) {
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        p.Sf[((size_t)bh * DK + 16 * mt + g4 + i) * DV + col0 + 16 * s + n_l] =
                            ok ? S[s][mt][i] : __builtin_nanf("");
        }
    }
};

// ---------------------------------------------------------------------------
// two-kernel form: the producer over every chunk, then one chain per head
// ---------------------------------------------------------------------------
template <int DK, int DV, bool AS, bool LG>
__global__ __launch_bounds__(256, 1) void prod_kernel(FwdParams p, unsigned char* ws) {
    using PR = Producer<DK, DV, AS, LG>;
    using R = RecF<DK, DV>;
    extern __shared__ __align__(16) unsigned char smem[];
    PR pr;
    pr.init(smem, p.flags);
    const int CN = p.T / C;
    const int total = p.BH * CN;
    int idx = blockIdx.x;
    auto tok_of = [&](int i) { return (size_t)(i / CN) * p.T + (size_t)(i % CN) * C; };
    if (idx < total) {
        const size_t t0 = tok_of(idx);
        pr.issue(p, t0, 0);
        pr.issue(p, t0, 1);
        pr.issue(p, t0, 2);
    }
    struct Hook {
        NextItem nx;
        __device__ void before() {}
        __device__ NextItem after() { return nx; }
    } hook;
    for (; idx < total; idx += gridDim.x) {
        const int nx = idx + (int)gridDim.x;
        hook.nx.has = nx < total;
        hook.nx.tok0 = hook.nx.has ? tok_of(nx) : 0;
        hook.nx.len = C;
        pr.chunk(p, ws + (size_t)idx * R::bytes, hook);
    }
}

// Packed variable-length sequences (p.cu_seqlens and the prep arrays set; p.BH
// = H heads of p.T packed tokens).  Work item = (head, chunk r of the head's
// concatenated sequences), looked up in the chunk table; records numbered
// head * (chunk count) + r, as the two-pass kernels number them.
template <int DK, int DV, bool AS, bool LG>
__global__ __launch_bounds__(256, 1) void prod_kernel_vl(FwdParams p, unsigned char* ws) {
    using PR = Producer<DK, DV, AS, LG, true>;
    using R = RecF<DK, DV>;
    extern __shared__ __align__(16) unsigned char smem[];
    const int CN = p.chunk_off[p.nseq];
    const int total = p.BH * CN;
    int idx = blockIdx.x;
    if (idx >= total) return;
    PR pr;
    pr.init(smem, p.flags);
    const int2* tab = reinterpret_cast<const int2*>(p.chunk_tab);
    auto item = [&](int i, size_t& t0, int& len) {
        const int h = i / CN, r = i - h * CN;
        const int2 e = tab[r];
        t0 = (size_t)h * p.T + (size_t)e.x;
        len = e.y;
    };
    {
        size_t t0;
        int len;
        item(idx, t0, len);
        pr.issue(p, t0, 0, len);
        pr.issue(p, t0, 1, len);
        pr.issue(p, t0, 2, len);
    }
    struct Hook {
        NextItem nx;
        __device__ void before() {}
        __device__ NextItem after() { return nx; }
    } hook;
    for (; idx < total; idx += gridDim.x) {
        const int nx = idx + (int)gridDim.x;
        size_t t0;
        int len;
        item(idx, t0, len);
        hook.nx.has = nx < total;
        hook.nx.tok0 = 0;
        hook.nx.len = C;
        if (hook.nx.has) item(nx, hook.nx.tok0, hook.nx.len);
        pr.chunk(p, ws + (size_t)idx * R::bytes, hook, len);
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(256, 1) void chain_kernel(FwdParams p, const unsigned char* ws) {
    using CH = Chain<DK, DV>;
    using R = RecF<DK, DV>;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int WPH = CH::L::WPH;
    const int bh = blockIdx.x / WPH;
    const int NC = p.T / C;
    CH ch;
    ch.init(smem);
    struct Always {
        __device__ void poll(int) {}
        __device__ bool wait(int) { return true; }
    } rd;
    ch.run(p, ws + (size_t)bh * NC * R::bytes, R::bytes, NC, bh, (size_t)bh * p.T, (blockIdx.x % WPH) * kChainCols, rd);
}

// Packed sequences: one chain per (sequence, head) and column block, the
// longest sequences first (p.seq_order); the state of sequence s on head h is
// S0[s * H + h].
template <int DK, int DV>
__global__ __launch_bounds__(256, 1) void chain_kernel_vl(FwdParams p, const unsigned char* ws) {
    using CH = Chain<DK, DV>;
    using R = RecF<DK, DV>;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int WPH = CH::L::WPH;
    int blk = 0;
    const int bh = wy::packed_chain(p.seq_order, p.BH, WPH, (int)blockIdx.x, (int)gridDim.x, blk);
    const wy::PackedSpan sp = wy::packed_span(p.cu_seqlens, p.chunk_off, p.nseq, p.BH, p.T, bh);
    CH ch;
    ch.init(smem);
    struct Always {
        __device__ void poll(int) {}
        __device__ bool wait(int) { return true; }
    } rd;
    const int last = sp.len - (sp.NC > 0 ? (sp.NC - 1) * C : 0);
    ch.run(p, ws + sp.chunk0 * R::bytes, R::bytes, sp.NC, bh, sp.tok0, blk * kChainCols, rd, last);
}

// ---------------------------------------------------------------------------
// one persistent kernel: producers and chains side by side
// ---------------------------------------------------------------------------
// The grid is one workgroup per compute unit.  Each workgroup reads the id of
// the XCD it runs on and takes a rank among that XCD's workgroups.  Heads are
// dealt to the XCDs (head h to XCD slot h mod NX); on each XCD the first
// workgroups (at most CAP, a whole number of heads' column blocks) run the
// chains of its heads, the others produce that XCD's chunks, claimed one at a
// time from a per-XCD counter, in the order the chains consume them
// (chunk-major within each batch of heads chained at once).  A record is written to the XCD's L2 and read from there: producer
// and consumer share the L2, which orders their accesses.  A producer
// publishes a chunk (a flag, written after every wave has seen its record
// stores complete) while it works on its next chunk; a chain waits for the
// flag with a bounded spin (on time-out it stops and writes NaN to its state).
// Control words (zeroed by fz_clear before every call):
//   ctl[0..15]  workgroups seen per XCD slot      ctl[16..31] chunks claimed per slot
struct FusedCfg {
    int* flags;        // [BH * NC] chunk published
    int* ctl;          // [64]
    int NX;            // XCD slots
    int CAP;           // chain workgroups per slot at most (at least one head's blocks)
    unsigned spin;     // polls before a chain gives up
};

__global__ void fz_clear(int* a, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) a[i] = 0;
}

__device__ __forceinline__ int xcc_id() {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return (int)(x & 0xf);
}

template <int DK, int DV, bool AS, bool LG>
__global__ __launch_bounds__(256, 1) void fused_kernel(FwdParams p, unsigned char* ws, FusedCfg cfg) {
    using PR = Producer<DK, DV, AS, LG>;
    using CH = Chain<DK, DV>;
    using R = RecF<DK, DV>;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_role[2];
    __shared__ int s_item;
    const int NC = p.T / C;
    if (threadIdx.x == 0) {
        const int slot = xcc_id() % cfg.NX;
        s_role[0] = slot;
        s_role[1] = atomicAdd(&cfg.ctl[slot], 1);
    }
    __syncthreads();
    const int slot = s_role[0], rank = s_role[1];
    constexpr int WPH = CH::L::WPH;                                          // column blocks per head
    const int nh = slot < p.BH ? (p.BH - slot + cfg.NX - 1) / cfg.NX : 0;   // heads of this slot
    const int cap = cfg.CAP / WPH > 0 ? cfg.CAP / WPH : 1;
    const int nch = nh < cap ? nh : cap;                                     // heads chained at once
    if (rank < nch * WPH) {
        CH ch;
        ch.init(smem);
        for (int j = rank / WPH; j < nh; j += nch) {
            const int h = slot + cfg.NX * j;
            // the flags of this head's chunks; poll() issues the load, wait()
            // uses it and spins (bounded) while the flag is still clear
            struct Flags {
                const int* fl;
                unsigned spin;
                int seen;
                __device__ void poll(int c) {
                    seen = __hip_atomic_load(fl + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                __device__ bool wait(int c) {
                    unsigned n = 0;
                    while (seen == 0) {
                        if (++n > spin) return false;
                        __builtin_amdgcn_s_sleep(2);
                        seen = __hip_atomic_load(fl + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    return true;
                }
            } rd;
            rd.fl = cfg.flags + (size_t)h * NC;
            rd.spin = cfg.spin;
            rd.seen = 0;
            ch.run(p, ws + (size_t)h * NC * R::bytes, R::bytes, NC, h, (size_t)h * p.T, (rank % WPH) * kChainCols, rd);
        }
        return;
    }
    // producer: claim this slot's chunks in order; chunk `it` of the slot is
    // chunk c of local head jj = gen * nch + (rem mod w), the heads chained
    // together (a batch of nch, the last one possibly smaller) in chunk-major order
    const int total = nh * NC;
    int* ctr = cfg.ctl + 16 + slot;
    auto locate = [&](int it, int& h, int& c) {
        const int gen = it / (NC * nch);
        const int rem = it - gen * NC * nch;
        const int left = nh - gen * nch;
        const int w = left < nch ? left : nch;
        c = rem / w;
        h = slot + cfg.NX * (gen * nch + rem % w);
    };
    // thread 0 keeps one claim in hand (`pending`): at the start of every chunk it
    // hands that one on (the chunk after the current one) and claims another, so
    // no thread waits for a claim's round trip
    int pending = 0;
    if (threadIdx.x == 0) {
        s_item = atomicAdd(ctr, 1);
        pending = atomicAdd(ctr, 1);
    }
    __syncthreads();
    int it = s_item;
    __syncthreads();                                   // everyone has read it before the next claim
    if (it >= total) return;
    PR pr;
    pr.init(smem, p.flags);
    {
        int h, c;
        locate(it, h, c);
        const size_t t0 = (size_t)h * p.T + (size_t)c * C;
        pr.issue(p, t0, 0);
        pr.issue(p, t0, 1);
        pr.issue(p, t0, 2);
    }
    struct Hook {
        int* fl;
        int prev;          // the chunk to publish after the first barrier (-1: none)
        int* s_item;
        int claimed;       // the chunk claimed for after this one (read after the first barrier)
        int total;
        int NC, T;
        int tid;
        decltype(locate)* loc;
        __device__ void before() {
            // this wave's stores of the previous chunk's record are complete
            if (prev >= 0) wait_vm<0>();
        }
        __device__ NextItem after() {
            if (prev >= 0 && tid == 0) {
                int h, c;
                (*loc)(prev, h, c);
                __hip_atomic_store(fl + (size_t)h * NC + c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            const int nx = *s_item;
            claimed = nx;
            NextItem r;
            r.has = nx < total;
            r.tok0 = 0;
            r.len = C;
            if (r.has) {
                int h, c;
                (*loc)(nx, h, c);
                r.tok0 = (size_t)h * T + (size_t)c * C;
            }
            return r;
        }
    } hook;
    hook.fl = cfg.flags;
    hook.prev = -1;
    hook.s_item = &s_item;
    hook.total = total;
    hook.NC = NC;
    hook.T = p.T;
    hook.tid = threadIdx.x;
    hook.loc = &locate;
    while (true) {
        // the chunk after this one (read by every thread after the first barrier)
        if (threadIdx.x == 0) {
            s_item = pending;
            pending = atomicAdd(ctr, 1);
        }
        int h, c;
        locate(it, h, c);
        pr.chunk(p, ws + ((size_t)h * NC + c) * R::bytes, hook);
        hook.prev = it;
        if (hook.claimed >= total) break;
        it = hook.claimed;
    }
    // publish the last chunk
    wait_vm<0>();
    lds_barrier();
    if (threadIdx.x == 0) {
        int h, c;
        locate(it, h, c);
        __hip_atomic_store(cfg.flags + (size_t)h * NC + c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// workspace: records, then the chunk flags and the control words
template <int DK, int DV>
static size_t flags_offset(int BH, int T) {
    return (((size_t)BH * (T / C) * RecF<DK, DV>::bytes) + 255) & ~size_t(255);
}

struct Topology {
    int ncu, nx;
};
static Topology topology() {
    Topology t{256, 8};
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        t.ncu = n;
    // an MI355X XCD holds 32 compute units
    t.nx = t.ncu >= 32 ? t.ncu / 32 : 1;
    if (t.nx > 16) t.nx = 16;
    return t;
}

template <int DK, int DV, bool AS, bool LG>
static hipError_t launch_t(const FwdParams& p, void* ws, hipStream_t st) {
    using PL = ProdLayout<DK, DV>;
    using CL = ChainLayout<DK, DV>;
    constexpr size_t LDS = PL::bytes > CL::bytes ? PL::bytes : CL::bytes;
    static_assert(LDS + 64 <= 160 * 1024, "LDS budget");
    auto kf = fused_kernel<DK, DV, AS, LG>;
    static std::atomic<unsigned long long> done{0};
    hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(kf), (int)LDS, done);
    if (e != hipSuccess) return e;
    const Topology tp = topology();
    const int NC = p.T / C;
    unsigned char* base = reinterpret_cast<unsigned char*>(ws);
    FusedCfg cfg;
    cfg.flags = reinterpret_cast<int*>(base + flags_offset<DK, DV>(p.BH, p.T));
    cfg.ctl = cfg.flags + (((size_t)p.BH * NC + 63) & ~size_t(63));
    cfg.NX = tp.nx;
    cfg.CAP = (tp.ncu / tp.nx) / 4 > 0 ? (tp.ncu / tp.nx) / 4 : 1;
    cfg.spin = 1u << 23;
    const size_t nclr = (((size_t)p.BH * NC + 63) & ~size_t(63)) + 64;
    hipLaunchKernelGGL(fz_clear, dim3((unsigned)((nclr + 1023) / 1024 < 1024 ? (nclr + 1023) / 1024 : 1024)),
                       dim3(1024), 0, st, cfg.flags, nclr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kf, dim3((unsigned)tp.ncu), dim3(256), LDS, st, p, base, cfg);
    return hipGetLastError();
}

// the two-kernel form (the producer over every chunk, then the chains)
template <int DK, int DV, bool AS, bool LG>
static hipError_t launch_split_t(const FwdParams& p, void* ws, hipStream_t st) {
    using PL = ProdLayout<DK, DV>;
    using CL = ChainLayout<DK, DV>;
    auto kp = prod_kernel<DK, DV, AS, LG>;
    auto kc = chain_kernel<DK, DV>;
    static std::atomic<unsigned long long> done_p{0}, done_c{0};
    hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(kp), (int)PL::bytes, done_p);
    if (e != hipSuccess) return e;
    e = ensure_dyn_lds(reinterpret_cast<const void*>(kc), (int)CL::bytes, done_c);
    if (e != hipSuccess) return e;
    const Topology tp = topology();
    const int total = p.BH * (p.T / C);
    const int gp = total < tp.ncu ? total : tp.ncu;
    hipLaunchKernelGGL(kp, dim3((unsigned)gp), dim3(PL::NT), PL::bytes, st, p, reinterpret_cast<unsigned char*>(ws));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kc, dim3((unsigned)(p.BH * CL::WPH)), dim3(256), CL::bytes, st, p,
                       reinterpret_cast<const unsigned char*>(ws));
    return hipGetLastError();
}

template <int DK, int DV, bool AS, bool LG>
static hipError_t launch_pick(const FwdParams& p, void* ws, hipStream_t st) {
    if (p.flags & GDR_FWD_SPLIT) return launch_split_t<DK, DV, AS, LG>(p, ws, st);
    return launch_t<DK, DV, AS, LG>(p, ws, st);
}

template <int DK, int DV>
static hipError_t launch_modes(const FwdParams& p, void* ws, hipStream_t st) {
    const bool as = (p.flags & GDR_ALPHA_SCALAR) != 0;
    const bool lg = (p.flags & GDR_GATE_LOGITS) != 0;
    if (as) return lg ? launch_pick<DK, DV, true, true>(p, ws, st) : launch_pick<DK, DV, true, false>(p, ws, st);
    return lg ? launch_pick<DK, DV, false, true>(p, ws, st) : launch_pick<DK, DV, false, false>(p, ws, st);
}

// packed sequences: the producer over every chunk, then the chains
template <int DK, int DV, bool AS, bool LG>
static hipError_t launch_vl_t(const FwdParams& p, void* records, hipStream_t st) {
    using PL = ProdLayout<DK, DV>;
    using CL = ChainLayout<DK, DV>;
    auto kp = prod_kernel_vl<DK, DV, AS, LG>;
    auto kc = chain_kernel_vl<DK, DV>;
    static std::atomic<unsigned long long> done_p{0}, done_c{0};
    hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(kp), (int)PL::bytes, done_p);
    if (e != hipSuccess) return e;
    e = ensure_dyn_lds(reinterpret_cast<const void*>(kc), (int)CL::bytes, done_c);
    if (e != hipSuccess) return e;
    const Topology tp = topology();
    hipLaunchKernelGGL(kp, dim3((unsigned)tp.ncu), dim3(256), PL::bytes, st, p,
                       reinterpret_cast<unsigned char*>(records));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long chains = (long long)p.nseq * p.BH * CL::WPH;
    hipLaunchKernelGGL(kc, dim3((unsigned)chains), dim3(256), CL::bytes, st, p,
                       reinterpret_cast<const unsigned char*>(records));
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_vl_modes(const FwdParams& p, void* records, hipStream_t st) {
    const bool as = (p.flags & GDR_ALPHA_SCALAR) != 0;
    const bool lg = (p.flags & GDR_GATE_LOGITS) != 0;
    if (as) return lg ? launch_vl_t<DK, DV, true, true>(p, records, st) : launch_vl_t<DK, DV, true, false>(p, records, st);
    return lg ? launch_vl_t<DK, DV, false, true>(p, records, st) : launch_vl_t<DK, DV, false, false>(p, records, st);
}

template <int DK, int DV>
static size_t vl_records_bytes(int H, long long T, int nseq) {
    return (size_t)H * packed_max_chunks(T, nseq) * RecF<DK, DV>::bytes;
}

}  // namespace fz

static size_t fz_vl_records_bytes(int H, long long T, int nseq, int dk, int dv) {
    if (dk == 128 && dv == 128) return fz::vl_records_bytes<128, 128>(H, T, nseq);
    if (dk == 64 && dv == 64) return fz::vl_records_bytes<64, 64>(H, T, nseq);
    if (dk == 128 && dv == 64) return fz::vl_records_bytes<128, 64>(H, T, nseq);
    if (dk == 64 && dv == 128) return fz::vl_records_bytes<64, 128>(H, T, nseq);
    return 0;
}

size_t fwd_fz_varlen_workspace_bytes(int H, long long T, int nseq, int dk, int dv) {
    const size_t rb = fz_vl_records_bytes(H, T, nseq, dk, dv);
    if (rb == 0 || H < 1 || nseq < 1 || T < 0) return 0;
    return ((rb + 255) & ~size_t(255)) + packed_prep_bytes(T, nseq);
}

hipError_t launch_fwd_fz_varlen(const FwdParams& p0, int dk, int dv, void* ws, size_t ws_bytes, hipStream_t st) {
    const size_t need = fwd_fz_varlen_workspace_bytes(p0.BH, p0.T, p0.nseq, dk, dv);
    if (need == 0 || ws_bytes < need || !p0.cu_seqlens) return hipErrorInvalidValue;
    FwdParams p = p0;
    const size_t rb = (fz_vl_records_bytes(p.BH, p.T, p.nseq, dk, dv) + 255) & ~size_t(255);
    unsigned char* prep = reinterpret_cast<unsigned char*>(ws) + rb;
    hipError_t e = launch_packed_prep(p.cu_seqlens, p.nseq, p.T, prep, &p.chunk_off, &p.chunk_tab, &p.seq_order, st);
    if (e != hipSuccess) return e;
    if (dk == 128 && dv == 128) return fz::launch_vl_modes<128, 128>(p, ws, st);
    if (dk == 64 && dv == 64) return fz::launch_vl_modes<64, 64>(p, ws, st);
    if (dk == 128 && dv == 64) return fz::launch_vl_modes<128, 64>(p, ws, st);
    if (dk == 64 && dv == 128) return fz::launch_vl_modes<64, 128>(p, ws, st);
    return hipErrorInvalidValue;
}

size_t fwd_fz_workspace_bytes(int BH, int T, int dk, int dv) {
    size_t off = 0;
    if (dk == 128 && dv == 128) off = fz::flags_offset<128, 128>(BH, T);
    else if (dk == 64 && dv == 64) off = fz::flags_offset<64, 64>(BH, T);
    else if (dk == 128 && dv == 64) off = fz::flags_offset<128, 64>(BH, T);
    else if (dk == 64 && dv == 128) off = fz::flags_offset<64, 128>(BH, T);
    else return 0;
    // chunk flags (padded to 64) and 64 control words, int32
    return off + ((((size_t)BH * (size_t)(T / fz::C) + 63) & ~size_t(63)) + 64) * 4;
}

hipError_t launch_fwd_fz(const FwdParams& p, int dk, int dv, void* ws, hipStream_t st) {
    if (p.T == 0 || p.T % fz::C != 0) return hipErrorInvalidValue;
    if (dk == 128 && dv == 128) return fz::launch_modes<128, 128>(p, ws, st);
    if (dk == 64 && dv == 64) return fz::launch_modes<64, 64>(p, ws, st);
    if (dk == 128 && dv == 64) return fz::launch_modes<128, 64>(p, ws, st);
    if (dk == 64 && dv == 128) return fz::launch_modes<64, 128>(p, ws, st);
    return hipErrorInvalidValue;
}

}  // namespace gdr
