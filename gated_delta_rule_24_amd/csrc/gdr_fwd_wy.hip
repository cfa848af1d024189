// Two-pass chunkwise forward of the gated delta rule (bf16 activations, chunk
// 64, d_k and d_v in {64, 128}); used when the caller provides a workspace.
//
// The WY form of a chunk (Gated DeltaNet-2 Q&A page, Q4; "Gated DeltaNet-2
// Review" §3-2 item 5) splits into a part that does not depend on the state
// and a short state chain.  With E, Qs, Kh, X, A, P as in the other forward
// kernels, T = (I + A)^-1 and
//   W = T E,   Ũ = T X,   Q̃ = Qs - P W,
// the chunk update is
//   S' = diag(e^{g_C}) S,   U = Ũ - W S',   O = Q̃ S' + P Ũ,   S <- S' + Kh^T U.
//
// Pass 1 (wy_kernel) computes W, Q̃, Ũ, P, Kh^T and e^{g_C} for every chunk of
// every head in parallel: all the element-wise gate work, the exponentials and
// the triangular inverse happen here, once per chunk.  It writes them to the
// workspace as ready-made MFMA fragments (each 16-byte lane piece in the order
// the state pass reads it).
// Pass 2 (chain_kernel) runs the state chain: one workgroup per (head, two
// 16-column strips of the state).  One wave keeps the fp32 strips in MFMA
// accumulators and issues only the chain (Y = W S', U = Ũ - Y, S += Kh^T U);
// a second wave computes the chunk's output O = Q̃ S' + P Ũ from the S'
// fragments the first publishes in LDS.  Both read their fragments directly
// from the workspace (L2) one chunk ahead of use, and the chunks after that
// are touched so they are already in L2.  Every fragment feeds both strips.
#include "gdr_device.h"
#include "gdr_launch.h"
#include "gdr_wy.h"

namespace gdr {

namespace wy {

// ---------------------------------------------------------------------------
// pass 1: chunk-local WY operands
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct PrepLayout {
    static constexpr int NT = 256;          // threads per workgroup
    static constexpr int LDE = DK + 8;      // E, Qs, Kh rows        [C][LDE]  f16
    static constexpr int LDT = C + 8;       // token-contiguous rows  [*][LDT]  f16
    static constexpr int LDT2 = C + 2;      // E^T and X^T rows (odd dword stride: their
                                            // transposed writes spread over the banks)
    static constexpr int LDA = C + 4;       // A                      [C][LDA]  fp32
    static constexpr int CO = DK / 8;       // key-side channel octets per row
    static constexpr int NPART = NT / CO;   // token parts of the key-side mapping
    static constexpr int TPP = C / NPART;   // tokens per thread
    static constexpr int VO = DV / 8;
    static constexpr int XPART = NT / VO;
    static constexpr int XTP = C / XPART;
    static constexpr size_t oE = 0;
    static constexpr size_t oQ = oE + (size_t)C * LDE * 2;
    static constexpr size_t oK = oQ + (size_t)C * LDE * 2;
    static constexpr size_t oEt = oK + (size_t)C * LDE * 2;     // E^T  [DK][LDT2]
    static constexpr size_t oXt = oEt + (size_t)DK * LDT2 * 2;  // X^T  [DV][LDT2]
    static constexpr size_t oT = (oXt + (size_t)DV * LDT2 * 2 + 15) & ~size_t(15);   // T [C][LDT]
    static constexpr size_t oP = oT + (size_t)C * LDT * 2;      // P    [C][LDT]
    static constexpr size_t oZ = oP + (size_t)C * LDT * 2;      // Z^T  [C/2][LDT]
    static constexpr size_t oA = oZ + (size_t)(C / 2) * LDT * 2;
    static constexpr size_t oTot = oA + (size_t)C * LDA * 4;    // [NPART][DK] fp32
    // W^T [DK][LDT] reuses the space of A and the prefix partials: it is written
    // after the last read of A (the doubling) and read before the next chunk's
    // prefix is written
    static constexpr size_t oWt = oA;
    static_assert((size_t)DK * LDT * 2 <= (size_t)C * LDA * 4 + (size_t)NPART * DK * 4, "W^T alias");
    static constexpr int LDD = 20;                               // diagonal blocks of A, transposed
    static constexpr size_t oAd = oTot + (size_t)NPART * DK * 4; // [C/16][16][LDD] fp32
    static constexpr size_t oFl = oAd + (size_t)(C / 16) * 16 * LDD * 4;   // [NT/64] int
    static constexpr size_t bytes = oFl + (size_t)(NT / 64) * 4;
};

// The chunk of work item idx (CN chunks per head): its first token in the
// activation streams and its number of tokens.  Fixed length: item =
// (sequence, chunk).  Packed sequences (VL): item = (head, chunk r of the
// head's concatenated sequences), looked up in the chunk table; a sequence's
// last chunk may be partial.
template <bool VL>
__device__ __forceinline__ void chunk_item(const FwdParams& p, int CN, int idx, size_t& tok0, int& len) {
    const int h = idx / CN, r = idx - h * CN;
    if constexpr (VL) {
        const int2 e = reinterpret_cast<const int2*>(p.chunk_tab)[r];
        tok0 = (size_t)h * p.T + (size_t)e.x;
        len = e.y;
    } else {
        tok0 = (size_t)h * p.T + (size_t)r * C;
        len = C;
    }
}

template <int DK, int DV, bool AS, bool BS, bool WS, bool BL, bool VL, bool LG>
__global__ __launch_bounds__((PrepLayout<DK, DV>::NT), 1) void wy_kernel(FwdParams p, unsigned char* ws) {
    using L = PrepLayout<DK, DV>;
    constexpr int NT = L::NT, NW = NT / 64;
    using R = Rec<DK, DV>;
    static_assert(L::bytes <= 160 * 1024, "LDS budget");
    static_assert(L::NPART >= 1 && L::TPP >= 1 && L::XTP >= 1, "mapping");
    constexpr int LDE = L::LDE, LDT = L::LDT, LDT2 = L::LDT2, LDA = L::LDA;
    constexpr int CO = L::CO, TPP = L::TPP, VO = L::VO, XTP = L::XTP;
    constexpr int NB = C / 16, NKK = DK / 32, NST = DV / 16;

    extern __shared__ __align__(16) unsigned char smem[];
    _Float16* sE = reinterpret_cast<_Float16*>(smem + L::oE);
    _Float16* sQ = reinterpret_cast<_Float16*>(smem + L::oQ);
    _Float16* sK = reinterpret_cast<_Float16*>(smem + L::oK);
    _Float16* sEt = reinterpret_cast<_Float16*>(smem + L::oEt);
    _Float16* sXt = reinterpret_cast<_Float16*>(smem + L::oXt);
    _Float16* sWt = reinterpret_cast<_Float16*>(smem + L::oWt);
    _Float16* sT = reinterpret_cast<_Float16*>(smem + L::oT);
    _Float16* sP = reinterpret_cast<_Float16*>(smem + L::oP);
    _Float16* sZ = reinterpret_cast<_Float16*>(smem + L::oZ);
    float* sA = reinterpret_cast<float*>(smem + L::oA);
    float* sTot = reinterpret_cast<float*>(smem + L::oTot);
    float* sAd = reinterpret_cast<float*>(smem + L::oAd);
    int* sFl = reinterpret_cast<int*>(smem + L::oFl);
    constexpr int LDD = L::LDD;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = 4 * (lane >> 4);
    const int co = tid % CO, part = tid / CO;       // channels 8co.., tokens part*TPP..
    const int vo = tid % VO, xpart = tid / VO;      // columns 8vo.., tokens xpart*XTP..
    const int CN = VL ? p.chunk_off[p.nseq] : p.T / C;      // chunks per head
    const int total = p.BH * CN;
    const uint16_t* bg = reinterpret_cast<const uint16_t*>(p.b);
    const uint16_t* vg = reinterpret_cast<const uint16_t*>(p.v);
    const uint16_t* wg = reinterpret_cast<const uint16_t*>(p.w);

    // upper tiles of T and P stay zero (only lower tiles are written per chunk)
    for (int idx = tid; idx < C * C; idx += NT) {
        const int r = idx / C, c = idx % C;
        if ((c >> 4) > (r >> 4)) {
            sT[r * LDT + c] = (_Float16)0.f;
            sP[r * LDT + c] = (_Float16)0.f;
        }
    }

    // raw inputs of one chunk: 8 channels x TPP tokens (key side), 8 columns x XTP
    // tokens (value side), in 16-byte loads (few enough to stay in flight together)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 rq[TPP], rk[TPP], rb[TPP], rv[XTP], rw[XTP];
    floatx4 rla[TPP][2];
    // The loads of a chunk are issued in three groups spread over the previous
    // chunk's phases (q and k, then b and log alpha, then v and w), so that
    // their transfer overlaps computation instead of stalling one issue point.
    // (packed sequences: the tokens past a sequence's end in its last chunk read
    // as zeros, log alpha 0 included, so they leave the state unchanged; the
    // loads themselves go to the chunk's first token)
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    // gates given as logits (LG, GDR_GATE_LOGITS): absent tokens get the decay
    // logit +inf (log sigmoid = 0)
    constexpr bool lg = LG;
    const float la_absent = lg ? __builtin_inff() : 0.f;
    const floatx4 la_absent4 = {la_absent, la_absent, la_absent, la_absent};
    auto issue = [&](size_t tok0, int len, int group) __attribute__((always_inline)) {
        if (group < 2) {
#pragma unroll
            for (int j = 0; j < TPP; ++j) {
                const int row = part * TPP + j;
                const bool ok = !VL || row < len;
                const size_t t = tok0 + (ok ? row : 0);
                const size_t ix = t * DK + 8 * co;
                if (group == 0) {
                    rq[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.q) + ix);
                    rk[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.k) + ix);
                    if (!ok) rq[j] = rk[j] = z4;
                } else {
                    if constexpr (BS) rb[j][0] = bg[t];
                    else rb[j] = *reinterpret_cast<const u32x4*>(bg + ix);
                    if constexpr (AS) {
                        rla[j][0][0] = p.la[t];
                    } else {
                        rla[j][0] = *reinterpret_cast<const floatx4*>(p.la + ix);
                        rla[j][1] = *reinterpret_cast<const floatx4*>(p.la + ix + 4);
                    }
                    if (!ok) {
                        rb[j] = z4;
                        rla[j][0] = rla[j][1] = la_absent4;
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < XTP; ++j) {
                const int row = xpart * XTP + j;
                const bool ok = !VL || row < len;
                const size_t t = tok0 + (ok ? row : 0);
                const size_t ix = t * DV + 8 * vo;
                rv[j] = *reinterpret_cast<const u32x4*>(vg + ix);
                if constexpr (WS) rw[j][0] = wg[t];
                else rw[j] = *reinterpret_cast<const u32x4*>(wg + ix);
                if (!ok) rv[j] = rw[j] = z4;
            }
        }
    };
    auto unpack8 = [](u32x4 u, float (&f)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    };

    int idx = blockIdx.x;
    if (idx < total) {
        size_t tok0;
        int len;
        chunk_item<VL>(p, CN, idx, tok0, len);
        issue(tok0, len, 0);
        issue(tok0, len, 1);
        issue(tok0, len, 2);
    }
    for (; idx < total; idx += gridDim.x) {
        const int nx = idx + (int)gridDim.x < total ? idx + (int)gridDim.x : idx;
        // the next item's chunk (its table entry loads while this one is processed)
        size_t ntok0;
        int nlen;
        chunk_item<VL>(p, CN, nx, ntok0, nlen);
        constexpr size_t RB = BL ? R::bwd_bytes : R::bytes;
        unsigned char* rec = ws + (size_t)idx * RB;
        // ---------------- element-wise: in-chunk prefix, E, Qs, Kh, X (fp32 -> f16)
        float gl[TPP][8];
        floatx4 off[2];
        if (lg) {
            // decay logits -> log alpha = log sigmoid(logit), fp32
#pragma unroll
            for (int j = 0; j < TPP; ++j)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!AS || (hh == 0 && i == 0)) rla[j][hh][i] = gate_log_sigmoid(rla[j][hh][i]);
        }
        {
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
            // prefix over the token parts: within the wave across the lane groups
            // (lanes CO apart hold the same channels), then over the waves in LDS
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
            for (int i = 0; i < 8; ++i) off[i >> 2][i & 3] = inc[i] - run[i];
            if (lane >= 64 - CO) {
                floatx4 r0, r1;
#pragma unroll
                for (int i = 0; i < 4; ++i) { r0[i] = inc[i]; r1[i] = inc[4 + i]; }
                *reinterpret_cast<floatx4*>(sTot + wave * DK + 8 * co) = r0;
                *reinterpret_cast<floatx4*>(sTot + wave * DK + 8 * co + 4) = r1;
            }
        }
        lds_barrier();
        int over = 0;
        {
            floatx4 gC[2] = {zero4(), zero4()};
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                const floatx4 t0 = *reinterpret_cast<const floatx4*>(sTot + w2 * DK + 8 * co);
                const floatx4 t1 = *reinterpret_cast<const floatx4*>(sTot + w2 * DK + 8 * co + 4);
                if (w2 < wave) { off[0] += t0; off[1] += t1; }
                gC[0] += t0;
                gC[1] += t1;
            }
            if (part == 0) {
                constexpr float lim = kDecayLimit * kLog2e;
#pragma unroll
                for (int i = 0; i < 8; ++i) over |= !(gl[0][i] - gC[i >> 2][i & 3] <= lim);
                floatx4 e0, e1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e0[i] = __builtin_amdgcn_exp2f(gC[0][i]);
                    e1[i] = __builtin_amdgcn_exp2f(gC[1][i]);
                }
                st_nt(rec + R::G + 32 * co, e0);
                st_nt(rec + R::G + 32 * co + 16, e1);
            }
            _Float16 et[8][TPP];
#pragma unroll
            for (int j = 0; j < TPP; ++j) {
                const int t = part * TPP + j;
                float q8[8], k8[8], b8[8];
                unpack8(rq[j], q8);
                unpack8(rk[j], k8);
                if constexpr (BS) {
                    float bs = __uint_as_float(rb[j][0] << 16);
                    if (lg) bs = gate_sigmoid(bs);
#pragma unroll
                    for (int i = 0; i < 8; ++i) b8[i] = bs;
                } else {
                    unpack8(rb[j], b8);
                    if (lg) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) b8[i] = gate_sigmoid(b8[i]);
                    }
                }
                half8 e, qq, kk;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float d = off[i >> 2][i & 3] + gl[j][i] - gC[i >> 2][i & 3];
                    const float eg = __builtin_amdgcn_exp2f(d), ek = __builtin_amdgcn_exp2f(-d);
                    e[i] = (_Float16)(b8[i] * k8[i] * eg);
                    qq[i] = (_Float16)(q8[i] * eg);
                    kk[i] = (_Float16)(k8[i] * ek);
                    et[i][j] = e[i];
                }
                *reinterpret_cast<half8*>(sE + t * LDE + 8 * co) = e;
                *reinterpret_cast<half8*>(sQ + t * LDE + 8 * co) = qq;
                *reinterpret_cast<half8*>(sK + t * LDE + 8 * co) = kk;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < TPP; j += 2) {
                    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                    h2 v;
                    v[0] = et[i][j];
                    v[1] = et[i][j + 1];
                    *reinterpret_cast<h2*>(sEt + (8 * co + i) * LDT2 + part * TPP + j) = v;
                }
            _Float16 xt[8][XTP];
#pragma unroll
            for (int j = 0; j < XTP; ++j) {
                float v8[8], w8[8];
                unpack8(rv[j], v8);
                if constexpr (WS) {
                    float wsv = __uint_as_float(rw[j][0] << 16);
                    if (lg) wsv = gate_sigmoid(wsv);
#pragma unroll
                    for (int i = 0; i < 8; ++i) w8[i] = wsv;
                } else {
                    unpack8(rw[j], w8);
                    if (lg) {
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
                    *reinterpret_cast<h2*>(sXt + (8 * vo + i) * LDT2 + xpart * XTP + j) = v;
                }
        }
        {
            // block-wide OR of the decay check through LDS
            const int any = __any(over);
            if (lane == 0) sFl[wave] = any;
            lds_barrier();
            over = 0;
#pragma unroll
            for (int w = 0; w < NT / 64; ++w) over |= sFl[w];
        }
        if (tid == 0) *reinterpret_cast<int*>(rec + R::G + DK * 4) = over;
        // the next chunk's inputs load while this one is processed
        issue(ntok0, nlen, 0);

        // ---------------- A = strict_lower(E Kh^T) (fp32), P = lower(Qs Kh^T) (f16)
        // One lower tile (mt, nt) per task gives both its A and its P tile: the
        // Kh fragments are read once and the two MFMA chains interleave.
        constexpr int NLT = NB * (NB + 1) / 2;
#pragma unroll
        for (int s2 = 0; s2 < (NLT + NW - 1) / NW; ++s2) {
            const int task = wave + NW * s2;
            if (task >= NLT) break;
            int t = task, mt = 0;
            while (t > mt) { t -= mt + 1; ++mt; }
            const int nt = t;
            const _Float16* xe = sE + (16 * mt + r16) * LDE + 2 * g4;
            const _Float16* xq = sQ + (16 * mt + r16) * LDE + 2 * g4;
            const _Float16* xk = sK + (16 * nt + r16) * LDE + 2 * g4;
            half8 fe[NKK], fq[NKK], fk[NKK];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                fe[kk] = ld_h8(xe + 32 * kk);
                fk[kk] = ld_h8(xk + 32 * kk);
                fq[kk] = ld_h8(xq + 32 * kk);
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
                    sA[r * LDA + c] = a[i];
                }
                // diagonal blocks also transposed: sAd[blk][col][row]
                if (mt == nt) *reinterpret_cast<floatx4*>(sAd + (mt * 16 + r16) * LDD + g4) = a;
            }
            {
                // P^T tile (s = 16 nt + .., t = 16 mt + ..): lane holds P[16mt + r16][16nt + g4 + i]
                const int tr = 16 * mt + r16;
                floatx4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = (16 * nt + g4 + i <= tr) ? acp[i] : 0.f;
                *reinterpret_cast<half4*>(sP + tr * LDT + 16 * nt + g4) = to_h4(v);
            }
        }
        lds_barrier();
        issue(ntok0, nlen, 1);
        if (wave == 0) {
            // diagonal 16x16 blocks of T: right-looking forward substitution in fp32,
            // lane (blk, column jc), the columns of A streamed from the transposed copy
            const int blk = lane >> 4, jc = lane & 15;
            const float* ad = sAd + blk * 16 * LDD;
            floatx4 acol[2][4];
#pragma unroll
            for (int q = 0; q < 4; ++q) acol[0][q] = *reinterpret_cast<const floatx4*>(ad + 4 * q);
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == jc) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                if (m + 1 < 15) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acol[(m + 1) & 1][q] = *reinterpret_cast<const floatx4*>(ad + (m + 1) * LDD + 4 * q);
                }
                const float xm = x[m];
#pragma unroll
                for (int r = m + 1; r < 16; ++r) x[r] -= acol[m & 1][r >> 2][r & 3] * xm;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sT[(16 * blk + r) * LDT + 16 * blk + jc] = (_Float16)x[r];
        } else {
            // meanwhile: fragments of P (K = tokens) and Kh^T (K = tokens)
            // (the backward reads P^T instead: no P rows then)
            constexpr int NPB = BL ? 0 : NB * (C / 32), NKB = (DK / 16) * (C / 32);
            for (int task = wave - 1; task < NPB + NKB; task += NT / 64 - 1) {
                if (task < NPB) {
                    const int rt = task / (C / 32), kk = task % (C / 32);
                    const _Float16* src = sP + (16 * rt + r16) * LDT + 32 * kk + g4;
                    st_nt(rec + R::P + ((size_t)(rt * (C / 32) + kk) * 64 + lane) * 16,
                        cat8(ld_h4(src), ld_h4(src + 16)));
                } else {
                    const int tk = task - NPB, mt = tk / (C / 32), kk = tk % (C / 32);
                    const _Float16* src = sK + (32 * kk + g4) * LDE + 16 * mt + r16;
                    st_nt(rec + R::K + ((size_t)(mt * (C / 32) + kk) * 64 + lane) * 16,
                        cat8(ld_col4(src, LDE), ld_col4(src + 16 * LDE, LDE)));
                }
            }
        }
        lds_barrier();
        // ---------------- off-diagonal blocks by doubling: T_BA = -T_BB (A_BA T_AA)
#pragma unroll
        for (int sz = 16; sz < C; sz *= 2) {
            const int nsub = sz / 16, ntask = (C / (2 * sz)) * nsub * nsub;
            for (int task = wave; task < ntask; task += NT / 64) {
                const int pr = task / (nsub * nsub), mi = (task / nsub) % nsub, ni = task % nsub;
                const int a0 = 2 * sz * pr, b0 = a0 + sz;
                floatx4 acc = zero4();
#pragma unroll
                for (int k = 0; k < sz; k += 16) {
                    const floatx4 av = *reinterpret_cast<const floatx4*>(sA + (b0 + 16 * mi + r16) * LDA + a0 + k + g4);
                    acc = mfma16(to_h4(av), ld_col4(sT + (a0 + k + g4) * LDT + a0 + 16 * ni + r16, LDT), acc);
                }
                // Z^T[col][row]
                *reinterpret_cast<half4*>(sZ + (pr * sz + 16 * ni + r16) * LDT + 16 * mi + g4) = to_h4(acc);
            }
            lds_barrier();
            for (int task = wave; task < ntask; task += NT / 64) {
                const int pr = task / (nsub * nsub), mi = (task / nsub) % nsub, ni = task % nsub;
                const int a0 = 2 * sz * pr, b0 = a0 + sz;
                floatx4 acc = zero4();
#pragma unroll
                for (int k = 0; k < sz; k += 16)
                    acc = mfma16(ld_h4(sT + (b0 + 16 * mi + r16) * LDT + b0 + k + g4),
                                 ld_h4(sZ + (pr * sz + 16 * ni + r16) * LDT + k + g4), acc);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sT[(b0 + 16 * mi + g4 + i) * LDT + a0 + 16 * ni + r16] = (_Float16)(-acc[i]);
            }
            lds_barrier();
        }
        // ---------------- W^T = E^T T^T (fragments of W out, W^T kept) and Ũ = T X.
        // T's upper tiles are zero, so every product runs over the full K = C.
        // Pairs of 16-token blocks form the 32-deep MFMA operands (both sides in
        // the same K order).
        static_assert((NB * NKK) % NW == 0 && (NST * (C / 32)) % NW == 0, "tasks per wave");
#pragma unroll
        for (int s2 = 0; s2 < NB * NKK / (NT / 64); ++s2) {
            const int task = wave + (NT / 64) * s2;
            const int rt = task / NKK, kk = task % NKK;
            half4 fx[2][NB], fy[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                fy[k] = ld_h4(sT + (16 * rt + r16) * LDT + 16 * k + g4);
#pragma unroll
                for (int h = 0; h < 2; ++h) fx[h][k] = ld_h4w(sEt + (32 * kk + 16 * h + r16) * LDT2 + 16 * k + g4);
            }
            floatx4 acc[2] = {zero4(), zero4()};
#pragma unroll
            for (int k = 0; k < NB; k += 2)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    acc[h] = mfma32(cat8(fx[h][k], fx[h][k + 1]), cat8(fy[k], fy[k + 1]), acc[h]);
            st_nt(rec + R::W + ((size_t)(rt * NKK + kk) * 64 + lane) * 16,
                cat8(to_h4(acc[0]), to_h4(acc[1])));
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sWt[(32 * kk + 16 * h + g4 + i) * LDT + 16 * rt + r16] = (_Float16)acc[h][i];
        }
#pragma unroll
        for (int s2 = 0; s2 < NST * (C / 32) / (NT / 64); ++s2) {
            const int task = wave + (NT / 64) * s2;
            const int nt = task / (C / 32), kk = task % (C / 32);
            half4 fx[2][NB], fy[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                fy[k] = ld_h4w(sXt + (16 * nt + r16) * LDT2 + 16 * k + g4);
#pragma unroll
                for (int h = 0; h < 2; ++h) fx[h][k] = ld_h4(sT + (16 * (2 * kk + h) + r16) * LDT + 16 * k + g4);
            }
            floatx4 acc[2] = {zero4(), zero4()};
#pragma unroll
            for (int k = 0; k < NB; k += 2)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    acc[h] = mfma32(cat8(fx[h][k], fx[h][k + 1]), cat8(fy[k], fy[k + 1]), acc[h]);
            st_nt(rec + R::U + ((size_t)(nt * (C / 32) + kk) * 64 + lane) * 16,
                cat8(to_h4(acc[0]), to_h4(acc[1])));
        }
        lds_barrier();
        issue(ntok0, nlen, 2);
        // ---------------- Q̃^T = Qs^T - W^T P^T (fragments of Q̃ out); P's upper tiles are zero
#pragma unroll
        for (int s2 = 0; s2 < NB * NKK / (NT / 64); ++s2) {
            const int task = wave + (NT / 64) * s2;
            const int rt = task / NKK, kk = task % NKK;
            half4 fx[2][NB], fy[NB], fq[2];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                fy[k] = ld_h4(sP + (16 * rt + r16) * LDT + 16 * k + g4);
#pragma unroll
                for (int h = 0; h < 2; ++h) fx[h][k] = ld_h4(sWt + (32 * kk + 16 * h + r16) * LDT + 16 * k + g4);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) fq[h] = ld_h4(sQ + (16 * rt + r16) * LDE + 32 * kk + 16 * h + g4);
            floatx4 acc[2] = {zero4(), zero4()};
#pragma unroll
            for (int k = 0; k < NB; k += 2)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    acc[h] = mfma32(cat8(fx[h][k], fx[h][k + 1]), cat8(fy[k], fy[k + 1]), acc[h]);
            const half4 q0 = to_h4(f4(fq[0]) - acc[0]), q1 = to_h4(f4(fq[1]) - acc[1]);
            if constexpr (!BL) st_nt(rec + R::Q + ((size_t)(rt * NKK + kk) * 64 + lane) * 16, cat8(q0, q1));
            if constexpr (BL) {
                // Q̃^T [ch][t] into the (now free) E^T buffer for the channel-row fragments
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sEt[(32 * kk + g4 + i) * LDT2 + 16 * rt + r16] = q0[i];
                    sEt[(32 * kk + 16 + g4 + i) * LDT2 + 16 * rt + r16] = q1[i];
                }
            }
        }
        if constexpr (BL) {
            // fragments for the backward: Kh by rows (K = channels), W^T and Q̃^T by
            // channel rows (K = tokens)
            for (int task = wave; task < NB * NKK; task += NT / 64) {
                const int rt = task / NKK, kk = task % NKK;
                const _Float16* src = sK + (16 * rt + r16) * LDE + 32 * kk + g4;
                st_nt(rec + R::KW + ((size_t)(rt * NKK + kk) * 64 + lane) * 16,
                    cat8(ld_h4(src), ld_h4(src + 16)));
            }
            for (int task = wave; task < (DK / 16) * (C / 32); task += NT / 64) {
                const int mt = task / (C / 32), kk = task % (C / 32);
                const _Float16* src = sWt + (16 * mt + r16) * LDT + 32 * kk + g4;
                st_nt(rec + R::WT + ((size_t)(mt * (C / 32) + kk) * 64 + lane) * 16,
                    cat8(ld_h4(src), ld_h4(src + 16)));
            }
            // P^T and T^T by rows (columns of P and T), K = tokens; blocks left of
            // the diagonal pair (kk < rt / 2) are zero
            for (int task = wave; task < NB * (C / 32); task += NT / 64) {
                const int rt = task / (C / 32), kk = task % (C / 32);
                if (kk < rt / 2) continue;
                const size_t off = ((size_t)(rt * (C / 32) + kk) * 64 + lane) * 16;
                const _Float16* sp = sP + (32 * kk + g4) * LDT + 16 * rt + r16;
                const _Float16* stt = sT + (32 * kk + g4) * LDT + 16 * rt + r16;
                st_nt(rec + R::PT + off, cat8(ld_col4(sp, LDT), ld_col4(sp + 16 * LDT, LDT)));
                st_nt(rec + R::TT + off, cat8(ld_col4(stt, LDT), ld_col4(stt + 16 * LDT, LDT)));
            }
            lds_barrier();
            for (int task = wave; task < (DK / 16) * (C / 32); task += NT / 64) {
                const int mt = task / (C / 32), kk = task % (C / 32);
                const _Float16* src = sEt + (16 * mt + r16) * LDT2 + 32 * kk + g4;
                st_nt(rec + R::QT + ((size_t)(mt * (C / 32) + kk) * 64 + lane) * 16,
                    cat8(ld_h4w(src), ld_h4w(src + 16)));
            }
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// pass 2: the state chain
// ---------------------------------------------------------------------------
// Pass 2.  One workgroup of two waves per (head, NS 16-column strips of the
// state).  Both waves read their operand fragments straight from the
// workspace (L2) into registers two chunks ahead of use (two register sets,
// used alternately):
//   wave 0 (state):  S' = diag(gamma) S, publishes f16 S' fragments in LDS,
//                    Y = W S', U = Ũ - Y, S = S' + Kh^T U;
//   wave 1 (output): O = P Ũ + Q̃ S' for the same chunk, and pulls a share of
//                    the chunks further ahead into L2 (one dword per 128-byte
//                    line; the workgroups of a head split the lines).
// The S' fragments are double-buffered, so one barrier per chunk suffices.
template <int DK, int DV, int NS>
struct StateFrags {
    half8 fw[DK / 32][C / 16], fk[DK / 16][C / 32], ur[NS][C / 32];
    floatx4 gm[DK / 16];
    int flag;
};
template <int DK, int NS>
struct OutFrags {
    half8 fq[DK / 32][C / 16], fp[C / 16][C / 32], ur[NS][C / 32];
    int flag;
};

template <int DK, int DV, int NS, bool VL>
__global__ __launch_bounds__(128, 1) void chain_kernel(FwdParams p, const unsigned char* ws, size_t RB) {
    using R = Rec<DK, DV>;
    constexpr int NGRP = DV / (16 * NS), NKT = DK / 16, NKK = DK / 32, NB = C / 16, NK2 = C / 32;
    __shared__ __align__(16) half8 sSF[2][NS][NKK][64];
    constexpr int LDO = 16 * NS + 4;                    // output tile row stride (floats)
    __shared__ __align__(16) float sO[C * LDO];         // output wave only: O tile, row-major

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // chain bh: a (batch, head) sequence, or for packed sequences sequence
    // bh / H of head bh % H (its state is S0[bh], as [nseq, H] is laid out)
    // (packed sequences: chains of very different lengths, the longest first)
    int bh, ng;                                          // strips NS*ng .. NS*ng+NS-1
    if constexpr (VL) {
        bh = packed_chain(p.seq_order, p.BH, NGRP, (int)blockIdx.x, (int)gridDim.x, ng);
    } else {
        const int lid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
        bh = lid / NGRP;
        ng = lid % NGRP;
    }
    int NC, seq_len;
    size_t tok_base;                                     // the chain's first token
    size_t chunk0;                                       // its first chunk (records, fragments)
    if constexpr (VL) {
        const PackedSpan sp = packed_span(p.cu_seqlens, p.chunk_off, p.nseq, p.BH, p.T, bh);
        NC = sp.NC;
        seq_len = sp.len;
        tok_base = sp.tok0;
        chunk0 = sp.chunk0;
    } else {
        NC = p.T / C;
        seq_len = p.T;
        tok_base = (size_t)bh * p.T;
        chunk0 = (size_t)bh * NC;
    }
    const unsigned char* rec0 = ws + chunk0 * RB;
    const int n_l = lane & 15, g4 = 4 * (lane >> 4);
    auto frag = [&](const unsigned char* rec, size_t off) __attribute__((always_inline)) {
        return *reinterpret_cast<const half8*>(rec + off + (size_t)lane * 16);
    };
    auto recp = [&](int c) __attribute__((always_inline)) {
        return rec0 + (size_t)(c < NC ? c : NC - 1) * RB;
    };

    if (wave == 1) {
        // ------------------------------------------------ output wave
        using F = OutFrags<DK, NS>;
        F fa, fb;
        auto fetch = [&](int c, F& f) __attribute__((always_inline)) {
            const unsigned char* rec = recp(c);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int rt = 0; rt < NB; ++rt) f.fq[kk][rt] = frag(rec, R::Q + (size_t)(rt * NKK + kk) * 1024);
#pragma unroll
            for (int rt = 0; rt < NB; ++rt)
#pragma unroll
                for (int kk = 0; kk <= rt / 2; ++kk) f.fp[rt][kk] = frag(rec, R::P + (size_t)(rt * NK2 + kk) * 1024);
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int kk = 0; kk < NK2; ++kk)
                    f.ur[s][kk] = frag(rec, R::U + (size_t)((NS * ng + s) * NK2 + kk) * 1024);
            f.flag = *reinterpret_cast<const int*>(rec + R::G + DK * 4);
        };
        // L2 prefetch of this workgroup's share of the record's lines; the values
        // are folded two chunks later (never waited on while in flight)
        constexpr int NLINE = (int)(R::bytes / 128);   // the forward part of a record
        constexpr int LPL = (NLINE + 64 * NGRP - 1) / (64 * NGRP);
        uint32_t tacc = 0, ta[LPL] = {}, tb[LPL] = {};
        auto touch = [&](int c, uint32_t (&tr)[LPL]) __attribute__((always_inline)) {
            const unsigned char* rec = recp(c);
#pragma unroll
            for (int r = 0; r < LPL; ++r) {
                tacc ^= tr[r];
                const int li = ng + NGRP * (lane + 64 * r);
                tr[r] = *reinterpret_cast<const uint32_t*>(rec + (size_t)(li < NLINE ? li : NLINE - 1) * 128);
            }
        };
        constexpr int TD = 5;
        if (p.o == nullptr) {
            // state-only pass (the backward's recompute): no output to form, only
            // the L2 touches of the state wave's part of the records ahead of it,
            // with one barrier per chunk as the state wave expects
            constexpr int SLINE = (int)(R::state_bytes / 128);
            constexpr int SPL = (SLINE + 64 * NGRP - 1) / (64 * NGRP);
            static_assert(SPL <= LPL, "touch registers");
            auto touch_s = [&](int c, uint32_t (&tr)[LPL]) __attribute__((always_inline)) {
                const unsigned char* rec = recp(c);
#pragma unroll
                for (int r = 0; r < SPL; ++r) {
                    tacc ^= tr[r];
                    const int li = ng + NGRP * (lane + 64 * r);
                    tr[r] = *reinterpret_cast<const uint32_t*>(rec + (size_t)(li < SLINE ? li : SLINE - 1) * 128);
                }
            };
            if (NC > 0) {
                touch_s(2, ta);
                touch_s(3, tb);
            }
            for (int c = 0; c < NC; c += 2) {
                lds_barrier();
                touch_s(c + TD, ta);
                if (c + 1 < NC) {
                    lds_barrier();
                    touch_s(c + 1 + TD, tb);
                }
            }
#pragma unroll
            for (int r = 0; r < LPL; ++r) tacc ^= ta[r] ^ tb[r];
            // a register sink that keeps the touch loads (no store)
            asm volatile("" ::"v"(tacc));
            return;
        }
        if (NC > 0) {
            touch(2, ta);
            touch(3, tb);
            fetch(0, fa);
            fetch(1, fb);
        }
        bool poisoned = false;
        auto step = [&](int c, F& f, uint32_t (&tr)[LPL]) __attribute__((always_inline)) {
            if (f.flag) poisoned = true;
            floatx4 O[NS][NB];
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int rt = 0; rt < NB; ++rt) {
                    O[s][rt] = zero4();
#pragma unroll
                    for (int kk = 0; kk <= rt / 2; ++kk) O[s][rt] = mfma32(f.fp[rt][kk], f.ur[s][kk], O[s][rt]);
                }
            lds_barrier();                                   // S' of chunk c is published
            half8 sf[NS][NKK];
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) sf[s][kk] = sSF[c & 1][s][kk][lane];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int rt = 0; rt < NB; ++rt)
#pragma unroll
                    for (int s = 0; s < NS; ++s) O[s][rt] = mfma32(f.fq[kk][rt], sf[s][kk], O[s][rt]);
            fetch(c + 2, f);                                 // operands two chunks ahead
            touch(c + TD, tr);
            // the tile goes through LDS (this wave only) so that each lane stores
            // four consecutive columns of a row
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int rt = 0; rt < NB; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sO[(16 * rt + g4 + i) * LDO + 16 * s + n_l] = O[s][rt][i];
            const size_t tok0 = tok_base + (size_t)c * C;
            constexpr int QPR = 4 * NS;                      // column quads per row
#pragma unroll
            for (int r = 0; r < C * QPR / 64; ++r) {
                const int e = lane + 64 * r, row = e / QPR, cq = e % QPR;
                if (VL && c * C + row >= seq_len) continue;  // past the sequence's end
                floatx4 o = *reinterpret_cast<const floatx4*>(sO + row * LDO + 4 * cq);
                if (poisoned) o = o * __builtin_nanf("");
                const size_t base = (tok0 + row) * DV + 16 * NS * ng + 4 * cq;
                if (p.flags & GDR_OUT_BF16) {
                    uint2 u;
                    u.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
                    u.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.o) + base) = u;
                } else {
                    *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(p.o) + base) = o;
                }
            }
        };
        for (int c = 0; c < NC; c += 2) {
            step(c, fa, ta);
            if (c + 1 < NC) step(c + 1, fb, tb);
        }
#pragma unroll
        for (int r = 0; r < LPL; ++r) tacc ^= ta[r] ^ tb[r];
        // a register sink that keeps the touch loads (no store)
        asm volatile("" ::"v"(tacc));
        return;
    }

    // ---------------------------------------------------- state wave
    using F = StateFrags<DK, DV, NS>;
    floatx4 S[NS][NKT];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[s][mt][i] = p.S0 ? p.S0[((size_t)bh * DK + 16 * mt + g4 + i) * DV + 16 * (NS * ng + s) + n_l] : 0.f;
    F fa, fb;
    auto fetch_g = [&](int c, F& f) __attribute__((always_inline)) {
        const unsigned char* rec = recp(c);
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt) f.gm[mt] = *reinterpret_cast<const floatx4*>(rec + R::G + (16 * mt + g4) * 4);
        f.flag = *reinterpret_cast<const int*>(rec + R::G + DK * 4);
    };
    auto fetch_w = [&](int c, F& f) __attribute__((always_inline)) {
        const unsigned char* rec = recp(c);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) f.fw[kk][rt] = frag(rec, R::W + (size_t)(rt * NKK + kk) * 1024);
    };
    auto fetch_u = [&](int c, F& f) __attribute__((always_inline)) {
        const unsigned char* rec = recp(c);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int kk = 0; kk < NK2; ++kk) f.ur[s][kk] = frag(rec, R::U + (size_t)((NS * ng + s) * NK2 + kk) * 1024);
    };
    auto fetch_k = [&](int c, F& f) __attribute__((always_inline)) {
        const unsigned char* rec = recp(c);
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
            for (int kk = 0; kk < NK2; ++kk) f.fk[mt][kk] = frag(rec, R::K + (size_t)(mt * NK2 + kk) * 1024);
    };
    if (NC > 0) {
        fetch_g(0, fa); fetch_w(0, fa); fetch_u(0, fa); fetch_k(0, fa);
        fetch_g(1, fb); fetch_w(1, fb); fetch_u(1, fb); fetch_k(1, fb);
    }
    bool poisoned = false;
    auto step = [&](int c, F& f) __attribute__((always_inline)) {
        const bool was_poisoned = poisoned;
        if (f.flag) poisoned = true;
        // S' = diag(gamma) S and its f16 fragments (K = channels), published for the output wave
        half8 sf[NS][NKK];
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
            for (int s = 0; s < NS; ++s) S[s][mt] = S[s][mt] * f.gm[mt];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                sf[s][kk] = cat8(to_h4(S[s][2 * kk]), to_h4(S[s][2 * kk + 1]));
                sSF[c & 1][s][kk][lane] = sf[s][kk];
            }
        if (p.state_frags) {
            // the backward's copy of S' (after an out-of-range chunk: NaN)
            using SFB = StateFrag<DK, DV>;
            unsigned char* dst = reinterpret_cast<unsigned char*>(p.state_frags) + (chunk0 + c) * SFB::bytes;
            half8 nan8;
#pragma unroll
            for (int e = 0; e < 8; ++e) nan8[e] = (_Float16)__builtin_nanf("");
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk)
                    *reinterpret_cast<half8*>(dst + SFB::block(NS * ng + s, kk) + (size_t)lane * 16) =
                        was_poisoned ? nan8 : sf[s][kk];
        }
        fetch_g(c + 2, f);
        lds_barrier();
        // Y = W S'
        floatx4 Y[NS][NB];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int rt = 0; rt < NB; ++rt) Y[s][rt] = zero4();
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int rt = 0; rt < NB; ++rt)
#pragma unroll
                for (int s = 0; s < NS; ++s) Y[s][rt] = mfma32(f.fw[kk][rt], sf[s][kk], Y[s][rt]);
        fetch_w(c + 2, f);
        // U = Ũ - W S' as B fragments (K = tokens)
        half8 uf[NS][NK2];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int kk = 0; kk < NK2; ++kk)
                uf[s][kk] = cat8(to_h4(f4(lo4(f.ur[s][kk])) - Y[s][2 * kk]),
                                 to_h4(f4(hi4(f.ur[s][kk])) - Y[s][2 * kk + 1]));
        fetch_u(c + 2, f);
        // S = S' + Kh^T U
#pragma unroll
        for (int kk = 0; kk < NK2; ++kk)
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
                for (int s = 0; s < NS; ++s) S[s][mt] = mfma32(f.fk[mt][kk], uf[s][kk], S[s][mt]);
        fetch_k(c + 2, f);
    };
    for (int c = 0; c < NC; c += 2) {
        step(c, fa);
        if (c + 1 < NC) step(c + 1, fb);
    }
    if (p.Sf) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.Sf[((size_t)bh * DK + 16 * mt + g4 + i) * DV + 16 * (NS * ng + s) + n_l] =
                        poisoned ? __builtin_nanf("") : S[s][mt][i];
    }
}

constexpr int kChainStrips = 1;

template <int DK, int DV, bool AS, bool BS, bool WS, bool BL, bool VL>
static hipError_t launch_t(const FwdParams& p, void* ws, hipStream_t st, int passes) {
    using LP = PrepLayout<DK, DV>;
    const bool lg = (p.flags & GDR_GATE_LOGITS) != 0;
    auto kp = lg ? wy_kernel<DK, DV, AS, BS, WS, BL, VL, true> : wy_kernel<DK, DV, AS, BS, WS, BL, VL, false>;
    // the backward's state chain carries two strips per workgroup: half the
    // record reads from the L2 that the reverse chain, running beside it, shares
    // (packed backward 1.88 against 2.00 ms; fixed-length calls unchanged, their
    // state chain becoming the longer of the two).  Packed and fixed-length
    // backwards use the same chain, so equal-length documents give the same bits.
    constexpr int NSC = BL ? 2 : kChainStrips;
    auto ks = chain_kernel<DK, DV, NSC, VL>;
    constexpr size_t RB = BL ? Rec<DK, DV>::bwd_bytes : Rec<DK, DV>::bytes;
    static std::atomic<unsigned long long> done[2];
    {
        const hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(kp), (int)LP::bytes, done[lg]);
        if (e != hipSuccess) return e;
    }
    // (packed sequences: the chunk count is on the device; the WY grid is one
    // workgroup per compute unit)
    const int total = VL ? 1 << 30 : p.BH * (p.T / C);
    int ncu = 256;
    {
        int dev = 0;
        if (hipGetDevice(&dev) == hipSuccess) {
            int n = 0;
            if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
                ncu = n;
        }
    }
    const int gp = total < ncu ? total : ncu;
    if (passes & kWyPass) {
        hipLaunchKernelGGL(kp, dim3((unsigned)gp), dim3(LP::NT), LP::bytes, st, p,
                           reinterpret_cast<unsigned char*>(ws));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (passes & kChainPass) {
        const int chains = VL ? p.nseq * p.BH : p.BH;
        hipLaunchKernelGGL(ks, dim3((unsigned)(chains * (DV / (16 * NSC)))), dim3(128), 0, st, p,
                           reinterpret_cast<const unsigned char*>(ws), RB);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int DK, int DV, bool BL, bool VL = false>
static hipError_t launch_modes(const FwdParams& p, void* ws, hipStream_t st, int passes) {
    const bool as = p.flags & GDR_ALPHA_SCALAR, bs = p.flags & GDR_B_SCALAR, wsc = p.flags & GDR_W_SCALAR;
    const int m = (as ? 4 : 0) | (bs ? 2 : 0) | (wsc ? 1 : 0);
    switch (m) {
        case 0: return launch_t<DK, DV, false, false, false, BL, VL>(p, ws, st, passes);
        case 1: return launch_t<DK, DV, false, false, true, BL, VL>(p, ws, st, passes);
        case 2: return launch_t<DK, DV, false, true, false, BL, VL>(p, ws, st, passes);
        case 3: return launch_t<DK, DV, false, true, true, BL, VL>(p, ws, st, passes);
        case 4: return launch_t<DK, DV, true, false, false, BL, VL>(p, ws, st, passes);
        case 5: return launch_t<DK, DV, true, false, true, BL, VL>(p, ws, st, passes);
        case 6: return launch_t<DK, DV, true, true, false, BL, VL>(p, ws, st, passes);
        default: return launch_t<DK, DV, true, true, true, BL, VL>(p, ws, st, passes);
    }
}

// chunk_off[s] = number of chunks of the packed sequences before s (each
// sequence's last chunk may be partial), chunk_off[nseq] their total; one
// workgroup: contiguous runs of sequences per thread, then a scan of the runs.
// Also order[]: the sequences by descending class floor(log2(chunks)) + 1
// (class 0: empty), any order within a class (the chains are independent, so
// the order changes only which workgroup runs which chain).
__global__ __launch_bounds__(1024) void varlen_chunk_offsets(const int* cu, int n, int* off, int* order) {
    __shared__ int part[1024];
    __shared__ int cls_n[33], cls_fill[33];
    if (threadIdx.x < 33) cls_n[threadIdx.x] = cls_fill[threadIdx.x] = 0;
    const int t = threadIdx.x;
    const int per = (n + 1023) / 1024;
    const int s0 = min(n, t * per), s1 = min(n, s0 + per);
    int sum = 0;
    for (int s = s0; s < s1; ++s) sum += (cu[s + 1] - cu[s] + C - 1) / C;
    part[t] = sum;
    __syncthreads();
    for (int d = 1; d < 1024; d *= 2) {
        const int v = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int run = t ? part[t - 1] : 0;
    for (int s = s0; s < s1; ++s) {
        off[s] = run;
        run += (cu[s + 1] - cu[s] + C - 1) / C;
    }
    if (t == 1023) off[n] = part[1023];
    // longest-first order by class: count, start of each class, then place
    for (int s = s0; s < s1; ++s) {
        const int nc = (cu[s + 1] - cu[s] + C - 1) / C;
        atomicAdd(&cls_n[nc ? 32 - __clz(nc) : 0], 1);
    }
    __syncthreads();
    if (t == 0) {
        int run = 0;
        for (int c = 32; c >= 0; --c) {
            const int k = cls_n[c];
            cls_n[c] = run;
            run += k;
        }
    }
    __syncthreads();
    for (int s = s0; s < s1; ++s) {
        const int nc = (cu[s + 1] - cu[s] + C - 1) / C;
        const int c = nc ? 32 - __clz(nc) : 0;
        order[cls_n[c] + atomicAdd(&cls_fill[c], 1)] = s;
    }
}

// chunk_tab[r] = (first token, token count) of chunk r of the packed sequences
// (r < chunk_off[n]; the grid covers the largest possible chunk count)
__global__ __launch_bounds__(256) void varlen_chunk_table(const int* cu, const int* off, int n,
                                                          int max_chunks, int* tab) {
    const int r = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (r >= max_chunks || r >= off[n]) return;
    int lo = 0, hi = n;                               // off[lo] <= r < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= r) lo = mid;
        else hi = mid;
    }
    const int start = cu[lo] + (r - off[lo]) * C;
    tab[2 * r] = start;
    tab[2 * r + 1] = min(C, cu[lo + 1] - start);
}

}  // namespace wy

bool fwd_wy_supported(int dk, int dv, int chunk, uint32_t flags) {
    if (flags & (GDR_ACT_F32 | GDR_FWD_GENERIC)) return false;
    if (chunk != 64) return false;
    return (dk == 128 || dk == 64) && (dv == 128 || dv == 64);
}

size_t fwd_wy_workspace_bytes(int BH, int T, int dk, int dv, bool bwd_layouts) {
    size_t rec = 0;
    if (dk == 128 && dv == 128) rec = bwd_layouts ? wy::Rec<128, 128>::bwd_bytes : wy::Rec<128, 128>::bytes;
    else if (dk == 64 && dv == 64) rec = bwd_layouts ? wy::Rec<64, 64>::bwd_bytes : wy::Rec<64, 64>::bytes;
    else if (dk == 128 && dv == 64) rec = bwd_layouts ? wy::Rec<128, 64>::bwd_bytes : wy::Rec<128, 64>::bytes;
    else if (dk == 64 && dv == 128) rec = bwd_layouts ? wy::Rec<64, 128>::bwd_bytes : wy::Rec<64, 128>::bytes;
    return (size_t)BH * (size_t)(T / wy::C) * rec;
}

hipError_t launch_fwd_wy(const FwdParams& p, int dk, int dv, void* ws, hipStream_t st, bool bwd_layouts,
                         int passes) {
    if (p.T == 0) return hipErrorInvalidValue;
    if (bwd_layouts) {
        if (dk == 128 && dv == 128) return wy::launch_modes<128, 128, true>(p, ws, st, passes);
        if (dk == 64 && dv == 64) return wy::launch_modes<64, 64, true>(p, ws, st, passes);
        return hipErrorInvalidValue;
    }
    if (dk == 128 && dv == 128) return wy::launch_modes<128, 128, false>(p, ws, st, passes);
    if (dk == 64 && dv == 64) return wy::launch_modes<64, 64, false>(p, ws, st, passes);
    if (dk == 128 && dv == 64) return wy::launch_modes<128, 64, false>(p, ws, st, passes);
    if (dk == 64 && dv == 128) return wy::launch_modes<64, 128, false>(p, ws, st, passes);
    return hipErrorInvalidValue;
}


static size_t round256(size_t n) { return (n + 255) / 256 * 256; }

size_t packed_max_chunks(long long T, int nseq) {
    // every sequence has at most len / C + 1 chunks
    return (size_t)(T / wy::C) + (size_t)nseq;
}

size_t packed_prep_bytes(long long T, int nseq) {
    return round256(((size_t)nseq + 1) * sizeof(int)) + round256(packed_max_chunks(T, nseq) * 2 * sizeof(int)) +
           round256((size_t)nseq * sizeof(int));
}

hipError_t launch_packed_prep(const int* cu_seqlens, int nseq, long long T, void* mem, int** chunk_off,
                              int** chunk_tab, int** seq_order, hipStream_t st) {
    unsigned char* m = reinterpret_cast<unsigned char*>(mem);
    const size_t max_chunks = packed_max_chunks(T, nseq);
    *chunk_off = reinterpret_cast<int*>(m);
    m += round256(((size_t)nseq + 1) * sizeof(int));
    *chunk_tab = reinterpret_cast<int*>(m);
    m += round256(max_chunks * 2 * sizeof(int));
    *seq_order = reinterpret_cast<int*>(m);
    hipLaunchKernelGGL(wy::varlen_chunk_offsets, dim3(1), dim3(1024), 0, st, cu_seqlens, nseq, *chunk_off,
                       *seq_order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wy::varlen_chunk_table, dim3((unsigned)((max_chunks + 255) / 256)), dim3(256), 0, st,
                       cu_seqlens, *chunk_off, nseq, (int)max_chunks, *chunk_tab);
    return hipGetLastError();
}

hipError_t launch_fwd_wy_packed(const FwdParams& p, int dk, int dv, void* records, hipStream_t st,
                                bool bwd_layouts, int passes) {
    if (!p.cu_seqlens || !p.chunk_off || !p.chunk_tab || !p.seq_order) return hipErrorInvalidValue;
    if (bwd_layouts) {
        if (dk == 128 && dv == 128) return wy::launch_modes<128, 128, true, true>(p, records, st, passes);
        if (dk == 64 && dv == 64) return wy::launch_modes<64, 64, true, true>(p, records, st, passes);
        return hipErrorInvalidValue;
    }
    if (dk == 128 && dv == 128) return wy::launch_modes<128, 128, false, true>(p, records, st, passes);
    if (dk == 64 && dv == 64) return wy::launch_modes<64, 64, false, true>(p, records, st, passes);
    if (dk == 128 && dv == 64) return wy::launch_modes<128, 64, false, true>(p, records, st, passes);
    if (dk == 64 && dv == 128) return wy::launch_modes<64, 128, false, true>(p, records, st, passes);
    return hipErrorInvalidValue;
}

}  // namespace gdr
