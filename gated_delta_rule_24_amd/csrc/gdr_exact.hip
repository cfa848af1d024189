// Token-by-token recompute of the forward and of the backward, for the
// (sequence, head) units whose chunkwise result left the range of its
// operands.
//
// The chunkwise kernels that reference the decay to a chunk's end (the
// single-kernel forward, the packed forward, every backward) scale operands
// by e^{±(g_r - g_C)}; when one chunk's decay spans more than their f16 (or
// fp32) range they write NaN to that unit's outputs instead of numbers.  The
// kernels here then recompute exactly those units from the recurrence as the
// pages define it ("Gated DeltaNet-2 — decoupling erase and write in linear
// attention", Q3; "Gated DeltaNet-2 Review" §3-1), one token at a time in
// fp32, where every factor is a single token's decay α = e^{log α} <= 1 and
// nothing can leave its range:
//     S1 = diag(α) S,  r = S1^T (b⊙k),  u = w⊙v - r,  S = S1 + k u^T,  o = S^T q.
// The backward is the reverse mode of the same loop (the gradients of
// L = <dO, o> + <dS_final, S_final>, erase and write gates apart: the Q&A
// page, Q4): states are kept at checkpoints every 64 tokens and each
// segment's per-token states are recomputed into the caller's workspace.
//
// A unit is clean when its marker output is a number: the last token's o row
// (forward) or the first token's dq row (backward; the reverse chain carries
// the NaN to the first chunk).  A workgroup reads the marker and returns at
// once for a clean unit, so on inputs within range these launches cost one
// small kernel each.
//
// The forward runs one wave per (unit, 4 value columns), the state's columns
// being independent under the update (see exact_fwd_kernel).  The backward
// keeps a unit in one workgroup, since its key-side gradients sum over all
// columns.  Layout of the state over a backward workgroup of 256 threads: a 16 x 16 grid of
// tiles of (d_k/16) x (d_v/16) elements; thread t owns tile row t >> 4 and
// tile column t & 15, so a row sum over the columns is a 16-lane shuffle
// reduction and a column sum over the rows is a shuffle over the wave's four
// tile rows plus a four-wave sum through LDS.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {
namespace ex {

constexpr int NT = 256;     // threads per workgroup
constexpr int TB = 8;       // tokens staged in LDS at a time
constexpr int SEG = 64;     // checkpoint interval of the backward (tokens)

struct UnitSpan {
    size_t tok0;            // the unit's first token in the [.., T, d] streams
    int len;
};

// fixed length: unit u is sequence u of T tokens; packed: unit u is sequence
// u / H of head u % H (states [nseq][H] in that order)
__device__ __forceinline__ UnitSpan unit_span(const int* cu, int H, int T, int u) {
    UnitSpan r;
    if (cu) {
        const int s = u / H, h = u % H;
        r.tok0 = (size_t)h * T + (size_t)cu[s];
        r.len = cu[s + 1] - cu[s];
    } else {
        r.tok0 = (size_t)u * T;
        r.len = T;
    }
    return r;
}

template <int DK, int DV>
struct Stage {
    float q[TB][DK], k[TB][DK], a[TB][DK], e[TB][DK], b[TB][DK];
    float x[TB][DV], v[TB][DV], w[TB][DV], dO[TB][DV];
    float red[2][4][DV];     // column sums, double-buffered
    float bred[2][4];        // block sums, double-buffered
};

// Token inputs of tokens tok .. tok + n - 1 into LDS: a = alpha, e = b⊙k,
// x = w⊙v (gates from logits when lg; scalar gates broadcast).
template <int DK, int DV, bool F32>
__device__ void stage_tokens(Stage<DK, DV>& sm, const void* q, const void* k, const void* v, const float* la,
                             const void* b, const void* w, const void* dO, size_t tok, int n, uint32_t flags) {
    const bool as = flags & GDR_ALPHA_SCALAR, bs = flags & GDR_B_SCALAR, wsc = flags & GDR_W_SCALAR;
    const bool lg = flags & GDR_GATE_LOGITS;
    // Every load of the block first (a fixed count per thread, so they are
    // issued together and the block waits for one load latency), then the
    // stores.  Rows past the block's n tokens load its first token (in bounds)
    // and are never read.
    constexpr int MK = (TB * DK + NT - 1) / NT, MV = (TB * DV + NT - 1) / NT;
    float rq[MK], rk[MK], rl[MK], rb[MK], rv[MV], rw[MV], rd[MV];
#pragma unroll
    for (int m = 0; m < MK; ++m) {
        const int idx = threadIdx.x + NT * m, j = idx / DK, i = idx % DK;
        const size_t t = tok + (idx < TB * DK && j < n ? j : 0);
        rk[m] = load_act1<F32>(k, t * DK + i);
        rq[m] = load_act1<F32>(q, t * DK + i);
        rl[m] = as ? la[t] : la[t * DK + i];
        rb[m] = bs ? load_act1<F32>(b, t) : load_act1<F32>(b, t * DK + i);
    }
#pragma unroll
    for (int m = 0; m < MV; ++m) {
        const int idx = threadIdx.x + NT * m, j = idx / DV, c = idx % DV;
        const size_t t = tok + (idx < TB * DV && j < n ? j : 0);
        rv[m] = load_act1<F32>(v, t * DV + c);
        rw[m] = wsc ? load_act1<F32>(w, t) : load_act1<F32>(w, t * DV + c);
        rd[m] = dO ? load_act1<F32>(dO, t * DV + c) : 0.f;
    }
#pragma unroll
    for (int m = 0; m < MK; ++m) {
        const int idx = threadIdx.x + NT * m, j = idx / DK, i = idx % DK;
        if (TB * DK % NT == 0 || idx < TB * DK) {
            float l = rl[m], bb = rb[m];
            if (lg) {
                l = gate_log_sigmoid(l);
                bb = gate_sigmoid(bb);
            }
            sm.q[j][i] = rq[m];
            sm.k[j][i] = rk[m];
            sm.a[j][i] = __expf(l);
            sm.b[j][i] = bb;
            sm.e[j][i] = bb * rk[m];
        }
    }
#pragma unroll
    for (int m = 0; m < MV; ++m) {
        const int idx = threadIdx.x + NT * m, j = idx / DV, c = idx % DV;
        if (TB * DV % NT == 0 || idx < TB * DV) {
            float ww = rw[m];
            if (lg) ww = gate_sigmoid(ww);
            sm.v[j][c] = rv[m];
            sm.w[j][c] = ww;
            sm.x[j][c] = ww * rv[m];
            if (dO) sm.dO[j][c] = rd[m];
        }
    }
}

template <int DK, int DV>
struct Tile {
    static constexpr int TR = DK / 16, TC = DV / 16;
    int tr, tc, lane, wave;
    __device__ __forceinline__ void init() {
        tr = threadIdx.x >> 4;
        tc = threadIdx.x & 15;
        lane = threadIdx.x & 63;
        wave = threadIdx.x >> 6;
    }
    __device__ __forceinline__ int row(int r) const { return tr * TR + r; }
    __device__ __forceinline__ int col(int c) const { return tc * TC + c; }
    // sum over the d_k rows of part (per column of this thread's tile); every
    // thread receives the sums of its tile's columns
    __device__ __forceinline__ void colsum(Stage<DK, DV>& sm, float (&part)[TC], int& rb) const {
#pragma unroll
        for (int c = 0; c < TC; ++c) {
            part[c] += __shfl_xor(part[c], 16);
            part[c] += __shfl_xor(part[c], 32);
        }
        if (lane < 16) {
#pragma unroll
            for (int c = 0; c < TC; ++c) sm.red[rb][wave][col(c)] = part[c];
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < TC; ++c) {
            const int j = col(c);
            part[c] = sm.red[rb][0][j] + sm.red[rb][1][j] + sm.red[rb][2][j] + sm.red[rb][3][j];
        }
        rb ^= 1;
    }
    // sum over the d_v columns (per row of this thread's tile), in every lane
    // of the tile row
    __device__ __forceinline__ void rowsum(float (&part)[TR]) const {
#pragma unroll
        for (int r = 0; r < TR; ++r)
#pragma unroll
            for (int m = 1; m < 16; m *= 2) part[r] += __shfl_xor(part[r], m);
    }
    // sum of one value per thread over the workgroup
    __device__ __forceinline__ float blocksum(Stage<DK, DV>& sm, float x, int& bb) const {
#pragma unroll
        for (int m = 1; m < 64; m *= 2) x += __shfl_xor(x, m);
        if (lane == 0) sm.bred[bb][wave] = x;
        __syncthreads();
        const float s = sm.bred[bb][0] + sm.bred[bb][1] + sm.bred[bb][2] + sm.bred[bb][3];
        bb ^= 1;
        return s;
    }
};

// one token step of the forward on this thread's tile: S <- diag(a) S;
// r = S^T e; u = x - r; S <- S + k u^T (u returned per tile column)
template <int DK, int DV>
__device__ __forceinline__ void step(const Tile<DK, DV>& tl, Stage<DK, DV>& sm, int j,
                                     float (&S)[DK / 16][DV / 16], float (&u)[DV / 16], int& rb) {
    constexpr int TR = DK / 16, TC = DV / 16;
#pragma unroll
    for (int r = 0; r < TR; ++r) {
        const float a = sm.a[j][tl.row(r)];
#pragma unroll
        for (int c = 0; c < TC; ++c) S[r][c] *= a;
    }
    float part[TC];
#pragma unroll
    for (int c = 0; c < TC; ++c) {
        part[c] = 0.f;
#pragma unroll
        for (int r = 0; r < TR; ++r) part[c] += S[r][c] * sm.e[j][tl.row(r)];
    }
    tl.colsum(sm, part, rb);
#pragma unroll
    for (int c = 0; c < TC; ++c) u[c] = sm.x[j][tl.col(c)] - part[c];
#pragma unroll
    for (int r = 0; r < TR; ++r) {
        const float kk = sm.k[j][tl.row(r)];
#pragma unroll
        for (int c = 0; c < TC; ++c) S[r][c] += kk * u[c];
    }
}

template <int DK, int DV>
__device__ __forceinline__ void load_state(const float* src, float (&S)[DK / 16][DV / 16], const Tile<DK, DV>& tl) {
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
        for (int c = 0; c < DV / 16; ++c) S[r][c] = src ? src[(size_t)tl.row(r) * DV + tl.col(c)] : 0.f;
}
template <int DK, int DV>
__device__ __forceinline__ void store_state(float* dst, const float (&S)[DK / 16][DV / 16], const Tile<DK, DV>& tl) {
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
        for (int c = 0; c < DV / 16; ++c) dst[(size_t)tl.row(r) * DV + tl.col(c)] = S[r][c];
}
// a thread's tile as one contiguous run of the workspace (its own scratch)
template <int DK, int DV>
__device__ __forceinline__ void spill(float* dst, const float (&S)[DK / 16][DV / 16]) {
    float* d = dst + (size_t)threadIdx.x * (DK / 16) * (DV / 16);
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
        for (int c = 0; c < DV / 16; ++c) d[r * (DV / 16) + c] = S[r][c];
}
template <int DK, int DV>
__device__ __forceinline__ void fill(const float* src, float (&S)[DK / 16][DV / 16]) {
    const float* s = src + (size_t)threadIdx.x * (DK / 16) * (DV / 16);
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
        for (int c = 0; c < DV / 16; ++c) S[r][c] = s[r * (DV / 16) + c];
}

template <bool F32>
__device__ __forceinline__ float load_out(const void* o, size_t idx, bool bf16) {
    return bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(o)[idx]) : reinterpret_cast<const float*>(o)[idx];
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// One wave per (unit, FC value columns).  The update keeps the state's
// columns apart (S1 = diag(a) S, r = S1^T e, S = S1 + k u^T and o = S^T q are
// per column), so a unit's recompute splits over its value columns with no
// sum across workgroups.  Lane (c, g) = (lane % FC, lane / FC) holds column
// col0 + c over rows g RPL .. g RPL + RPL - 1; a sum over the rows is the
// lane's own sum plus four shuffles across the row groups.  Each workgroup
// checks the marker in its own first column (every column of a marked unit's
// last row is NaN), so no workgroup reads a marker another one has rewritten.
constexpr int FC = 4;                       // value columns per workgroup
constexpr int FTB = 64 / FC;                // tokens per staged block (one x value per lane)

template <int DK, int DV, bool F32>
__global__ __launch_bounds__(64) void exact_fwd_kernel(FwdParams p, long long items) {
    constexpr int RG = 64 / FC, RPL = DK / RG, NG = DV / FC;
    static_assert(DK % RG == 0 && DV % FC == 0, "lane layout");
    __shared__ float sq[FTB][DK], sk[FTB][DK], sa[FTB][DK], se[FTB][DK], sx[FTB][FC];
    const int lane = threadIdx.x, c = lane % FC, g = lane / FC;
    const bool out_bf16 = (p.flags & GDR_OUT_BF16) != 0;
    const bool as = p.flags & GDR_ALPHA_SCALAR, bs = p.flags & GDR_B_SCALAR, wsc = p.flags & GDR_W_SCALAR;
    const bool lg = p.flags & GDR_GATE_LOGITS;
    for (long long item = blockIdx.x; item < items; item += gridDim.x) {
        const int un = (int)(item / NG), grp = (int)(item % NG);
        const int col = grp * FC + c;
        const UnitSpan us = unit_span(p.cu_seqlens, p.BH, p.T, un);
        if (us.len <= 0) continue;
        const float mark = load_out<F32>(p.o, (us.tok0 + us.len - 1) * DV + (size_t)grp * FC, out_bf16);
        if (!__builtin_isnan(mark)) continue;
        float S[RPL];
#pragma unroll
        for (int r = 0; r < RPL; ++r)
            S[r] = p.S0 ? p.S0[((size_t)un * DK + g * RPL + r) * DV + col] : 0.f;
        // Token inputs of a block of TB tokens, loaded into registers one block
        // ahead (all of a block's loads issued together, so one block waits for
        // one load latency at most, behind the previous block's arithmetic).
        // Lanes past the unit's end load its first token (in bounds, unused).
        constexpr int NL = FTB * DK / 64;
        static_assert(FTB * DK % 64 == 0 && FTB * FC == 64, "staging layout");
        float rq[NL], rk[NL], rl[NL], rbv[NL], rw, rv;
        auto load_block = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < NL; ++m) {
                const int idx = lane + 64 * m, j = idx / DK, i = idx % DK;
                const size_t tt = us.tok0 + (t0 + j < us.len ? t0 + j : 0);
                rq[m] = load_act1<F32>(p.q, tt * DK + i);
                rk[m] = load_act1<F32>(p.k, tt * DK + i);
                rl[m] = as ? p.la[tt] : p.la[tt * DK + i];
                rbv[m] = bs ? load_act1<F32>(p.b, tt) : load_act1<F32>(p.b, tt * DK + i);
            }
            const int j = lane / FC, cl = grp * FC + lane % FC;
            const size_t tt = us.tok0 + (t0 + j < us.len ? t0 + j : 0);
            rw = wsc ? load_act1<F32>(p.w, tt) : load_act1<F32>(p.w, tt * DV + cl);
            rv = load_act1<F32>(p.v, tt * DV + cl);
        };
        load_block(0);
        for (int t0 = 0; t0 < us.len; t0 += FTB) {
            const int n = us.len - t0 < FTB ? us.len - t0 : FTB;
            __syncthreads();
            // a = alpha, e = b⊙k; this workgroup's columns of x = w⊙v
#pragma unroll
            for (int m = 0; m < NL; ++m) {
                const int idx = lane + 64 * m, j = idx / DK, i = idx % DK;
                float l = rl[m], bb = rbv[m];
                if (lg) {
                    l = gate_log_sigmoid(l);
                    bb = gate_sigmoid(bb);
                }
                sq[j][i] = rq[m];
                sk[j][i] = rk[m];
                sa[j][i] = __expf(l);
                se[j][i] = bb * rk[m];
            }
            sx[lane / FC][lane % FC] = (lg ? gate_sigmoid(rw) : rw) * rv;
            __syncthreads();
            if (t0 + FTB < us.len) load_block(t0 + FTB);
            for (int j = 0; j < n; ++j) {
                float r = 0.f;
#pragma unroll
                for (int i = 0; i < RPL; ++i) {
                    S[i] *= sa[j][g * RPL + i];
                    r += S[i] * se[j][g * RPL + i];
                }
#pragma unroll
                for (int m = FC; m < 64; m *= 2) r += __shfl_xor(r, m);
                const float u = sx[j][c] - r;
                float o = 0.f;
#pragma unroll
                for (int i = 0; i < RPL; ++i) {
                    S[i] += sk[j][g * RPL + i] * u;
                    o += S[i] * sq[j][g * RPL + i];
                }
#pragma unroll
                for (int m = FC; m < 64; m *= 2) o += __shfl_xor(o, m);
                if (g == 0) {
                    const size_t oi = (us.tok0 + t0 + j) * DV + col;
                    if (out_bf16) reinterpret_cast<uint16_t*>(p.o)[oi] = f32_to_bf16(o);
                    else reinterpret_cast<float*>(p.o)[oi] = o;
                }
            }
        }
        if (p.Sf) {
#pragma unroll
            for (int r = 0; r < RPL; ++r) p.Sf[((size_t)un * DK + g * RPL + r) * DV + col] = S[r];
        }
    }
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32>
__global__ __launch_bounds__(NT) void exact_bwd_kernel(BwdParams p, int units, float* ws, size_t slot_floats,
                                                       int nsegmax) {
    constexpr int TR = DK / 16, TC = DV / 16;
    __shared__ Stage<DK, DV> sm;
    Tile<DK, DV> tl;
    tl.init();
    const bool as = p.flags & GDR_ALPHA_SCALAR, bs = p.flags & GDR_B_SCALAR, wsc = p.flags & GDR_W_SCALAR;
    const bool lg = p.flags & GDR_GATE_LOGITS;
    const int H = p.BH;
    float* ck = ws + (size_t)blockIdx.x * slot_floats;        // [nsegmax] checkpoints
    float* sb = ck + (size_t)nsegmax * DK * DV;                // [SEG] states of one segment
    for (int un = blockIdx.x; un < units; un += gridDim.x) {
        const UnitSpan us = unit_span(p.cu_seqlens, H, p.T, un);
        if (us.len <= 0) continue;
        if (!__builtin_isnan(p.dq[us.tok0 * DK])) continue;
        const int nseg = (us.len + SEG - 1) / SEG;
        float S[TR][TC], u[TC];
        int rb = 0, bb = 0;
        // forward to the checkpoints
        load_state<DK, DV>(p.S0 ? p.S0 + (size_t)un * DK * DV : nullptr, S, tl);
        for (int t0 = 0; t0 < us.len; t0 += TB) {
            const int n = us.len - t0 < TB ? us.len - t0 : TB;
            __syncthreads();
            stage_tokens<DK, DV, F32>(sm, p.q, p.k, p.v, p.la, p.b, p.w, nullptr, us.tok0 + t0, n, p.flags);
            __syncthreads();
            for (int j = 0; j < n; ++j) {
                if ((t0 + j) % SEG == 0) spill<DK, DV>(ck + (size_t)((t0 + j) / SEG) * DK * DV, S);
                step<DK, DV>(tl, sm, j, S, u, rb);
            }
        }
        // reverse
        float dS[TR][TC];
        load_state<DK, DV>(p.dSf ? p.dSf + (size_t)un * DK * DV : nullptr, dS, tl);
        for (int sg = nseg - 1; sg >= 0; --sg) {
            const int ts = sg * SEG, te = (ts + SEG < us.len) ? ts + SEG : us.len;
            // the segment's states S_{t-1}, t = ts .. te - 1
            fill<DK, DV>(ck + (size_t)sg * DK * DV, S);
            for (int t0 = ts; t0 < te; t0 += TB) {
                const int n = te - t0 < TB ? te - t0 : TB;
                __syncthreads();
                stage_tokens<DK, DV, F32>(sm, p.q, p.k, p.v, p.la, p.b, p.w, nullptr, us.tok0 + t0, n, p.flags);
                __syncthreads();
                for (int j = 0; j < n; ++j) {
                    spill<DK, DV>(sb + (size_t)(t0 + j - ts) * DK * DV, S);
                    step<DK, DV>(tl, sm, j, S, u, rb);
                }
            }
            for (int t1 = te; t1 > ts; t1 -= TB) {
                const int t0 = (t1 - TB > ts) ? t1 - TB : ts, n = t1 - t0;
                __syncthreads();
                stage_tokens<DK, DV, F32>(sm, p.q, p.k, p.v, p.la, p.b, p.w, p.dO, us.tok0 + t0, n, p.flags);
                __syncthreads();
                for (int j = n - 1; j >= 0; --j) {
                    const size_t tok = us.tok0 + t0 + j;
                    float Sp[TR][TC], S1[TR][TC];
                    fill<DK, DV>(sb + (size_t)(t0 + j - ts) * DK * DV, Sp);
                    // recompute: S1 = diag(a) S_{t-1}, r = S1^T e, u = x - r
#pragma unroll
                    for (int r = 0; r < TR; ++r) {
                        const float a = sm.a[j][tl.row(r)];
#pragma unroll
                        for (int c = 0; c < TC; ++c) S1[r][c] = a * Sp[r][c];
                    }
                    float part[TC];
#pragma unroll
                    for (int c = 0; c < TC; ++c) {
                        part[c] = 0.f;
#pragma unroll
                        for (int r = 0; r < TR; ++r) part[c] += S1[r][c] * sm.e[j][tl.row(r)];
                    }
                    tl.colsum(sm, part, rb);
                    float dOc[TC];
#pragma unroll
                    for (int c = 0; c < TC; ++c) {
                        u[c] = sm.x[j][tl.col(c)] - part[c];
                        dOc[c] = sm.dO[j][tl.col(c)];
                    }
                    // o = S_t^T q with S_t = S1 + k u^T:  dS += q dO^T,
                    // dq = S1 dO + k (u . dO)
                    float prt[TR];
                    float udo = 0.f;
#pragma unroll
                    for (int c = 0; c < TC; ++c) udo += u[c] * dOc[c];
                    {
                        float tmp[1] = {udo};
                        // sum over the tile row's 16 lanes = over all d_v columns
#pragma unroll
                        for (int m = 1; m < 16; m *= 2) tmp[0] += __shfl_xor(tmp[0], m);
                        udo = tmp[0];
                    }
#pragma unroll
                    for (int r = 0; r < TR; ++r) {
                        const float qq = sm.q[j][tl.row(r)];
                        prt[r] = 0.f;
#pragma unroll
                        for (int c = 0; c < TC; ++c) {
                            prt[r] += S1[r][c] * dOc[c];
                            dS[r][c] += qq * dOc[c];
                        }
                    }
                    tl.rowsum(prt);
                    float dqv[TR];
#pragma unroll
                    for (int r = 0; r < TR; ++r) dqv[r] = prt[r] + sm.k[j][tl.row(r)] * udo;
                    // S_t = S1 + k u^T:  dk (this term) = dS u,  du = dS^T k
                    float dka[TR];
#pragma unroll
                    for (int r = 0; r < TR; ++r) {
                        dka[r] = 0.f;
#pragma unroll
                        for (int c = 0; c < TC; ++c) dka[r] += dS[r][c] * u[c];
                    }
                    tl.rowsum(dka);
                    float du[TC];
#pragma unroll
                    for (int c = 0; c < TC; ++c) {
                        du[c] = 0.f;
#pragma unroll
                        for (int r = 0; r < TR; ++r) du[c] += dS[r][c] * sm.k[j][tl.row(r)];
                    }
                    tl.colsum(sm, du, rb);
                    // u = w⊙v - r:  dr = -du;  S1 gets e dr^T;  de = S1 dr
#pragma unroll
                    for (int r = 0; r < TR; ++r) {
                        const float ee = sm.e[j][tl.row(r)];
#pragma unroll
                        for (int c = 0; c < TC; ++c) dS[r][c] -= ee * du[c];
                    }
                    float de[TR];
#pragma unroll
                    for (int r = 0; r < TR; ++r) {
                        de[r] = 0.f;
#pragma unroll
                        for (int c = 0; c < TC; ++c) de[r] -= S1[r][c] * du[c];
                    }
                    tl.rowsum(de);
                    // S1 = diag(a) S_{t-1}:  da = rowsum(dS1 ⊙ S_{t-1}),  dS_{t-1} = diag(a) dS1
                    float da[TR];
#pragma unroll
                    for (int r = 0; r < TR; ++r) {
                        da[r] = 0.f;
#pragma unroll
                        for (int c = 0; c < TC; ++c) da[r] += dS[r][c] * Sp[r][c];
                    }
                    tl.rowsum(da);
#pragma unroll
                    for (int r = 0; r < TR; ++r) {
                        const float a = sm.a[j][tl.row(r)];
#pragma unroll
                        for (int c = 0; c < TC; ++c) dS[r][c] *= a;
                    }
                    // per-row results: dq, dk = dka + de⊙b, db = de⊙k, dlog_alpha = da⊙a
                    float sdla = 0.f, sdb = 0.f;
#pragma unroll
                    for (int r = 0; r < TR; ++r) {
                        const int i = tl.row(r);
                        const float a = sm.a[j][i], bb = sm.b[j][i], kk = sm.k[j][i];
                        const float dla = da[r] * a, dbv = de[r] * kk;
                        if (tl.tc == 0) {
                            p.dq[tok * DK + i] = dqv[r];
                            p.dk[tok * DK + i] = dka[r] + de[r] * bb;
                            if (!as) p.dla[tok * DK + i] = lg ? dla * (1.f - a) : dla;
                            if (!bs) p.db[tok * DK + i] = lg ? dbv * bb * (1.f - bb) : dbv;
                            sdla += dla;
                            sdb += dbv;
                        }
                    }
                    // per-column results: dv = du⊙w, dw = du⊙v
                    float sdw = 0.f;
#pragma unroll
                    for (int c = 0; c < TC; ++c) {
                        const int col = tl.col(c);
                        const float ww = sm.w[j][col], vv = sm.v[j][col];
                        if (tl.tr == 0) {
                            p.dv[tok * DV + col] = du[c] * ww;
                            if (!wsc) p.dw[tok * DV + col] = lg ? du[c] * vv * ww * (1.f - ww) : du[c] * vv;
                            sdw += du[c] * vv;
                        }
                    }
                    // scalar gates: the sums over the channels (block-uniform branches)
                    if (as) {
                        const float s = tl.blocksum(sm, sdla, bb);
                        const float a = sm.a[j][0];
                        if (threadIdx.x == 0) p.dla[tok] = lg ? s * (1.f - a) : s;
                    }
                    if (bs) {
                        const float s = tl.blocksum(sm, sdb, bb);
                        const float b0 = sm.b[j][0];
                        if (threadIdx.x == 0) p.db[tok] = lg ? s * b0 * (1.f - b0) : s;
                    }
                    if (wsc) {
                        const float s = tl.blocksum(sm, sdw, bb);
                        const float w0 = sm.w[j][0];
                        if (threadIdx.x == 0) p.dw[tok] = lg ? s * w0 * (1.f - w0) : s;
                    }
                }
            }
        }
        if (p.dS0) store_state<DK, DV>(p.dS0 + (size_t)un * DK * DV, dS, tl);
        __syncthreads();
    }
}

template <int DK, int DV>
static hipError_t fwd_t(const FwdParams& p, int units, hipStream_t st) {
    const long long items = (long long)units * (DV / FC);
    const unsigned grid = (unsigned)(items < 8192 ? items : 8192);
    if (p.flags & GDR_ACT_F32) hipLaunchKernelGGL((exact_fwd_kernel<DK, DV, true>), dim3(grid), dim3(64), 0, st, p, items);
    else hipLaunchKernelGGL((exact_fwd_kernel<DK, DV, false>), dim3(grid), dim3(64), 0, st, p, items);
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t bwd_t(const BwdParams& p, int units, void* ws, size_t ws_bytes, int T, hipStream_t st) {
    const int nsegmax = (T + SEG - 1) / SEG;
    const size_t slot_floats = (size_t)(nsegmax + SEG) * DK * DV;
    size_t slots = ws_bytes / (slot_floats * 4);
    if (slots < 1) return hipSuccess;   // no room: the NaN results stay
    if (slots > (size_t)units) slots = (size_t)units;
    if (slots > 2048) slots = 2048;
    float* w = reinterpret_cast<float*>(ws);
    if (p.flags & GDR_ACT_F32)
        hipLaunchKernelGGL((exact_bwd_kernel<DK, DV, true>), dim3((unsigned)slots), dim3(NT), 0, st, p, units, w,
                           slot_floats, nsegmax);
    else
        hipLaunchKernelGGL((exact_bwd_kernel<DK, DV, false>), dim3((unsigned)slots), dim3(NT), 0, st, p, units, w,
                           slot_floats, nsegmax);
    return hipGetLastError();
}

}  // namespace ex

size_t exact_bwd_slot_bytes(int T, int dk, int dv) {
    const size_t nseg = ((size_t)(T > 0 ? T : 0) + ex::SEG - 1) / ex::SEG;
    return (nseg + ex::SEG) * (size_t)dk * dv * 4;
}

// (d_k, d_v) in {16, 32, 64, 128}^2 to the template instance
#define GDR_EX_CASES(CALL)                                                                        \
    switch (dk * 1000 + dv) {                                                                     \
        case 16016: return CALL(16, 16);   case 16032: return CALL(16, 32);                      \
        case 16064: return CALL(16, 64);   case 16128: return CALL(16, 128);                     \
        case 32016: return CALL(32, 16);   case 32032: return CALL(32, 32);                      \
        case 32064: return CALL(32, 64);   case 32128: return CALL(32, 128);                     \
        case 64016: return CALL(64, 16);   case 64032: return CALL(64, 32);                      \
        case 64064: return CALL(64, 64);   case 64128: return CALL(64, 128);                     \
        case 128016: return CALL(128, 16); case 128032: return CALL(128, 32);                    \
        case 128064: return CALL(128, 64); case 128128: return CALL(128, 128);                   \
    }                                                                                             \
    return hipErrorInvalidValue;

hipError_t launch_exact_fwd(const FwdParams& p, int dk, int dv, hipStream_t st) {
    const long long units = p.cu_seqlens ? (long long)p.nseq * p.BH : (long long)p.BH;
    if (units <= 0 || p.T <= 0 || !p.o) return hipSuccess;
    const int u = (int)units;
#define GDR_EX_FWD(DK, DV) ex::fwd_t<DK, DV>(p, u, st)
    GDR_EX_CASES(GDR_EX_FWD)
#undef GDR_EX_FWD
}

hipError_t launch_exact_bwd(const BwdParams& p, int dk, int dv, void* ws, size_t ws_bytes, hipStream_t st) {
    const long long units = p.cu_seqlens ? (long long)p.nseq * p.BH : (long long)p.BH;
    if (units <= 0 || p.T <= 0 || !ws) return hipSuccess;
    const int u = (int)units;
#define GDR_EX_BWD(DK, DV) ex::bwd_t<DK, DV>(p, u, ws, ws_bytes, p.T, st)
    GDR_EX_CASES(GDR_EX_BWD)
#undef GDR_EX_BWD
}
#undef GDR_EX_CASES

}  // namespace gdr
