// Recurrent decode step of the gated delta rule: one token per (sequence,
// head), state updated in place (constant memory per sequence: Gated
// DeltaNet-2 Q&A page, introduction; "Gated DeltaNet-2 Review" §3-2 item 1).
//
// Per (n, h), with a = exp(log_alpha), e = b ⊙ k, x = w ⊙ v:
//   S_hat = diag(a) S            (decay along the key axis)
//   r     = S_hat^T e            (erase read of the decayed state)
//   p     = S_hat^T q
//   delta = x - r
//   S    <- S_hat + k delta^T    (erase and write, Q&A page Q3 update)
//   o     = S^T q = p + (q·k) delta   (read-out after the write)
//
// The kernel is HBM-bound: the fp32 state (64 KiB per head at d=128) is
// streamed exactly once in and once out.  One workgroup owns one head; each
// thread keeps a (rows x 4 columns) slice of the state in registers between
// the read and the write, so the only on-chip traffic is the two column
// reductions (r, p) across row groups through LDS.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

template <int DK, int DV, bool F32, bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
    constexpr int NT = 256;
    constexpr int CQ = DV / 4;                      // column quads
    constexpr int RG0 = NT / CQ;                    // row groups if all threads work
    constexpr int RG = RG0 < DK ? RG0 : DK;         // row groups
    constexpr int RPT = DK / RG;                    // rows per thread
    static_assert(RG * RPT == DK, "row split");

    __shared__ float s_q[DK], s_k[DK], s_e[DK], s_a[DK];
    __shared__ float s_x[DV], s_dl[DV];
    __shared__ float s_r[RG][DV], s_p[RG][DV];
    __shared__ float s_qk;

    const int tid = threadIdx.x;
    const size_t nh = blockIdx.x;
    const int cq = tid % CQ, rg = tid / CQ;
    const bool active = rg < RG;
    float* S = p.S + nh * (size_t)DK * DV;

    // 1. stream this thread's slice of the state in first (longest latency)
    floatx4 s[RPT];
    if (active) {
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            s[i] = *reinterpret_cast<const floatx4*>(S + (size_t)(rg * RPT + i) * DV + 4 * cq);
    }

    // 2. token vectors into LDS
    // (gates given as logits: alpha = sigmoid(logit), b and w through sigmoid)
    const bool lg = (p.flags & GDR_GATE_LOGITS) != 0;
    for (int c = tid; c < DK; c += NT) {
        float qv = load_act1<F32>(p.q, nh * DK + c);
        float kv = load_act1<F32>(p.k, nh * DK + c);
        float la = (p.flags & GDR_ALPHA_SCALAR) ? p.la[nh] : p.la[nh * DK + c];
        float bv = (p.flags & GDR_B_SCALAR) ? load_act1<F32>(p.b, nh) : load_act1<F32>(p.b, nh * DK + c);
        if (lg) bv = gate_sigmoid(bv);
        s_q[c] = qv;
        s_k[c] = kv;
        s_e[c] = bv * kv;
        s_a[c] = lg ? gate_sigmoid(la) : __expf(la);
    }
    for (int j = tid; j < DV; j += NT) {
        float vv = load_act1<F32>(p.v, nh * DV + j);
        float wv = (p.flags & GDR_W_SCALAR) ? load_act1<F32>(p.w, nh) : load_act1<F32>(p.w, nh * DV + j);
        if (lg) wv = gate_sigmoid(wv);
        s_x[j] = wv * vv;
    }
    __syncthreads();

    // q·k by wave 0
    if (tid < 64) {
        float acc = 0.f;
        for (int c = tid; c < DK; c += 64) acc += s_q[c] * s_k[c];
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if (tid == 0) s_qk = acc;
    }

    // 3. decay, partial column reductions
    if (active) {
        floatx4 pr = zero4(), pp = zero4();
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg * RPT + i;
            const float a = s_a[row], e = s_e[row], qv = s_q[row];
            s[i] = s[i] * a;
            pr += s[i] * e;
            pp += s[i] * qv;
        }
        *reinterpret_cast<floatx4*>(&s_r[rg][4 * cq]) = pr;
        *reinterpret_cast<floatx4*>(&s_p[rg][4 * cq]) = pp;
    }
    __syncthreads();

    // 4. finish the reductions: delta and o
    for (int j = tid; j < DV; j += NT) {
        float r = 0.f, pv = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            r += s_r[g][j];
            pv += s_p[g][j];
        }
        const float dl = s_x[j] - r;
        s_dl[j] = dl;
        const float ov = pv + s_qk * dl;
        if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(p.o)[nh * DV + j] = f32_to_bf16(ov);
        else reinterpret_cast<float*>(p.o)[nh * DV + j] = ov;
    }
    __syncthreads();

    // 5. rank-one write and store back in place.  Non-temporal stores: the
    // state is not read again in this step, and streaming it past the caches
    // (instead of write-allocating in L2) takes the step from about 5.1 to
    // about 6.8 TB/s on the 256 x 32 workload.
    if (active) {
        const floatx4 dl = *reinterpret_cast<const floatx4*>(&s_dl[4 * cq]);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg * RPT + i;
            floatx4 v = s[i] + dl * s_k[row];
            __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(S + (size_t)row * DV + 4 * cq));
        }
    }
}

template <int DK, int DV>
static hipError_t launch_decode_dv(const DecodeParams& p, bool f32, bool obf16, hipStream_t st) {
    dim3 grid((unsigned)p.NH), block(256);
    if (f32) {
        if (obf16) hipLaunchKernelGGL((decode_kernel<DK, DV, true, true>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((decode_kernel<DK, DV, true, false>), grid, block, 0, st, p);
    } else {
        if (obf16) hipLaunchKernelGGL((decode_kernel<DK, DV, false, true>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((decode_kernel<DK, DV, false, false>), grid, block, 0, st, p);
    }
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_decode_dk(const DecodeParams& p, int dv, bool f32, bool obf16, hipStream_t st) {
    switch (dv) {
        case 16: return launch_decode_dv<DK, 16>(p, f32, obf16, st);
        case 32: return launch_decode_dv<DK, 32>(p, f32, obf16, st);
        case 64: return launch_decode_dv<DK, 64>(p, f32, obf16, st);
        case 128: return launch_decode_dv<DK, 128>(p, f32, obf16, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, int dk, int dv, hipStream_t st) {
    const bool f32 = (p.flags & GDR_ACT_F32) != 0;
    const bool obf16 = (p.flags & GDR_OUT_BF16) != 0;
    switch (dk) {
        case 16: return launch_decode_dk<16>(p, dv, f32, obf16, st);
        case 32: return launch_decode_dk<32>(p, dv, f32, obf16, st);
        case 64: return launch_decode_dk<64>(p, dv, f32, obf16, st);
        case 128: return launch_decode_dk<128>(p, dv, f32, obf16, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
