// gdr_chunk_fwd_noalloc: the chunkwise forward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The two-pass forward's workspace is a
// file-scope device array of GDR_NOALLOC_SCRATCH_BYTES per GPU, held from the
// library's load until the process ends; nothing is allocated per call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdr_launch.h"

namespace {

constexpr size_t kScratchBytes = GDR_NOALLOC_SCRATCH_BYTES;

// The array's name is a host-side stand-in: host code uses only the device
// address that hipGetSymbolAddress returns for the current device.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device

// The current device's copy of the array, looked up once per device.
gdr_status scratch_on_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDR_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return GDR_ERR_DEVICE;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GDR_OK;
}

}  // namespace

extern "C" gdr_status gdr_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                            const float* log_alpha, const void* b, const void* w,
                                            const float* S0, void* o, float* S_final, int B, int H,
                                            int T, int d_k, int d_v, int chunk, uint32_t flags,
                                            void* stream) {
    // the size check first: it needs no device
    const size_t need = gdr_chunk_fwd_workspace_bytes(B, H, T, d_k, d_v, chunk, flags);
    if (need > kScratchBytes) return GDR_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const gdr_status s = scratch_on_device(&ws);
        if (s != GDR_OK) return s;
    }
    return gdr_chunk_fwd(q, k, v, log_alpha, b, w, S0, o, S_final, B, H, T, d_k, d_v, chunk, flags,
                         ws, ws ? kScratchBytes : 0, stream);
}
