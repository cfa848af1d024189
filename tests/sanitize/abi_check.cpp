// Argument-validation sweep of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (the test that builds it compiles the ABI layer,
// gdr_api.cpp, into this program with the same flags).  No device memory is
// touched: every pointer is a fake, aligned or misaligned, address.  A call
// that passes validation reaches the device check and must return
// GDR_ERR_DEVICE, so the program refuses to run where a device is visible.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "gdr.h"

namespace {

uint64_t state = 0x243F6A8885A308D3ull;
uint64_t next() {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return state >> 17;
}
template <typename T, size_t N>
T pick(const T (&a)[N]) { return a[next() % N]; }

const int kInts[] = {INT_MIN, -1, 0, 1, 2, 3, 7, 16, 32, 48, 63, 64, 65, 128, 129, 4096, 1 << 20, 1 << 28,
                     (1 << 28) + 1, INT_MAX};
const int kHeads[] = {-1, 0, 8, 16, 24, 32, 64, 96, 128, 129, 256, INT_MAX};
const int kChunks[] = {-1, 0, 8, 16, 32, 48, 64, 128};
const uint32_t kFlags[] = {0u, 1u, 2u, 3u, 4u, 8u, 0x10u, 0x1cu, 0x20u, 0x40u, 0x41u, 0x80u, 0x100u,
                           0x80000000u, 0xffffffffu};
void* const kPtrs[] = {nullptr, reinterpret_cast<void*>(0x10000), reinterpret_cast<void*>(0x10004)};

int failures = 0;
long calls = 0;

void expect(const char* fn, gdr_status st) {
    ++calls;
    // no device is visible: nothing may report success
    if (st == GDR_OK || (int)st < 0 || (int)st > GDR_ERR_DEVICE) {
        std::fprintf(stderr, "%s returned %d\n", fn, (int)st);
        ++failures;
    }
    if (gdr_status_string(st) == nullptr) ++failures;
}

void* P() { return pick(kPtrs); }
float* F() { return static_cast<float*>(pick(kPtrs)); }

}  // namespace

int main() {
    int n = 0;
    if (hipGetDeviceCount(&n) == hipSuccess && n > 0) {
        std::printf("skipped: a device is visible\n");
        return 0;
    }
    if (gdr_abi_version() != GDR_ABI_VERSION) ++failures;
    for (int s = -3; s < 12; ++s)
        if (gdr_status_string(static_cast<gdr_status>(s)) == nullptr) ++failures;
    for (int it = 0; it < 20000; ++it) {
        const int B = pick(kInts), H = pick(kInts), T = pick(kInts), dk = pick(kHeads), dv = pick(kHeads);
        const int chunk = pick(kChunks);
        const uint32_t fl = pick(kFlags);
        (void)gdr_chunk_fwd_workspace_bytes(B, H, T, dk, dv, chunk, fl);
        (void)gdr_chunk_bwd_workspace_bytes(B, H, T, dk, dv, chunk, fl);
        (void)gdr_chunk_fwd_varlen_workspace_bytes(B, H, T, dk, dv, fl);
        (void)gdr_chunk_bwd_varlen_workspace_bytes(B, H, T, dk, dv, fl);
        (void)gdr_mixer_bwd_workspace_bytes(B, H, T, dk, dv);
        const size_t wsb = (next() & 1) ? (size_t)next() : SIZE_MAX;
        switch (it % 9) {
            case 0:
                expect("gdr_chunk_fwd", gdr_chunk_fwd(P(), P(), P(), F(), P(), P(), F(), P(), F(), B, H, T, dk, dv,
                                                      chunk, fl, P(), wsb, nullptr));
                break;
            case 1:
                expect("gdr_chunk_fwd_noalloc", gdr_chunk_fwd_noalloc(P(), P(), P(), F(), P(), P(), F(), P(), F(), B, H,
                                                                      T, dk, dv, chunk, fl, nullptr));
                break;
            case 2:
                expect("gdr_chunk_fwd_varlen",
                       gdr_chunk_fwd_varlen(P(), P(), P(), F(), P(), P(), F(), P(), F(),
                                            static_cast<const int*>(P()), B, H, T, dk, dv, fl, P(), wsb, nullptr));
                break;
            case 3:
                expect("gdr_decode_step", gdr_decode_step(P(), P(), P(), F(), P(), P(), F(), P(), B, H, dk, dv, fl,
                                                          nullptr));
                break;
            case 4:
                expect("gdr_chunk_bwd", gdr_chunk_bwd(P(), P(), P(), F(), P(), P(), F(), P(), F(), F(), F(), F(), F(),
                                                      F(), F(), F(), B, H, T, dk, dv, chunk, fl, P(), wsb, nullptr));
                break;
            case 5:
                expect("gdr_chunk_bwd_varlen",
                       gdr_chunk_bwd_varlen(P(), P(), P(), F(), P(), P(), F(), P(), F(), F(), F(), F(), F(), F(), F(),
                                            F(), static_cast<const int*>(P()), B, H, T, dk, dv, fl, P(), wsb,
                                            nullptr));
                break;
            case 6:
                expect("gdr_mixer_prologue",
                       gdr_mixer_prologue(P(), P(), P(), F(), F(), F(), F(), P(), P(), P(), P(), P(), F(), P(), P(),
                                          B, H, T, dk, dv, fl, nullptr));
                break;
            case 7:
                expect("gdr_mixer_epilogue", gdr_mixer_epilogue(F(), P(), F(), P(), B, H, T, dv, fl, nullptr));
                expect("gdr_mixer_epilogue_bwd", gdr_mixer_epilogue_bwd(F(), P(), F(), F(), F(), F(), F(), B, H, T,
                                                                        dv, fl, P(), wsb, nullptr));
                break;
            default:
                expect("gdr_mixer_prologue_bwd",
                       gdr_mixer_prologue_bwd(P(), P(), P(), F(), F(), F(), F(), F(), F(), F(), F(), F(), F(), F(),
                                              F(), B, H, T, dk, dv, fl, P(), wsb, nullptr));
                break;
        }
    }
    std::printf("%s: %ld calls, %d failures\n", failures ? "FAILED" : "ok", calls, failures);
    return failures ? 1 : 0;
}
