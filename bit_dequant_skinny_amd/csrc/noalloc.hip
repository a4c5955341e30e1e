// The allocation-free entry point: q4_gemm_skinny_ex with its scratch in a
// fixed device array instead of the library's per-stream workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops and harnesses that forbid allocation).
//
// `scratch` is a file-scope device array of Q4_NOALLOC_SCRATCH_BYTES: each
// device the library runs on holds its own copy until the process ends.  In
// host code its name is not a device address, so its address on a device is
// looked up once per device (with that device current) and only that
// address reaches the kernels.  Every call on a device shares the array:
// calls that overlap on one device (different streams, or threads) race.
// The kernels write every scratch byte they read within a call (activation
// planes, fp32 partial outputs, dequantized weights), so nothing needs
// clearing between calls.
#include <mutex>

#include "launch.h"

namespace {

__device__ __align__(256) unsigned char scratch[Q4_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[256];  // per device; nullptr until looked up

q4_status scratch_for_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return q4::report(Q4_ERR_HIP, "hipGetDevice", e);
    if (dev < 0 || dev >= 256) return q4::report(Q4_ERR_UNSUPPORTED, "device index", hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return q4::report(Q4_ERR_HIP, "hipGetSymbolAddress(scratch)",
                              e != hipSuccess ? e : hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return Q4_OK;
}

}  // namespace

extern "C" q4_status q4_gemm_skinny_ex_noalloc(const void *A, int a_dtype, const uint8_t *Wpacked,
                                               const float *absmax, const float *codebook,
                                               const void *bias, int M, int N, int K,
                                               int blocksize, void *C, int c_dtype, void *stream,
                                               int path) {
    void *p = nullptr;
    const q4_status st = scratch_for_device(&p);
    if (st != Q4_OK) return st;
    return q4::gemm_ex_fixed_scratch(A, a_dtype, Wpacked, absmax, codebook, bias, M, N, K,
                                     blocksize, C, c_dtype, stream, path, p,
                                     Q4_NOALLOC_SCRATCH_BYTES);
}
