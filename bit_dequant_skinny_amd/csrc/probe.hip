// Plain 128-bit streaming copy.  A measurement aid: it gives the achievable
// HBM rate with the same load width as the GEMM kernels, and a transfer of
// known size against which hardware byte counters are scaled.
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4 *__restrict__ src,
                                                        uint4 *__restrict__ dst, uint64_t n) {
    const uint64_t stride = (uint64_t)gridDim.x * kThreads * kUnroll;
    for (uint64_t base = (uint64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n;
         base += stride) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t i = base + (uint64_t)u * kThreads;
            if (i < n) v[u] = src[i];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t i = base + (uint64_t)u * kThreads;
            if (i < n) dst[i] = v[u];
        }
    }
}

}  // namespace

hipError_t launch_copy_probe(const void *src, void *dst, size_t bytes, hipStream_t s) {
    const uint64_t n = bytes / 16;
    const DeviceInfo info = device_info();
    uint64_t blocks = (n + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    const uint64_t cap = (uint64_t)info.num_cus * 16;
    if (blocks > cap) blocks = cap;
    if (blocks == 0) blocks = 1;
    copy_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
        reinterpret_cast<const uint4 *>(src), reinterpret_cast<uint4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace q4
