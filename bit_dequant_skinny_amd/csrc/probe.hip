// Measurement aids: a 128-bit streaming copy and a 128-bit streaming read.
//
// The copy gives the achievable HBM copy rate with the same load width as the
// GEMM kernels, and a transfer of known size against which hardware byte
// counters are scaled.  The read gives the achievable HBM read rate of one
// launch over a buffer of a given size: the ceiling for the weight-streaming
// kernels, which read their bytes once and write almost nothing (the
// bitsandbytes pull request "[ROCm] Optimize kgemm_4bit_inference_naive for
// ROCm, use it for batch sizes other than 1" quotes its kernel's rate against
// a measured peak in the same way, table "kgemm_4bit_inference_naive
// benchmark").
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

constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

// Read-only stream.  Workgroup b reads its share of the buffer in batches of
// THREADS * U 16-byte pieces (lane t of the workgroup takes pieces t,
// t + THREADS, ...), the next batch issued before the current one is
// consumed, so about 2 * U loads per lane stay in flight.  Contiguous shares
// (interleave = 0): workgroup b reads bytes [b * share, (b + 1) * share).
// Interleaved (interleave = 1): batch i of workgroup b is batch i * G + b of
// the buffer.  Buffer loads return zeros past `bytes`, so the tail needs no
// branch.  The loaded words are folded into one value that is stored only if
// it equals `magic`, which keeps every load live while writing (almost)
// nothing.  NT selects the non-temporal cache policy, as on the weight loads
// of the fused kernels.
template <int THREADS, int U, int NT>
__global__ __launch_bounds__(THREADS) void read_kernel(const void *__restrict__ src,
                                                       uint32_t bytes, uint32_t share,
                                                       int interleave, uint32_t *sink,
                                                       uint32_t magic) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(src), (short)0, (int)bytes, kBufferFlags);
    constexpr uint32_t kBatch = (uint32_t)THREADS * U * 16;
    const uint32_t G = gridDim.x;
    const uint32_t lane_off = threadIdx.x * 16u;
    uint32_t first, stride, nbatch;
    if (interleave) {
        first = blockIdx.x * kBatch;
        stride = G * kBatch;
        const uint32_t total = (bytes + kBatch - 1) / kBatch;
        nbatch = total > blockIdx.x ? (total - blockIdx.x + G - 1) / G : 0;
    } else {
        first = blockIdx.x * share;
        stride = kBatch;
        const uint32_t end = first + share < bytes ? first + share : bytes;
        nbatch = end > first ? (end - first + kBatch - 1) / kBatch : 0;
    }
    uint32_t acc = 0;
    auto load = [&](uint4 (&v)[U], uint32_t base) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           rs, (int)(base + (uint32_t)u * THREADS * 16u + lane_off), 0, NT ? 2 : 0));
    };
    auto fold = [&](const uint4 (&v)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    };
    if (nbatch > 0) {
        uint4 cur[U], nxt[U];
        load(cur, first);
        for (uint32_t i = 1; i < nbatch; ++i) {
            load(nxt, first + i * stride);
            fold(cur);
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
        fold(cur);
    }
    if (acc == magic) sink[0] = acc;
}

template <int THREADS, int U>
hipError_t launch_read_t(const void *src, uint32_t bytes, uint32_t share, int interleave,
                         uint32_t *sink, int nt, unsigned grid, hipStream_t s) {
    const uint32_t magic = 0x9e3779b9u;
    if (nt)
        read_kernel<THREADS, U, 1><<<dim3(grid), dim3(THREADS), 0, s>>>(src, bytes, share,
                                                                        interleave, sink, magic);
    else
        read_kernel<THREADS, U, 0><<<dim3(grid), dim3(THREADS), 0, s>>>(src, bytes, share,
                                                                        interleave, sink, magic);
    return hipGetLastError();
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

bool read_probe_shape_ok(int threads, int unroll) {
    return (threads == 256 || threads == 512 || threads == 1024) &&
           (unroll == 2 || unroll == 4 || unroll == 8);
}

hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, int threads,
                             int unroll, int wgs_per_cu, int nt, int interleave, hipStream_t s) {
    if (!read_probe_shape_ok(threads, unroll) || wgs_per_cu < 1 || bytes >= (1ull << 32))
        return hipErrorInvalidValue;
    const unsigned grid = (unsigned)(device_info().num_cus * wgs_per_cu);
    const uint32_t batch = (uint32_t)threads * (uint32_t)unroll * 16u;
    // equal shares in whole batches
    const uint64_t per = ((uint64_t)bytes + grid - 1) / grid;
    const uint32_t share = (uint32_t)((per + batch - 1) / batch * batch);
    const uint32_t b32 = (uint32_t)bytes;
#define Q4_READ(T, U) \
    if (threads == T && unroll == U) return launch_read_t<T, U>(src, b32, share, interleave, sink, nt, grid, s)
    Q4_READ(256, 2); Q4_READ(256, 4); Q4_READ(256, 8);
    Q4_READ(512, 2); Q4_READ(512, 4); Q4_READ(512, 8);
    Q4_READ(1024, 2); Q4_READ(1024, 4); Q4_READ(1024, 8);
#undef Q4_READ
    return hipErrorInvalidValue;
}

}  // namespace q4
