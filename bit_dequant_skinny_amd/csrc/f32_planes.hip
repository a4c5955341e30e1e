// fp32 activations on the matrix cores, for the fused 4-bit path.
//
// The fused GEMM of the bitsandbytes pull request "[ROCm] Optimize
// kgemm_4bit_inference_naive for ROCm, use it for batch sizes other than 1"
// takes fp32 activations as well (maintainer's comment: fp32/fp16/bf16
// variants, all accumulating in fp32).  Here an fp32 row is written as the sum
// of three bf16 rows taken by truncation: hi = a with its low 16 bits
// cleared, mid = (a - hi) likewise, lo = a - hi - mid.  Each subtraction is
// exact in fp32 and lo keeps at most 8 significant bits, so hi + mid + lo
// equals a for |a| >= 2^-110; below that the part under 2^-133 is dropped.
// Truncation cannot round a value near the fp32 maximum up to infinity.
//
// The three planes form 3M bf16 rows, [hi rows | mid rows | lo rows], which
// the bf16 matrix-core kernel multiplies into fp32 partials without a bias;
// the sum kernel then adds, for each output, (hi + mid) + lo and the bias in
// fp32 and rounds once to the output type.  Both kernels are elementwise and
// HBM-bound: 4 B read and 6 B written per activation, 12 B read and 2 to 4 B
// written per output.
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void split_planes_kernel(const float *__restrict__ A,
                                                                 size_t n,
                                                                 uint16_t *__restrict__ planes) {
    for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < n;
         i += (size_t)gridDim.x * kThreads) {
        const uint32_t a = __float_as_uint(A[i]);
        const uint32_t hi = a & 0xffff0000u;
        const float r1 = __uint_as_float(a) - __uint_as_float(hi);
        const uint32_t mid = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(mid);
        planes[i] = (uint16_t)(hi >> 16);
        planes[n + i] = (uint16_t)(mid >> 16);
        planes[2 * n + i] = (uint16_t)(__float_as_uint(r2) >> 16);
    }
}

__global__ __launch_bounds__(kThreads) void sum_planes_kernel(const float *__restrict__ P,
                                                               size_t mn, int N,
                                                               const void *__restrict__ bias,
                                                               void *__restrict__ C, int c_dt) {
    for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < mn;
         i += (size_t)gridDim.x * kThreads) {
        float v = (P[i] + P[mn + i]) + P[2 * mn + i];
        if (bias) v += load_elem(bias, i % (size_t)N, c_dt);  // before the single rounding
        store_elem(C, i, v, c_dt);
    }
}

int grid_for(size_t n) {
    const size_t blocks = (n + kThreads - 1) / kThreads;
    const size_t cap = (size_t)device_info().num_cus * 16;
    return (int)(blocks < cap ? (blocks ? blocks : 1) : cap);
}

}  // namespace

hipError_t launch_split_planes(const float *A, size_t n, uint16_t *planes, hipStream_t s) {
    if (n == 0) return hipSuccess;
    split_planes_kernel<<<grid_for(n), kThreads, 0, s>>>(A, n, planes);
    return hipGetLastError();
}

hipError_t launch_sum_planes(const float *P, int M, int N, const void *bias, void *C, int c_dt,
                             hipStream_t s) {
    const size_t mn = (size_t)M * (size_t)N;
    if (mn == 0) return hipSuccess;
    sum_planes_kernel<<<grid_for(mn), kThreads, 0, s>>>(P, mn, N, bias, C, c_dt);
    return hipGetLastError();
}

}  // namespace q4
