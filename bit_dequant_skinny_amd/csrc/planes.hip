// fp16 and fp32 activations on the matrix cores, for the fused 4-bit path.
//
// The fused GEMM of the bitsandbytes pull request "[ROCm] Optimize
// kgemm_4bit_inference_naive for ROCm, use it for batch sizes other than 1"
// takes fp16 and fp32 activations as well (maintainer's comment: fp32/fp16/
// bf16 variants, all accumulating in fp32).  Here each activation row is
// written as a sum of bf16 rows taken by truncation:
//   fp32: hi = a with its low 16 bits cleared, mid = (a - hi) likewise,
//         lo = a - hi - mid.  Each subtraction is exact in fp32 and lo keeps
//         at most 8 significant bits, so hi + mid + lo equals a for
//         |a| >= 2^-110; below that the part under 2^-133 is dropped.
//         Truncation cannot round a value near the fp32 maximum up to
//         infinity.
//   fp16: hi as above from the exactly widened value, lo = a - hi, which
//         holds at most 3 significant bits: exact for every fp16 value.
// The NP planes form NP*M bf16 rows, [hi rows | (mid rows) | lo rows], which
// the bf16 matrix-core kernel multiplies into fp32 partials without a bias;
// the sum kernel then adds the partials of each output in plane order, adds
// the bias in fp32 and rounds once to the output type.  The same sum combines
// the K parts of the split path's tiled GEMM (up to 4 partials).  Both kernels are
// elementwise and HBM-bound.
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

constexpr int kThreads = 256;

template <int IT>
__global__ __launch_bounds__(kThreads) void split_planes_kernel(const void *__restrict__ A,
                                                                 size_t n,
                                                                 uint16_t *__restrict__ planes) {
    for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < n;
         i += (size_t)gridDim.x * kThreads) {
        if constexpr (IT == kF32) {
            const uint32_t a = __float_as_uint(static_cast<const float *>(A)[i]);
            const uint32_t hi = a & 0xffff0000u;
            const float r1 = __uint_as_float(a) - __uint_as_float(hi);
            const uint32_t mid = __float_as_uint(r1) & 0xffff0000u;
            const float r2 = r1 - __uint_as_float(mid);
            planes[i] = (uint16_t)(hi >> 16);
            planes[n + i] = (uint16_t)(mid >> 16);
            planes[2 * n + i] = (uint16_t)(__float_as_uint(r2) >> 16);
        } else {
            const float a = f16_to_f32(static_cast<const uint16_t *>(A)[i]);
            const uint32_t hi = __float_as_uint(a) & 0xffff0000u;
            const float r = a - __uint_as_float(hi);
            planes[i] = (uint16_t)(hi >> 16);
            planes[n + i] = (uint16_t)(__float_as_uint(r) >> 16);
        }
    }
}

template <int NP>
__global__ __launch_bounds__(kThreads) void sum_planes_kernel(const float *__restrict__ P,
                                                               size_t mn, int N,
                                                               const void *__restrict__ bias,
                                                               void *__restrict__ C, int c_dt) {
    for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < mn;
         i += (size_t)gridDim.x * kThreads) {
        float v = P[i];
#pragma unroll
        for (int q = 1; q < NP; ++q) v += P[q * mn + i];  // in slab order
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

int activation_planes(int a_dt) { return a_dt == kF32 ? 3 : a_dt == kF16 ? 2 : 1; }

hipError_t launch_split_planes(const void *A, int a_dt, size_t n, uint16_t *planes,
                               hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (a_dt == kF32) split_planes_kernel<kF32><<<grid_for(n), kThreads, 0, s>>>(A, n, planes);
    else if (a_dt == kF16) split_planes_kernel<kF16><<<grid_for(n), kThreads, 0, s>>>(A, n, planes);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_sum_planes(const float *P, int np, int M, int N, const void *bias, void *C,
                             int c_dt, hipStream_t s) {
    const size_t mn = (size_t)M * (size_t)N;
    if (mn == 0) return hipSuccess;
#define Q4_SUM(NP) sum_planes_kernel<NP><<<grid_for(mn), kThreads, 0, s>>>(P, mn, N, bias, C, c_dt)
    switch (np) {
    case 2: Q4_SUM(2); break;
    case 3: Q4_SUM(3); break;
    case 4: Q4_SUM(4); break;
    case 5: Q4_SUM(5); break;
    case 6: Q4_SUM(6); break;
    case 7: Q4_SUM(7); break;
    case 8: Q4_SUM(8); break;
    default: return hipErrorInvalidValue;
    }
#undef Q4_SUM
    return hipGetLastError();
}

}  // namespace q4
