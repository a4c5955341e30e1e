// Fused blockwise-4-bit dequantize + skinny GEMM on the vector ALUs:
// C[M,N] = A[M,K] * dequant(W)^T (+ bias).  Serves blocksize 32, whose blocks
// are narrower than the 64-wide scale granule of the matrix-core kernel, fp32
// activations (widened exactly, multiplied in fp32), and shapes beyond the
// matrix-core kernel's 32-bit offsets.
//
// The fused path of the bitsandbytes pull request "[ROCm] Optimize
// kgemm_4bit_inference_naive for ROCm, use it for batch sizes other than 1"
// (sections "Kernel optimization" and "Fused path support for M > 1"): each
// packed weight byte is read from HBM once, decoded through the 16-entry
// table, scaled by its block's absmax and multiplied into fp32 accumulators
// for every token row.
//
// Work split: one wave owns ROWS consecutive output features.  Its 64 lanes
// walk the row in 16-byte chunks (32 codes), lane l taking chunks l, l+64, ...
// so a wave reads 1 KiB of each row per step with one global_load_dwordx4 per
// lane.  A chunk never straddles a quantization block (bs >= 32), so a lane
// sums its 32 products per token first and applies the block scale once.  The
// 64 per-lane partial sums of each output are combined with a fixed-order
// cross-lane tree (no atomics; the result is deterministic).
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

constexpr int kThreads = 256;

// Eight consecutive activations of type AT (bf16, fp16 or fp32), widened to
// fp32 exactly.
template <int AT>
__device__ __forceinline__ void load8(const void *A, size_t i, float (&a)[8]) {
    if constexpr (AT == kF32) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(A) + i);
        const float4 u = p[0], v = p[1];
        a[0] = u.x; a[1] = u.y; a[2] = u.z; a[3] = u.w;
        a[4] = v.x; a[5] = v.y; a[6] = v.z; a[7] = v.w;
    } else {
        const uint4 av = ld128(static_cast<const uint16_t *>(A) + i);
        const uint32_t d[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (AT == kF16) {
                a[2 * t] = f16_to_f32(d[t] & 0xffffu);
                a[2 * t + 1] = f16_to_f32(d[t] >> 16);
            } else {
                a[2 * t] = bf16_lo(d[t]);
                a[2 * t + 1] = bf16_hi(d[t]);
            }
        }
    }
}

template <int AT, int MT, int ROWS>
__global__ __launch_bounds__(kThreads) void fused_rows_kernel(
    const void *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ absmax, const float *__restrict__ codebook,
    const void *__restrict__ bias, int M, int N, int K, int bs_log2, void *__restrict__ C,
    int c_dt) {
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int n0 = wave * ROWS;
    if (n0 >= N) return;  // whole wave leaves together
    const int table = __float_as_int(codebook[lane & 15]);
    const int chunks = K >> 5;
    const int nb = K >> bs_log2;
    const size_t row_bytes = (size_t)K >> 1;

    int rows[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) rows[r] = (n0 + r < N) ? n0 + r : N - 1;

    float acc[ROWS][MT];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

    for (int c0 = 0; c0 < chunks; c0 += 64) {
        const int c = c0 + lane;
        const bool valid = c < chunks;
        const int cc = valid ? c : chunks - 1;
        uint4 w[ROWS];
        float am[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            w[r] = ld128(Wp + (size_t)rows[r] * row_bytes + (size_t)cc * 16);
            am[r] = absmax[(size_t)rows[r] * nb + ((cc << 5) >> bs_log2)];
        }
        float part[ROWS][MT];
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) part[r][m] = 0.f;
#pragma unroll 1
        for (int q = 0; q < 4; ++q) {
            // Decode this dword of every row once, then stream the token rows
            // past it one at a time (8 activations live, whatever MT is).
            float v[ROWS][8];
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const uint32_t d = (q == 0) ? w[r].x : (q == 1) ? w[r].y : (q == 2) ? w[r].z : w[r].w;
#pragma unroll
                for (int j = 0; j < 8; ++j) v[r][j] = cb_lookup(table, d >> (4 * j));
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float a[8];
                if (m < M && valid) {
                    load8<AT>(A, (size_t)m * K + (size_t)cc * 32 + q * 8, a);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = 0.f;
                }
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
#pragma unroll
                    for (int j = 0; j < 8; ++j) part[r][m] = fmaf(a[j], v[r][j], part[r][m]);
            }
        }
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = fmaf(am[r], part[r][m], acc[r][m]);
    }

#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[r][m] = wave_sum(acc[r][m]);

    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (n0 + r < N && m < M) {
                    float v = acc[r][m];
                    if (bias) v += load_elem(bias, n0 + r, c_dt);  // before the single rounding
                    store_elem(C, (size_t)m * N + n0 + r, v, c_dt);
                }
    }
}

template <int AT, int MT, int ROWS>
hipError_t launch_rows(const void *A, const uint8_t *Wp, const float *absmax,
                       const float *codebook, const void *bias, int M, int N, int K, int bs_log2,
                       void *C, int c_dt, hipStream_t s) {
    const int waves = (N + ROWS - 1) / ROWS;
    const int blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
    fused_rows_kernel<AT, MT, ROWS><<<dim3(blocks), dim3(kThreads), 0, s>>>(
        A, Wp, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt);
    return hipGetLastError();
}

template <int AT>
hipError_t launch_at(const void *A, const uint8_t *Wp, const float *absmax, const float *codebook,
                     const void *bias, int M, int N, int K, int bs_log2, void *C, int c_dt,
                     hipStream_t s) {
    if (M <= 1) return launch_rows<AT, 1, 8>(A, Wp, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt, s);
    if (M <= 2) return launch_rows<AT, 2, 8>(A, Wp, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt, s);
    if (M <= 4) return launch_rows<AT, 4, 4>(A, Wp, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt, s);
    if (M <= 8) return launch_rows<AT, 8, 2>(A, Wp, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt, s);
    return launch_rows<AT, 16, 1>(A, Wp, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt, s);
}

}  // namespace

hipError_t launch_q4_fused_simt(const void *A, int a_dt, const uint8_t *Wpacked,
                                const float *absmax, const float *codebook, const void *bias,
                                int M, int N, int K, int bs_log2, void *C, int c_dt,
                                hipStream_t s) {
    if (a_dt == kF32)
        return launch_at<kF32>(A, Wpacked, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt, s);
    if (a_dt == kF16)
        return launch_at<kF16>(A, Wpacked, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt, s);
    return launch_at<kBf16>(A, Wpacked, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt, s);
}

}  // namespace q4
