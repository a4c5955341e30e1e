// Fused blockwise-4-bit dequantize + skinny GEMM on the vector ALUs:
// C[M,N] = A[M,K] * dequant(W)^T.  Serves blocksize 32, whose blocks are
// narrower than the 64-wide scale granule of the matrix-core kernel.
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

template <int MT, int ROWS>
__global__ __launch_bounds__(kThreads) void fused_rows_kernel(
    const uint16_t *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ absmax, const float *__restrict__ codebook, int M, int N, int K,
    int bs_log2, uint16_t *__restrict__ C) {
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
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float a[MT][8];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                uint4 av = make_uint4(0, 0, 0, 0);
                if (m < M && valid) av = ld128(A + (size_t)m * K + (size_t)cc * 32 + q * 8);
                a[m][0] = bf16_lo(av.x); a[m][1] = bf16_hi(av.x);
                a[m][2] = bf16_lo(av.y); a[m][3] = bf16_hi(av.y);
                a[m][4] = bf16_lo(av.z); a[m][5] = bf16_hi(av.z);
                a[m][6] = bf16_lo(av.w); a[m][7] = bf16_hi(av.w);
            }
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const uint32_t d = (q == 0) ? w[r].x : (q == 1) ? w[r].y : (q == 2) ? w[r].z : w[r].w;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float v = cb_lookup(table, d >> (4 * j));
#pragma unroll
                    for (int m = 0; m < MT; ++m) part[r][m] = fmaf(a[m][j], v, part[r][m]);
                }
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
                if (n0 + r < N && m < M)
                    C[(size_t)m * N + n0 + r] = (uint16_t)f32_to_bf16_rne(acc[r][m]);
    }
}

template <int MT, int ROWS>
hipError_t launch_rows(const uint16_t *A, const uint8_t *Wp, const float *absmax,
                       const float *codebook, int M, int N, int K, int bs_log2, uint16_t *C,
                       hipStream_t s) {
    const int waves = (N + ROWS - 1) / ROWS;
    const int blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
    fused_rows_kernel<MT, ROWS><<<dim3(blocks), dim3(kThreads), 0, s>>>(A, Wp, absmax, codebook,
                                                                         M, N, K, bs_log2, C);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_fused_simt(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                                const float *codebook, int M, int N, int K, int bs_log2,
                                uint16_t *C, hipStream_t s) {
    if (M <= 1) return launch_rows<1, 8>(A, Wpacked, absmax, codebook, M, N, K, bs_log2, C, s);
    if (M <= 2) return launch_rows<2, 8>(A, Wpacked, absmax, codebook, M, N, K, bs_log2, C, s);
    if (M <= 4) return launch_rows<4, 4>(A, Wpacked, absmax, codebook, M, N, K, bs_log2, C, s);
    if (M <= 8) return launch_rows<8, 2>(A, Wpacked, absmax, codebook, M, N, K, bs_log2, C, s);
    return launch_rows<16, 2>(A, Wpacked, absmax, codebook, M, N, K, bs_log2, C, s);
}

}  // namespace q4
