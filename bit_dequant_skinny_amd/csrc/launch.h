// Host-side launchers of the q4skinny kernels (internal to the library).
// Each returns the HIP error of the launch (hipGetLastError, which also
// clears it).  Arguments have been validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "q4skinny.h"

namespace q4 {

struct DeviceInfo {
    int device;
    int num_cus;
};
DeviceInfo device_info();  // the current device, cached per device

// Element types are the Q4_DTYPE_* codes (kBf16, kF32, kF16 in device.h).
hipError_t launch_dequant(const uint8_t *Wpacked, const float *absmax, const float *codebook,
                          int N, int K, int bs_log2, int wl, void *out, int out_dt, hipStream_t s);
// Weight layouts (wl): 0 = row-major packed rows, 1 = 16-row tiles of 1 KiB
// units (N % 16 == 0, K % 128 == 0; see launch_repack_tiles).
hipError_t launch_repack_tiles(const uint8_t *Wpacked, uint8_t *Wtiles, int N, int K,
                               hipStream_t s);
// bf16 weights [N, K] -> 16-row tiles of 1 KiB units of 32 k (N % 16 == 0,
// K % 32 == 0, N*K*2 below 4 GiB).
hipError_t launch_bf16_repack_tiles(const uint16_t *W, uint16_t *Wtiles, int N, int K,
                                    hipStream_t s);

// Fused 4-bit GEMM, C = A * dequant(W)^T (+ bias), A of type a_dt, bias and C
// of type c_dt.  Dispatches to the matrix-core kernel (bf16 or fp16
// activations, blocksize >= 64) or the vector-ALU kernel (blocksize 32, fp32
// activations, offsets beyond 32 bits).  kpart: room for
// q4_fused_kparts(M, N, K) * M * N fp32 partial sums, which lets the skinny
// kernel split K over workgroups (then a second kernel adds the parts).
hipError_t launch_q4_fused(const void *A, int a_dt, const uint8_t *Wpacked, const float *absmax,
                           const float *codebook, const void *bias, int M, int N, int K,
                           int bs_log2, void *C, int c_dt, int wl, hipStream_t s,
                           float *kpart = nullptr);
// The skinny matrix-core kernel alone.  np = 2 / 3: A holds the exact bf16
// planes [np][M][K] of fp16 / fp32 activations, summed per token inside the
// kernel before the bias and the rounding (np * ceil(M / 4) <= 4, no kpart).
hipError_t launch_q4_fused_mfma(const void *A, int a_dt, const uint8_t *Wpacked,
                                const float *absmax, const float *codebook, const void *bias,
                                int M, int N, int K, int bs_log2, void *C, int c_dt, int wl,
                                hipStream_t s, float *kpart = nullptr, int np = 1);
// K parts the skinny kernel would use for M bf16 token rows (1 = none).
int q4_fused_kparts(int M, int N, int K);
hipError_t launch_q4_fused_simt(const void *A, int a_dt, const uint8_t *Wpacked,
                                const float *absmax, const float *codebook, const void *bias,
                                int M, int N, int K, int bs_log2, void *C, int c_dt,
                                hipStream_t s);

// fp16 / fp32 activations as 2 / 3 exact bf16 planes ([np][n]) and the sum of
// np (2..8) fp32 partials ([np][M][N]) plus bias, rounded once to c_dt.
int activation_planes(int a_dt);
hipError_t launch_split_planes(const void *A, int a_dt, size_t n, uint16_t *planes,
                               hipStream_t s);
hipError_t launch_sum_planes(const float *P, int np, int M, int N, const void *bias, void *C,
                             int c_dt, hipStream_t s);
bool q4_fused_mfma_fits(int M, int N, int K);
// 16-row tiles each workgroup of the skinny kernel covers per chunk (1..8).
int q4_fused_tiles_per_chunk(int N);
bool q4_fused_mfma_two_blocks(int N);

// Fused 4-bit GEMM with output tiles of 64 (32 for M <= 32) tokens (bf16 A,
// blocksize >= 64), for tens to hundreds of token rows.  Layout 0: 4 waves
// split K over a 64-feature tile; layout 1: 8 waves split a 256-feature tile.
// ksplit > 1 writes ksplit fp32 partial outputs [ksplit][M][N] (no bias) for
// launch_sum_planes to add.  q4_fused_tiled_plan picks both for a shape
// (ksplit <= max_ks; layout -1 = by shape, 0 or 1 = forced).
struct TiledPlan {
    int layout;
    int ksplit;
};
bool q4_fused_tiled_fits(int M, int N, int K);
TiledPlan q4_fused_tiled_plan(int M, int N, int K, int max_ks, int layout);
hipError_t launch_q4_fused_tiled(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                                 const float *codebook, const void *bias, int M, int N, int K,
                                 int bs_log2, int wl, const TiledPlan &plan, void *C, int c_dt,
                                 hipStream_t s);

// Tiled bf16 GEMM (bf16 A, 128 x 128 tiles through LDS) for the split path at
// larger M; gemm_tiled_fits checks its 32-bit offsets.
// ksplit > 1 writes ksplit fp32 partial outputs [ksplit][M][N] (no bias) for
// launch_sum_planes to add; gemm_tiled_ksplit picks the split for a shape.
bool gemm_tiled_fits(int M, int N, int K);
int gemm_tiled_ksplit(int M, int N, int K);
hipError_t launch_gemm_tiled(const uint16_t *A, const uint16_t *W, const void *bias, int M,
                             int N, int K, int ksplit, void *C, int c_dt, hipStream_t s);

// bf16-weight GEMM on the matrix cores, C = A * W^T (+ bias); A bf16 or fp16.
// wl = 1: W in the tile layout of launch_bf16_repack_tiles (bf16 A, M <= 16,
// bf16_tiles_fit(N, K)).
hipError_t launch_bf16_gemm(const void *A, int a_dt, const uint16_t *W, const void *bias, int M,
                            int N, int K, void *C, int c_dt, hipStream_t s, int wl = 0);
bool bf16_tiles_fit(int N, int K);

// Quantizer thresholds derived on the host from a strictly increasing table:
// mid[i] = (c[i] + c[i+1]) / 2 in fp64 (exact), zero_code = the entry nearest
// to 0 (ties to the lower one).
struct QuantizeTable {
    double mid[15];
    uint32_t zero_code;
};
hipError_t launch_quantize(const void *W, int w_dt, int N, int K, int bs_log2,
                           const QuantizeTable &tab, uint8_t *Wpacked, float *absmax,
                           hipStream_t s);

hipError_t launch_copy_probe(const void *src, void *dst, size_t bytes, hipStream_t s);

// q4_gemm_skinny_ex with every workspace request served from `scratch`
// (scratch_bytes long) instead of the per-stream workspace: a request that
// does not fit returns Q4_ERR_UNSUPPORTED before anything is launched.
// Defined in capi.cpp.
q4_status gemm_ex_fixed_scratch(const void *A, int a_dtype, const uint8_t *Wpacked,
                                const float *absmax, const float *codebook, const void *bias,
                                int M, int N, int K, int blocksize, void *C, int c_dtype,
                                void *stream, int path, void *scratch, size_t scratch_bytes);
// Drains the HIP error flag and records "what: <HIP message>" for
// q4_last_error; returns st.  Defined in capi.cpp.
q4_status report(q4_status st, const char *what, hipError_t e);
// Read-only stream over `bytes` (< 4 GiB) by num_cus * wgs_per_cu workgroups
// of `threads` (256, 512, 1024) lanes, `unroll` (2, 4, 8) 16-byte loads per
// lane per batch; nt = non-temporal loads, interleave = batches dealt round
// robin instead of contiguous shares.  `sink` (4 bytes) is written only if
// the folded data equals a fixed value.
bool read_probe_shape_ok(int threads, int unroll);
hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, int threads,
                             int unroll, int wgs_per_cu, int nt, int interleave, hipStream_t s);

}  // namespace q4
