// Host-side launchers of the q4skinny kernels (internal to the library).
// Each returns the HIP error of the launch (hipGetLastError, which also
// clears it).  Arguments have been validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4 {

struct DeviceInfo {
    int device;
    int num_cus;
};
DeviceInfo device_info();  // the current device, cached per device

hipError_t launch_dequant(const uint8_t *Wpacked, const float *absmax, const float *codebook,
                          int N, int K, int bs_log2, void *out, bool out_bf16, hipStream_t s);

// Dispatches to the matrix-core kernel (blocksize >= 64) or the vector-ALU
// kernel (blocksize 32).
hipError_t launch_q4_fused(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                           const float *codebook, int M, int N, int K, int bs_log2,
                           uint16_t *C, hipStream_t s);
hipError_t launch_q4_fused_mfma(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                                const float *codebook, int M, int N, int K, int bs_log2,
                                uint16_t *C, hipStream_t s);
hipError_t launch_q4_fused_simt(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                                const float *codebook, int M, int N, int K, int bs_log2,
                                uint16_t *C, hipStream_t s);

hipError_t launch_bf16_gemm(const uint16_t *A, const uint16_t *W, const uint16_t *bias,
                            int M, int N, int K, uint16_t *C, hipStream_t s);

hipError_t launch_copy_probe(const void *src, void *dst, size_t bytes, hipStream_t s);

}  // namespace q4
