// Blockwise 4-bit dequantize: out[n,k] = codebook[code(n,k)] * absmax[n, k/bs].
//
// The dequantize half of the split path of the bitsandbytes pull request
// "[ROCm] Optimize kgemm_4bit_inference_naive for ROCm, use it for batch sizes
// other than 1" (section "Fused path support for M > 1").
//
// HBM-bound: 0.5625 B read + 2 (bf16, fp16) or 4 (fp32) B written per weight.
// The fp32 product is written as is, or rounded once to bf16 or fp16
// (nearest even).  One
// lane handles one 32-bit word of packed codes (8 weights) per step, so a wave
// reads 256 contiguous bytes and writes 1 KiB (bf16) in one store; each lane
// has four such words in flight.  Because K % bs == 0, blocking the flattened
// matrix equals blocking each row, so the scale of flat code index i is
// absmax[i >> bs_log2].
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <int OT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint32_t *__restrict__ packed,
                                                           const float *__restrict__ absmax,
                                                           const float *__restrict__ codebook,
                                                           uint64_t words, int bs_log2,
                                                           void *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int table = __float_as_int(codebook[lane & 15]);
    // Each wave owns runs of 64 * kUnroll consecutive words; the loop bound is
    // uniform across the wave so the permute always runs with all lanes on.
    const uint64_t wave = (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const uint64_t nwaves = (uint64_t)gridDim.x * (kThreads / 64);
    for (uint64_t base = wave * 64 * kUnroll; base < words; base += nwaves * 64 * kUnroll) {
        uint32_t d[kUnroll];
        float am[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t i = base + u * 64 + lane;
            const uint64_t ic = i < words ? i : words - 1;
            d[u] = packed[ic];
            am[u] = absmax[(ic * 8) >> bs_log2];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t i = base + u * 64 + lane;
            float w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = cb_lookup(table, d[u] >> (4 * j)) * am[u];
            if (i < words) {
                if constexpr (OT == kBf16) {
                    uint4 o;
                    o.x = f32_to_bf16_rne(w[0]) | (f32_to_bf16_rne(w[1]) << 16);
                    o.y = f32_to_bf16_rne(w[2]) | (f32_to_bf16_rne(w[3]) << 16);
                    o.z = f32_to_bf16_rne(w[4]) | (f32_to_bf16_rne(w[5]) << 16);
                    o.w = f32_to_bf16_rne(w[6]) | (f32_to_bf16_rne(w[7]) << 16);
                    reinterpret_cast<uint4 *>(out)[i] = o;
                } else if constexpr (OT == kF16) {
                    // The fp32 product is pinned in a register first: the
                    // compiler would otherwise fold multiply and narrowing into
                    // one mixed-precision fma, a single rounding that differs
                    // from rounding the fp32 product (and drops the sign of a
                    // zero product).
#pragma unroll
                    for (int j = 0; j < 8; ++j) __asm__ volatile("" : "+v"(w[j]));
                    uint4 o;
                    o.x = f32_to_f16_rne(w[0]) | (f32_to_f16_rne(w[1]) << 16);
                    o.y = f32_to_f16_rne(w[2]) | (f32_to_f16_rne(w[3]) << 16);
                    o.z = f32_to_f16_rne(w[4]) | (f32_to_f16_rne(w[5]) << 16);
                    o.w = f32_to_f16_rne(w[6]) | (f32_to_f16_rne(w[7]) << 16);
                    reinterpret_cast<uint4 *>(out)[i] = o;
                } else {
                    float4 *o = reinterpret_cast<float4 *>(out) + 2 * i;
                    o[0] = make_float4(w[0], w[1], w[2], w[3]);
                    o[1] = make_float4(w[4], w[5], w[6], w[7]);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_dequant(const uint8_t *Wpacked, const float *absmax, const float *codebook,
                          int N, int K, int bs_log2, void *out, int out_dt, hipStream_t s) {
    const uint64_t words = (uint64_t)N * (uint64_t)K / 8;
    const DeviceInfo info = device_info();
    const uint64_t per_block = (uint64_t)kThreads * kUnroll;
    uint64_t blocks = (words + per_block - 1) / per_block;
    const uint64_t cap = (uint64_t)info.num_cus * 8;
    if (blocks > cap) blocks = cap;
    if (blocks == 0) blocks = 1;
    const uint32_t *packed = reinterpret_cast<const uint32_t *>(Wpacked);
    if (out_dt == kBf16)
        dequant_kernel<kBf16><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
            packed, absmax, codebook, words, bs_log2, out);
    else if (out_dt == kF16)
        dequant_kernel<kF16><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
            packed, absmax, codebook, words, bs_log2, out);
    else
        dequant_kernel<kF32><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
            packed, absmax, codebook, words, bs_log2, out);
    return hipGetLastError();
}

}  // namespace q4
