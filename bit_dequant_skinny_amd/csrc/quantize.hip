// Blockwise 4-bit quantization: W[N,K] -> Wpacked[N,K/2] + absmax[N,K/bs].
//
// The step before the path: it produces the packed weights and block scales
// the fused kernels read (blockwise absmax quantization to a 16-entry table,
// blocksize 64 by default, in the bitsandbytes pull request "[ROCm] Optimize
// kgemm_4bit_inference_naive for ROCm, use it for batch sizes other than 1",
// maintainer's comment).  For a strictly increasing table c[0..15]:
//   absmax = max |w| over the block (exact);
//   code   = the entry nearest to the exact ratio w / absmax, a tie going to
//            the lower entry; a block of zeros takes the ratio 0.
//
// No division: with m_i = (c[i] + c[i+1]) / 2 (computed exactly on the host
// in fp64), the code is the number of i with m_i * absmax < w.  That product
// is exact in fp64; the kernel rounds it up to U_i, the smallest fp32 above
// it, once per block, after which "m_i * absmax < w" is exactly "w >= U_i" for
// every fp32 w.  The U_i do not decrease with i, so "w >= U_i" holds for a
// prefix of i and the code (the length of that prefix) is found by a binary
// search: four compares per weight, each against a threshold picked by the
// earlier answers.
//
// Layout: one lane takes 8 consecutive weights (one packed 32-bit word of
// codes); LPB = bs/8 neighbouring lanes hold one block (K % bs == 0, so
// blocks of the flattened matrix are blocks of its rows), combine their
// maxima with a butterfly of lane swaps, and share the work of the fifteen
// thresholds: lane q of a block computes U_i for i = q mod LPB and reads the
// others from its neighbours.
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

constexpr int kThreads = 256;

// Smallest fp32 strictly above the fp64 value t (t finite, |t| below the
// fp32 range or the result is +-inf as rounding gives).
__device__ __forceinline__ float next_fp32_above(double t) {
    float f = (float)t;  // nearest
    if ((double)f <= t) {
        const uint32_t u = __float_as_uint(f);
        if ((u & 0x7fffffffu) == 0) f = __uint_as_float(1u);       // +-0 -> smallest subnormal
        else if ((u >> 31) == 0) f = __uint_as_float(u + 1u);      // positive: one ulp up
        else f = __uint_as_float(u - 1u);                          // negative: one ulp toward 0
    }
    return f;
}

template <int WT>
__device__ __forceinline__ void load8w(const void *W, uint64_t word, float (&w)[8]) {
    if constexpr (WT == kF32) {
        const float4 *p = reinterpret_cast<const float4 *>(W) + 2 * word;
        const float4 a = p[0], b = p[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
        const uint4 v = reinterpret_cast<const uint4 *>(W)[word];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (WT == kF16) {
                w[2 * t] = f16_to_f32(d[t] & 0xffffu);
                w[2 * t + 1] = f16_to_f32(d[t] >> 16);
            } else {
                w[2 * t] = bf16_lo(d[t]);
                w[2 * t + 1] = bf16_hi(d[t]);
            }
        }
    }
}

// Value select (a conditional on two array elements would select their
// addresses and index the array, which then lives in scratch memory).
__device__ __forceinline__ float sel(bool c, float a, float b) { return c ? a : b; }

// Number of i in 0..14 with x >= U[i], for non-decreasing U (NaN: 0).
__device__ __forceinline__ uint32_t code_of(float x, const float (&U)[15]) {
    const bool b3 = x >= U[7];
    const bool b2 = x >= sel(b3, U[11], U[3]);
    const bool b1 = x >= sel(b3, sel(b2, U[13], U[9]), sel(b2, U[5], U[1]));
    const float t0 = sel(b3, sel(b2, sel(b1, U[14], U[12]), sel(b1, U[10], U[8])),
                         sel(b2, sel(b1, U[6], U[4]), sel(b1, U[2], U[0])));
    const bool b0 = x >= t0;
    return (b3 ? 8u : 0u) | (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
}

template <int WT, int LPB>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const void *__restrict__ W, uint64_t words, QuantizeTable tab,
    uint32_t *__restrict__ packed, float *__restrict__ absmax) {
    constexpr int lpb = LPB;  // lanes per block (4..32)
    constexpr int bs_log2 = LPB == 4 ? 5 : LPB == 8 ? 6 : LPB == 16 ? 7 : 8;
    constexpr int S = (15 + LPB - 1) / LPB;  // thresholds each lane computes
    __shared__ double s_mid[16];
    if (threadIdx.x < 15) s_mid[threadIdx.x] = tab.mid[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int q = lane & (LPB - 1), base_lane = lane & ~(LPB - 1);
    const uint64_t wave = (uint64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const uint64_t nwaves = (uint64_t)gridDim.x * (kThreads / 64);
    // The loop bound is uniform across the wave (64 words = 512 weights, a
    // multiple of every blocksize), so the lane swaps run with all lanes on.
    for (uint64_t base = wave * 64; base < words; base += nwaves * 64) {
        const uint64_t word = base + lane;
        const bool live = word < words;
        float w[8];
        if (live) {
            load8w<WT>(W, word, w);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = 0.f;
        }
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(w[j]));
        for (int off = 1; off < lpb; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
        // U[i] is computed by lane i % LPB of the block (every lane runs the
        // shuffles, so they happen with all lanes on)
        float mine[S];
#pragma unroll
        for (int k = 0; k < S; ++k) {
            const int i = q + LPB * k;
            mine[k] = i < 15 ? next_fp32_above(s_mid[i] * (double)a) : 0.f;
        }
        float U[15];
#pragma unroll
        for (int i = 0; i < 15; ++i) U[i] = __shfl(mine[i / LPB], base_lane + i % LPB, 64);
        uint32_t out;
        if (a > 0.f) {
            out = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) out |= code_of(w[j], U) << (4 * j);
        } else {
            out = tab.zero_code * 0x11111111u;
        }
        if (live) {
            packed[word] = out;
            if ((lane & (lpb - 1)) == 0) absmax[(word * 8) >> bs_log2] = a;
        }
    }
}

}  // namespace

hipError_t launch_quantize(const void *W, int w_dt, int N, int K, int bs_log2,
                           const QuantizeTable &tab, uint8_t *Wpacked, float *absmax,
                           hipStream_t s) {
    const uint64_t words = (uint64_t)N * (uint64_t)K / 8;
    const DeviceInfo info = device_info();
    const uint64_t per_block = (uint64_t)kThreads;  // one word per thread per pass
    uint64_t blocks = (words + per_block - 1) / per_block;
    const uint64_t cap = (uint64_t)info.num_cus * 16;
    if (blocks > cap) blocks = cap;
    if (blocks == 0) blocks = 1;
    uint32_t *packed = reinterpret_cast<uint32_t *>(Wpacked);
#define Q4_QUANT(T, L) \
    quantize_kernel<T, L><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(W, words, tab, packed, absmax)
#define Q4_QUANT_BS(T)                         \
    switch (bs_log2) {                         \
    case 5: Q4_QUANT(T, 4); break;             \
    case 6: Q4_QUANT(T, 8); break;             \
    case 7: Q4_QUANT(T, 16); break;            \
    case 8: Q4_QUANT(T, 32); break;            \
    default: return hipErrorInvalidValue;      \
    }
    if (w_dt == kF32) {
        Q4_QUANT_BS(kF32)
    } else if (w_dt == kF16) {
        Q4_QUANT_BS(kF16)
    } else {
        Q4_QUANT_BS(kBf16)
    }
#undef Q4_QUANT_BS
#undef Q4_QUANT
    return hipGetLastError();
}

}  // namespace q4
