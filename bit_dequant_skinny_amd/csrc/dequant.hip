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
//
// Weights in the tile layout (16-row tiles of 1 KiB units, see
// repack_q4_tiles_kernel) take dequant_tiles_kernel: the same arithmetic in
// the order of the tiles, each lane turning one 16-byte piece (16 weights of
// each 64-wide half of one row's segment, each run inside one scale block
// since bs >= 64) into 32 outputs; 16-bit outputs go through LDS so that the
// stores run along rows (1 KiB per row and store), fp32 outputs are stored
// from the lanes (two runs of 64 bytes each).
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

template <int OT>
__global__ __launch_bounds__(kThreads) void dequant_tiles_kernel(
    const uint4 *__restrict__ tiles, const float *__restrict__ absmax,
    const float *__restrict__ codebook, uint32_t pieces, uint32_t nseg, int K, int bs_log2,
    void *__restrict__ out) {
    constexpr int kRowLds = 272, kUnitLds = 16 * kRowLds;
    __shared__ __attribute__((aligned(16))) char stage[OT == kF32 ? 16 : 4 * kUnitLds];
    const int lane = threadIdx.x & 63;
    const int table = __float_as_int(codebook[lane & 15]);
    const uint32_t nb = (uint32_t)K >> bs_log2;
    const uint32_t stride = gridDim.x * kThreads;
    // every thread runs each step (the lookup is cross-lane, the staging
    // needs the block's barriers); lanes past the end repeat the last piece
    // and store nothing
    const uint32_t p_end = (pieces + stride - 1) / stride * stride;
    for (uint32_t p0 = blockIdx.x * kThreads + threadIdx.x; p0 < p_end; p0 += stride) {
        const uint32_t p = p0 < pieces ? p0 : pieces - 1;
        const uint32_t unit = p >> 6, l = p & 63;
        const uint32_t t = unit / nseg, seg = unit - t * nseg;
        const uint32_t n = 16 * t + (l & 15);
        // the piece holds 16 weights of each 64-wide half of the segment,
        // starting at k0 and k0 + 64 (quarter a = 0, 2, 1, 3 by lane group)
        const uint32_t gl = l >> 4, a = 2 * (gl & 1) + (gl >> 1);
        const uint32_t k0 = 128 * seg + 16 * a;
        const uint4 v = tiles[p];
        const float am0 = absmax[n * nb + (k0 >> bs_log2)];
        const float am1 = absmax[n * nb + ((k0 + 64) >> bs_log2)];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        float w[32];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                w[8 * u + j] = cb_lookup(table, d[u] >> (4 * j)) * (u < 2 ? am0 : am1);
        const bool live = p0 < pieces;
        const size_t e0 = (size_t)n * (size_t)K + k0;  // first output element of each half
        if constexpr (OT == kF32) {
            float4 *o = reinterpret_cast<float4 *>(static_cast<float *>(out) + e0);
            if (live)
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    o[q + (q < 4 ? 0 : 12)] = make_float4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
        } else {
            if constexpr (OT == kF16) {
#pragma unroll
                for (int j = 0; j < 32; ++j) __asm__ volatile("" : "+v"(w[j]));
            }
            // Staged through LDS so that the stores run along rows: wave w
            // puts its unit's 16 rows x 256 bytes at w * kUnitLds (rows kRowLds
            // apart, 16 bytes of padding keep the 16 rows of a store in
            // distinct banks); then store c of the block writes row c / 64,
            // 16-byte chunk c % 64 of the four units' runs (one 1 KiB run per
            // row when the four units are consecutive segments of one tile).
            const int wv = threadIdx.x >> 6;
            char *mine = stage + wv * kUnitLds + (l & 15) * kRowLds + 32 * a;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t h[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    h[j] = OT == kBf16 ? f32_to_bf16_rne(w[8 * q + j]) : f32_to_f16_rne(w[8 * q + j]);
                *reinterpret_cast<uint4 *>(mine + 16 * q + (q < 2 ? 0 : 96)) =
                    make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                               h[6] | (h[7] << 16));
            }
            __syncthreads();
            const uint32_t unit0 = (p0 - threadIdx.x) >> 6;  // the block's first unit
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = (int)threadIdx.x + kThreads * i;
                const int r = c >> 6, uw = (c >> 4) & 3, y = c & 15;
                const uint32_t u = unit0 + (uint32_t)uw;
                const uint32_t ut = u / nseg, us = u - ut * nseg;
                const uint4 v16 = *reinterpret_cast<const uint4 *>(stage + uw * kUnitLds + r * kRowLds + 16 * y);
                if (u < pieces / 64) {
                    const size_t e = (size_t)(16 * ut + r) * (size_t)K + 128 * us + 8 * y;
                    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + e) = v16;
                }
            }
            __syncthreads();
        }
    }
}

// Row-major packed codes -> tile layout.  Tile t holds rows 16t..16t+15;
// (tile t, segment s) is the 1 KiB unit (t * K/128 + s): 64 pieces of 16
// bytes, piece l holding row 16t + l % 16, bytes 64s + 8a .. +8 and
// 64s + 32 + 8a .. +8 with a = 0, 2, 1, 3 for l / 16 = 0..3 (the 16 bytes a
// matrix-core lane l decodes for one 128-wide segment: 8 from each 64-wide
// block).  Each thread writes one piece per step, so the writes are
// contiguous.
__global__ __launch_bounds__(kThreads) void repack_q4_tiles_kernel(const uint2 *__restrict__ src,
                                                                   uint4 *__restrict__ dst,
                                                                   uint32_t pieces, uint32_t nseg,
                                                                   uint32_t row_halves) {
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t p = blockIdx.x * kThreads + threadIdx.x; p < pieces; p += stride) {
        const uint32_t unit = p >> 6, l = p & 63;
        const uint32_t t = unit / nseg, seg = unit - t * nseg;
        const uint32_t n = 16 * t + (l & 15), gl = l >> 4, a = 2 * (gl & 1) + (gl >> 1);
        const uint2 h0 = src[n * row_halves + 8 * seg + a];
        const uint2 h1 = src[n * row_halves + 8 * seg + a + 4];
        dst[p] = make_uint4(h0.x, h0.y, h1.x, h1.y);
    }
}

// Row-major bf16 weights -> their tile layout: (tile t, step s) is one unit
// of 64 pieces of 16 bytes, piece l being bytes 64s + 16(l / 16) .. +16 of
// row 16t + l % 16 (8 consecutive k).  A pure permutation of 16-byte pieces;
// each thread moves one piece per step, so the writes are contiguous and each
// wave reads 64-byte runs of 16 rows.
__global__ __launch_bounds__(kThreads) void repack_tiles_kernel(const uint4 *__restrict__ src,
                                                                uint4 *__restrict__ dst,
                                                                uint32_t pieces, uint32_t nseg,
                                                                uint32_t row_pieces) {
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t p = blockIdx.x * kThreads + threadIdx.x; p < pieces; p += stride) {
        const uint32_t unit = p >> 6, l = p & 63;
        const uint32_t t = unit / nseg, seg = unit - t * nseg;
        const uint32_t n = 16 * t + (l & 15);
        dst[p] = src[n * row_pieces + 4 * seg + (l >> 4)];
    }
}

}  // namespace

namespace {

// The 16-row tiling of bf16 weights: rows of row_bytes bytes (a multiple of
// 64) cut into 64-byte columns; (tile, column) is one 1 KiB unit.
hipError_t repack_rows16(const void *src, void *dst, int N, uint64_t row_bytes, hipStream_t s) {
    if (N % 16 != 0 || row_bytes % 64 != 0 || (uint64_t)N * row_bytes >= (1ull << 32))
        return hipErrorInvalidValue;
    const uint32_t pieces = (uint32_t)((uint64_t)N * row_bytes / 16);
    const DeviceInfo info = device_info();
    uint32_t blocks = (pieces + kThreads - 1) / kThreads;
    const uint32_t cap = (uint32_t)info.num_cus * 8;
    if (blocks > cap) blocks = cap;
    if (blocks == 0) return hipSuccess;
    repack_tiles_kernel<<<dim3(blocks), dim3(kThreads), 0, s>>>(
        reinterpret_cast<const uint4 *>(src), reinterpret_cast<uint4 *>(dst), pieces,
        (uint32_t)(row_bytes / 64), (uint32_t)(row_bytes / 16));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_repack_tiles(const uint8_t *Wpacked, uint8_t *Wtiles, int N, int K,
                               hipStream_t s) {
    const uint64_t row_bytes = (uint64_t)K / 2;
    if (K % 128 != 0 || N % 16 != 0 || (uint64_t)N * row_bytes >= (1ull << 32))
        return hipErrorInvalidValue;
    const uint32_t pieces = (uint32_t)((uint64_t)N * row_bytes / 16);
    uint32_t blocks = (pieces + kThreads - 1) / kThreads;
    const uint32_t cap = (uint32_t)device_info().num_cus * 8;
    if (blocks > cap) blocks = cap;
    if (blocks == 0) return hipSuccess;
    repack_q4_tiles_kernel<<<dim3(blocks), dim3(kThreads), 0, s>>>(
        reinterpret_cast<const uint2 *>(Wpacked), reinterpret_cast<uint4 *>(Wtiles), pieces,
        (uint32_t)(row_bytes / 64), (uint32_t)(row_bytes / 8));
    return hipGetLastError();
}

// bf16 weights: a unit is 16 rows x 32 k (the 64 bytes of a row one
// matrix-core step consumes), piece l = row l % 16, k 8(l / 16) .. +8.
hipError_t launch_bf16_repack_tiles(const uint16_t *W, uint16_t *Wtiles, int N, int K,
                                    hipStream_t s) {
    if (K % 32 != 0) return hipErrorInvalidValue;
    return repack_rows16(W, Wtiles, N, (uint64_t)K * 2, s);
}

hipError_t launch_dequant(const uint8_t *Wpacked, const float *absmax, const float *codebook,
                          int N, int K, int bs_log2, int wl, void *out, int out_dt, hipStream_t s) {
    if (wl && (N % 16 != 0 || K % 128 != 0 || (uint64_t)N * (uint64_t)K / 2 >= (1ull << 32)))
        return hipErrorInvalidValue;
    if (wl) {
        const uint32_t pieces = (uint32_t)((uint64_t)N * (uint64_t)K / 32);
        const DeviceInfo info = device_info();
        uint32_t blocks = (pieces + kThreads - 1) / kThreads;
        const uint32_t cap = (uint32_t)info.num_cus * 8;
        if (blocks > cap) blocks = cap;
        if (blocks == 0) return hipSuccess;
        const uint4 *tiles = reinterpret_cast<const uint4 *>(Wpacked);
        const uint32_t nseg = (uint32_t)K / 128;
        if (out_dt == kBf16)
            dequant_tiles_kernel<kBf16><<<dim3(blocks), dim3(kThreads), 0, s>>>(
                tiles, absmax, codebook, pieces, nseg, K, bs_log2, out);
        else if (out_dt == kF16)
            dequant_tiles_kernel<kF16><<<dim3(blocks), dim3(kThreads), 0, s>>>(
                tiles, absmax, codebook, pieces, nseg, K, bs_log2, out);
        else
            dequant_tiles_kernel<kF32><<<dim3(blocks), dim3(kThreads), 0, s>>>(
                tiles, absmax, codebook, pieces, nseg, K, bs_log2, out);
        return hipGetLastError();
    }
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
