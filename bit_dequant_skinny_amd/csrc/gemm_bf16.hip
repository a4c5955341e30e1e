// bf16 skinny GEMM on the matrix cores: C[M,N] = A[M,K] * W[N,K]^T (+ bias).
//
// Serves two steps of the path:
//  * the unquantized skinny GEMM for 1..5 token rows described in the report
//    on vLLM pull request 40687 "Support N=5 in wvSplitK skinny GEMM kernels
//    for speculative decoding" (section "关键源码片段": K % 8 == 0, optional
//    bias, a per-token-count tile);
//  * the GEMM half of the split path (dequantize to bf16, then GEMM) of the
//    bitsandbytes pull request "[ROCm] Optimize kgemm_4bit_inference_naive
//    ..." (section "Fused path support for M > 1").
//
// One wave computes a 16-feature x (16*MT)-token tile with
// v_mfma_f32_16x16x32_bf16.  Tokens go in the A operand (row i = lane % 16),
// weights in the B operand (column j = lane % 16); lane group g = lane / 16
// supplies 8 consecutive k of the 32 each instruction consumes, read with one
// 16-byte load per lane, so each weight row is read 64 contiguous bytes at a
// time and every weight byte exactly once.  Token rows >= M feed zeros.  At
// M <= 16 the arithmetic intensity is <= 16 flop/byte, far below the MFMA
// ridge: the kernel is HBM-bound and the matrix cores only remove the VALU
// work (no bf16 -> fp32 conversion, no per-element FMA).
//
// When N is small the waves of a workgroup split K and combine their fp32
// tiles through LDS in a fixed order (deterministic, no atomics).
//
// Up to 16 token rows (the skinny case and the split path's slabs of 16) take
// one of two streaming kernels, which use buffer loads whose hardware range
// check returns zeros past the end of a buffer, so absent token rows, weight
// rows past N and steps past the wave's share of K cost no memory traffic
// and need no branches.  Over this library's tile layout (bf16_repack_tiles:
// the 16 rows x 32 k one instruction consumes stored as one contiguous 1 KiB
// unit in lane order) each wave keeps kRing steps of weights and their
// activations in flight in a register ring, one 1 KiB load per step.  Over
// row-major weights each load instruction reads whole 512-byte runs of two
// rows, and the wave reorders them through LDS into the same operands.
// Lanes receive the same values in the same registers in both, so the two
// layouts give bit-identical results.  Wider slabs take the plain kernel.
//
// fp16 activations (split path of the 4-bit GEMM) are split exactly into
// bf16 hi + lo and take two MFMAs per step.  The bias (optional) has the
// output's type; the output is bf16, fp16 or fp32, rounded once from the fp32
// sum plus bias.
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

constexpr int kRing = 8;                     // steps of 32 k in flight per wave
constexpr uint32_t kPastEnd = 0x80000000u;   // an offset beyond every buffer: reads zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

template <int AT>
__device__ __forceinline__ floatx4 mfma_step(uint4 av, uint4 wv, floatx4 acc) {
    if constexpr (AT == kF16) {
        const uint2 x = f16x2_to_bf16_hilo(av.x), y = f16x2_to_bf16_hilo(av.y);
        const uint2 z = f16x2_to_bf16_hilo(av.z), w = f16x2_to_bf16_hilo(av.w);
        acc = mfma_bf16_16x16x32(as_bf16x8(make_uint4(x.x, y.x, z.x, w.x)), as_bf16x8(wv), acc);
        return mfma_bf16_16x16x32(as_bf16x8(make_uint4(x.y, y.y, z.y, w.y)), as_bf16x8(wv), acc);
    } else {
        return mfma_bf16_16x16x32(as_bf16x8(av), as_bf16x8(wv), acc);
    }
}

// Streaming kernel for M <= 16 over the tile layout (unit (tile, step) at
// (tile * K/32 + step) * 1 KiB, lane l's 16 bytes at 16 l; needs N % 16 == 0
// and K % 32 == 0): wave (tile, k part) as in bf16_gemm_kernel, every step
// one 16-byte weight load and one 16-byte activation load per lane, kRing
// steps ahead of the MFMA that consumes them.
template <int AT>
__global__ __launch_bounds__(kThreads) void bf16_stream_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W,
    const void *__restrict__ bias, int M, int N, int K, int ksplit,
    void *__restrict__ C, int c_dt) {
    __shared__ floatx4 red[kWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tiles_per_block = kWaves / ksplit;
    const int tile = blockIdx.x * tiles_per_block + wave / ksplit;
    const int kpart = wave % ksplit;
    const int n0 = tile * 16;
    const int j = lane & 15;
    const int g = lane >> 4;

    const int steps = (K + 31) >> 5;
    const int s_begin = (kpart * steps) / ksplit;
    const int s_end = ((kpart + 1) * steps) / ksplit;

    const __amdgpu_buffer_rsrc_t wres = make_rsrc(W, (uint32_t)N * (uint32_t)K * 2);
    const __amdgpu_buffer_rsrc_t ares = make_rsrc(A, (uint32_t)M * (uint32_t)K * 2);
    // tokens past M lie beyond the activations
    const uint32_t a_row = (uint32_t)j * (uint32_t)K * 2;
    auto offs = [&](int st, uint32_t row) -> uint32_t {
        const uint32_t k = (uint32_t)(st << 5) + (uint32_t)(g << 3);
        return (st < s_end && k < (uint32_t)K) ? row + 2 * k : kPastEnd;
    };
    // tiles past the last one lie beyond the weights as well
    const uint32_t w_tile = (uint32_t)tile * (uint32_t)K * 32u + (uint32_t)lane * 16u;
    auto woffs = [&](int st) -> uint32_t {
        return st < s_end ? w_tile + ((uint32_t)st << 10) : kPastEnd;
    };
    // Each weight load reads 1 KiB of contiguous memory once: the
    // non-temporal hint (cache policy bit 1) measured 9-11 % faster
    // (K = 2560, N = 16384 / 31040 / 248320, M = 1 and 5).
    constexpr int kWPolicy = 2;
    uint4 wv[kRing], av[kRing];
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
        wv[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wres, (int)woffs(s_begin + r), 0, kWPolicy));
        av[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, (int)offs(s_begin + r, a_row), 0, 0));
        __builtin_amdgcn_sched_barrier(0);  // issue in ring order
    }
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int s = s_begin; s < s_end; s += kRing) {
#pragma unroll
        for (int r = 0; r < kRing; ++r) {
            acc = mfma_step<AT>(av[r], wv[r], acc);
            const int nx = s + r + kRing;
            wv[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wres, (int)woffs(nx), 0, kWPolicy));
            av[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, (int)offs(nx, a_row), 0, 0));
            // keep each refill right after the MFMA that frees its registers,
            // so every step waits only for loads issued kRing steps earlier
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (ksplit > 1) {
        red[wave][lane] = acc;
        __syncthreads();
        if (kpart != 0) return;
        for (int p = 1; p < ksplit; ++p) {
            const floatx4 o = red[wave + p][lane];
            acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
        }
    }
    if (n0 + j >= N) return;
    const float b = bias ? load_elem(bias, n0 + j, c_dt) : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tok = g * 4 + r;
        if (tok < M) store_elem(C, (size_t)tok * N + n0 + j, acc[r] + b, c_dt);
    }
}

// Row-major weights staged through LDS, for M <= 16.  The operand layout
// wants 16 rows x 64 bytes per load instruction, which reads each 128-byte
// line in two halves from two instructions; here every load instruction
// reads whole 512-byte runs of two rows instead (lane l of load i takes 16
// bytes of chunk row 2i + l / 32 at 16 (l % 32)), the wave writes them into
// its own LDS region and reads them back in operand order.  A chunk is
// kChunk = 8 steps of 32 k: 16 rows x 512 bytes, 8 KiB, one chunk of loads
// in flight per wave.  Piece p (16 bytes) of chunk row r sits in slot
// 32 r + (p & 16) + ((p + r) & 15): the 16 lanes of a load that share a row,
// and the 16 lanes of an operand read that share a piece, fall in 16
// different 16-byte bank groups.  Each weight byte is read once, whole lines
// at a time, so the loads carry the non-temporal hint.  Every lane ends with
// the same operands in the same MFMA order as bf16_stream_kernel (steps past
// the wave's part included, with zero operands), so the results are
// bit-identical to it and to the tile-layout call.
constexpr int kChunk = 8;

template <int AT>
__global__ __launch_bounds__(kThreads) void bf16_rows_lds_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W,
    const void *__restrict__ bias, int M, int N, int K, int ksplit,
    void *__restrict__ C, int c_dt) {
    constexpr int PPR = 4 * kChunk;  // 16-byte pieces per chunk row
    __shared__ uint4 stage[kWaves][16 * PPR];
    __shared__ floatx4 red[kWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tiles_per_block = kWaves / ksplit;
    const int tile = blockIdx.x * tiles_per_block + wave / ksplit;
    const int kpart = wave % ksplit;
    const int n0 = tile * 16;
    const int j = lane & 15;
    const int g = lane >> 4;

    const int steps = (K + 31) >> 5;
    const int s_begin = (kpart * steps) / ksplit;
    const int s_end = ((kpart + 1) * steps) / ksplit;
    const int nch = (s_end - s_begin + kChunk - 1) / kChunk;

    const __amdgpu_buffer_rsrc_t wres = make_rsrc(W, (uint32_t)N * (uint32_t)K * 2);
    const __amdgpu_buffer_rsrc_t ares = make_rsrc(A, (uint32_t)M * (uint32_t)K * 2);
    // Loads: lane l of load i reads piece lp = l % 32 of chunk row 2i + l / 32
    // (rows past N lie beyond the buffer and read zeros).
    const int lp = lane & 31, lr = lane >> 5;
    const uint32_t w_lane = (uint32_t)(n0 + lr) * (uint32_t)K * 2 + 16u * (uint32_t)lp;
    const uint32_t w_load_step = 2u * (uint32_t)K * 2;  // two rows per load
    // Chunk c of the wave's part: the lane's offset for load 0, or past the
    // end when its step lies past the part or its k past K.  Past the end
    // plus up to 7 row pairs stays past the end and below 2^32 (callers keep
    // 16 rows of K below 2^31 bytes).
    auto w_off = [&](int c) -> uint32_t {
        const int st0 = s_begin + c * kChunk;
        const uint32_t k = (uint32_t)st0 * 32u + 8u * (uint32_t)lp;
        return (st0 + (lp >> 2) < s_end && k < (uint32_t)K) ? w_lane + 2u * (uint32_t)st0 * 32u
                                                           : kPastEnd;
    };
    // Activations of step st: token j's 8 values at k = 32 st + 8 g.
    const uint32_t a_row = (uint32_t)j * (uint32_t)K * 2;
    auto a_off = [&](int st) -> uint32_t {
        const uint32_t k = (uint32_t)(st << 5) + (uint32_t)(g << 3);
        return (st < s_end && k < (uint32_t)K) ? a_row + 2 * k : kPastEnd;
    };
    uint4 *my = stage[wave];
    auto slot = [](int r, int p) { return r * PPR + (p & 16) + ((p + r) & 15); };

    uint4 wv[kChunk], av[kChunk];
    auto load_w = [&](int c) {
        const uint32_t o = w_off(c);
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
            wv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                wres, (int)(o + (uint32_t)i * w_load_step), 0, 2));
    };
    load_w(0);
#pragma unroll
    for (int s = 0; s < kChunk; ++s)
        av[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, (int)a_off(s_begin + s), 0, 0));
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nch; ++c) {
        // LDS operations of one wave run in order: these writes follow the
        // previous chunk's reads, and the reads below see these writes.
#pragma unroll
        for (int i = 0; i < kChunk; ++i) my[slot(2 * i + lr, lp)] = wv[i];
        load_w(c + 1);
        // each step's activation registers are refilled for the next chunk
        // right after the MFMA that reads them
#pragma unroll
        for (int s = 0; s < kChunk; ++s) {
            acc = mfma_step<AT>(av[s], my[slot(j, 4 * s + g)], acc);
            av[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                ares, (int)a_off(s_begin + (c + 1) * kChunk + s), 0, 0));
        }
    }

    if (ksplit > 1) {
        red[wave][lane] = acc;
        __syncthreads();
        if (kpart != 0) return;
        for (int p = 1; p < ksplit; ++p) {
            const floatx4 o = red[wave + p][lane];
            acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
        }
    }
    if (n0 + j >= N) return;
    const float b = bias ? load_elem(bias, n0 + j, c_dt) : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tok = g * 4 + r;
        if (tok < M) store_elem(C, (size_t)tok * N + n0 + j, acc[r] + b, c_dt);
    }
}

template <int AT, int MT>
__global__ __launch_bounds__(kThreads) void bf16_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W,
    const void *__restrict__ bias, int M, int N, int K, int ksplit,
    void *__restrict__ C, int c_dt) {
    __shared__ floatx4 red[kWaves][MT][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tiles_per_block = kWaves / ksplit;
    const int tile = blockIdx.x * tiles_per_block + wave / ksplit;
    const int kpart = wave % ksplit;
    const int n0 = tile * 16;
    const int j = lane & 15;
    const int g = lane >> 4;
    const int n = (n0 + j < N) ? n0 + j : N - 1;  // clamped rows are computed and discarded

    const int steps = (K + 31) >> 5;
    const int s_begin = (kpart * steps) / ksplit;
    const int s_end = ((kpart + 1) * steps) / ksplit;

    floatx4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

    const uint16_t *wrow = W + (size_t)n * K;
    const uint4 zero = make_uint4(0, 0, 0, 0);

    for (int s = s_begin; s < s_end; ++s) {
        const int k = (s << 5) + (g << 3);
        const bool kin = k < K;  // K % 8 == 0: a lane's 8 values are all in or all out
        const uint4 wv = kin ? ld128(wrow + k) : zero;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int tok = t * 16 + j;
            const uint4 av = (kin && tok < M) ? ld128(A + (size_t)tok * K + k) : zero;
            if constexpr (AT == kF16) {
                const uint2 x = f16x2_to_bf16_hilo(av.x), y = f16x2_to_bf16_hilo(av.y);
                const uint2 z = f16x2_to_bf16_hilo(av.z), w = f16x2_to_bf16_hilo(av.w);
                acc[t] = mfma_bf16_16x16x32(as_bf16x8(make_uint4(x.x, y.x, z.x, w.x)), as_bf16x8(wv), acc[t]);
                acc[t] = mfma_bf16_16x16x32(as_bf16x8(make_uint4(x.y, y.y, z.y, w.y)), as_bf16x8(wv), acc[t]);
            } else {
                acc[t] = mfma_bf16_16x16x32(as_bf16x8(av), as_bf16x8(wv), acc[t]);
            }
        }
    }

    if (ksplit > 1) {
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
        __syncthreads();
        if (kpart != 0) return;
        for (int p = 1; p < ksplit; ++p)
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const floatx4 o = red[wave + p][t][lane];
                acc[t][0] += o[0]; acc[t][1] += o[1]; acc[t][2] += o[2]; acc[t][3] += o[3];
            }
    }

    if (n0 + j >= N) return;
    const float b = bias ? load_elem(bias, n0 + j, c_dt) : 0.f;
    // D layout: lane holds feature j and tokens 4*g + r of each 16-token tile.
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = t * 16 + g * 4 + r;
            if (tok < M) store_elem(C, (size_t)tok * N + n0 + j, acc[t][r] + b, c_dt);
        }
}

template <int AT, int MT>
hipError_t launch_mt(const uint16_t *A, const uint16_t *W, const void *bias, int M, int N,
                     int K, void *C, int c_dt, int wl, hipStream_t s) {
    const int tiles = (N + 15) / 16;
    const DeviceInfo info = device_info();
    // Split K across the waves of a workgroup when there are too few feature
    // tiles to give every SIMD of the chip a few waves.
    int ksplit = 1;
    if (tiles < info.num_cus * 8) ksplit = 2;
    if (tiles < info.num_cus * 2) ksplit = 4;
    const int tiles_per_block = kWaves / ksplit;
    const int blocks = (tiles + tiles_per_block - 1) / tiles_per_block;
    // The streaming kernel's offsets are 32-bit: weights (plus one tile of
    // rows past N) and 16 rows of activations must stay below 4 GiB.
    const bool stream = MT == 1 && ((uint64_t)N + 16) * (uint64_t)K * 2 < (1ull << 31) &&
                        16ull * (uint64_t)K * 2 < (1ull << 31);
    if (wl) {
        // the tile layout is read by the streaming kernel only
        if (AT != kBf16 || !stream || N % 16 != 0 || K % 32 != 0) return hipErrorInvalidValue;
        bf16_stream_kernel<kBf16><<<dim3(blocks), dim3(kThreads), 0, s>>>(A, W, bias, M, N, K,
                                                                             ksplit, C, c_dt);
    } else if (stream)
        bf16_rows_lds_kernel<AT><<<dim3(blocks), dim3(kThreads), 0, s>>>(A, W, bias, M, N, K,
                                                                            ksplit, C, c_dt);
    else
        bf16_gemm_kernel<AT, MT><<<dim3(blocks), dim3(kThreads), 0, s>>>(A, W, bias, M, N, K,
                                                                         ksplit, C, c_dt);
    return hipGetLastError();
}

template <int AT>
hipError_t launch_slabs(const uint16_t *A, const uint16_t *W, const void *bias, int M, int N,
                        int K, void *C, int c_dt, int wl, hipStream_t s) {
    // Token tiles of 16; above 64 tokens the weight is streamed once per
    // 64-token slab.
    const size_t c_size = c_dt == kF32 ? 4 : 2;
    for (int m0 = 0; m0 < M; m0 += 64) {
        const int mm = (M - m0) < 64 ? (M - m0) : 64;
        const uint16_t *Am = A + (size_t)m0 * K;
        void *Cm = static_cast<char *>(C) + (size_t)m0 * N * c_size;
        hipError_t e;
        if (mm <= 16) e = launch_mt<AT, 1>(Am, W, bias, mm, N, K, Cm, c_dt, wl, s);
        else if (wl) e = hipErrorInvalidValue;
        else if (mm <= 32) e = launch_mt<AT, 2>(Am, W, bias, mm, N, K, Cm, c_dt, 0, s);
        else e = launch_mt<AT, 4>(Am, W, bias, mm, N, K, Cm, c_dt, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_bf16_gemm(const void *A, int a_dt, const uint16_t *W, const void *bias, int M,
                            int N, int K, void *C, int c_dt, hipStream_t s, int wl) {
    const uint16_t *A16 = static_cast<const uint16_t *>(A);
    if (a_dt == kF16) return launch_slabs<kF16>(A16, W, bias, M, N, K, C, c_dt, wl, s);
    return launch_slabs<kBf16>(A16, W, bias, M, N, K, C, c_dt, wl, s);
}

bool bf16_tiles_fit(int N, int K) {
    // the streaming kernel's offsets: every tile of the grid (up to 3 past
    // the last) and 16 activation rows below 2 GiB
    return ((uint64_t)N + 64) * (uint64_t)K * 2 < (1ull << 31) &&
           16ull * (uint64_t)K * 2 < (1ull << 31);
}

}  // namespace q4
