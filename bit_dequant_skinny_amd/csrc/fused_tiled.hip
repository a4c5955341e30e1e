// Fused 4-bit dequantize + GEMM on the matrix cores for tens to hundreds of
// token rows: C[M,N] = A[M,K] * dequant(W)^T (+ bias), bf16 activations,
// blocksize >= 64.
//
// The bitsandbytes pull request "[ROCm] Optimize kgemm_4bit_inference_naive
// for ROCm, use it for batch sizes other than 1" finds (section "Fused path
// support for M > 1" and the review discussion) that a fused kernel which
// streams the packed weights once per few token rows falls behind
// dequantize-then-GEMM as M grows, and that matrix-core (MMA) fused kernels
// keep the fused path ahead at M = 32..128 and beyond.  This kernel is that
// variant for CDNA4: output tiles of 64 (or 32) tokens x 64 features reuse
// every decoded weight for all the tile's tokens, so the packed weights are
// read once per token block rather than once per 16 or 32 rows.
//
// Decode.  A 256-entry LDS table maps one packed byte to the bf16 hi and lo
// parts of its two codebook values (hi = bf16(cb), lo = bf16(cb - hi), so
// hi + lo is the fp32 value to within 2^-18 relative), 32 copies of each so
// that the lookups of a half-wave never share a bank.  Four lookups give the
// hi parts of a dword's 8 codes and four more the lo parts: two B operands of
// v_mfma_f32_16x16x32_bf16 against the same 8 activations as loaded, so the
// matrix core forms a*hi + a*lo in fp32.  The sum over each 64-wide block is
// kept apart and scaled by the block's absmax once (acc = fma(absmax, block
// sum, acc)).
//
// Work split.  A workgroup of 4 waves owns one output tile and one part of K
// (the whole K unless K is split over workgroups to fill the CUs).  The K
// range is walked in 128-wide segments, wave w taking segments w, w+4, ...,
// so the 4 waves read 256 contiguous bytes of each weight row at a time.
// Each wave computes the whole tile over its segments: per segment a lane
// loads 16 packed bytes of one feature row for each of the tile's 4 feature
// blocks (one v_permlane32_swap pair regroups them by 64-wide block) and the
// matching 16-byte activation pieces of each token block, two segments ahead
// of use; the A and W loads are buffer loads, whose range check returns zeros
// for rows past M or N and for k past K (K % 128 == 64 leaves half a
// segment), and a zero activation cancels whatever codes sit there.  At the
// end the 4 waves' fp32 tiles meet in LDS (over the decode table) and are
// summed in wave order, so results are deterministic.
//
// Placement.  Workgroups are dispatched to the 8 XCDs round-robin by index;
// the token blocks of one feature block get indices 8 apart, so they run on
// one XCD and the second reads the packed weights from that XCD's L2.
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

constexpr int kWaves = 4;
constexpr int kTileN = 64;                 // features per tile (4 MFMA columns blocks)
constexpr uint32_t kPastEnd = 0x80000000u;  // an offset beyond every buffer: reads zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// One segment's weights for one wave: 16 packed bytes per feature block and
// the absmax of both 64-wide halves per feature block.
struct SegW {
    uint4 w[4];
    float s[4][2];
};

// TM: 16-row token blocks per tile (2 or 4).
template <int TM>
__global__ __launch_bounds__(64 * kWaves) void fused_tiled_kernel(
    const uint16_t *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ absmax, const float *__restrict__ codebook,
    const void *__restrict__ bias, int M, int N, int K, int bs_log2, int m_blocks,
    int n_blocks, int n_groups, int segs_per_part, void *__restrict__ C, int c_dt) {
    // Entry e (a packed byte) fills bytes [256 e, 256 e + 256): 32 copies of
    // its hi pair, then 32 copies of its lo pair; lane l reads copy l % 32.
    // Afterwards the same memory holds the waves' partial tiles.
    __shared__ uint32_t table[256 * 64];
    static_assert(kWaves * TM * 4 * 64 * 16 <= (int)sizeof(table), "partial tiles fit the table");

    // Block b of a part: XCD slot b % 8, row r = b / 8; token block r %
    // m_blocks, feature block (r / m_blocks) * 8 + b % 8.  Parts (K splits)
    // follow one another.
    const uint32_t per_part = 8u * (uint32_t)m_blocks * (uint32_t)n_groups;
    const int part = (int)(blockIdx.x / per_part);
    const uint32_t q = blockIdx.x % per_part;
    const uint32_t r = q >> 3;
    const int mb = (int)(r % (uint32_t)m_blocks);
    const int nb_i = (int)(r / (uint32_t)m_blocks) * 8 + (int)(q & 7u);
    if (nb_i >= n_blocks) return;  // uniform over the workgroup
    const int m0 = mb * 16 * TM, n0 = nb_i * kTileN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
    const int j = lane & 15, g = lane >> 4;
    const char *tab = reinterpret_cast<const char *>(table);
    const uint32_t lane_off = (uint32_t)(lane & 31) * 4;  // hi copies
    const uint32_t lane_off_lo = lane_off + 128;          // lo copies

    const int nseg = (K + 127) >> 7;
    const int s_begin = part * segs_per_part;
    const int s_end = min(nseg, s_begin + segs_per_part);
    // segments of this wave: s_begin + wave + 4 i, i < my
    const int my = s_end - s_begin > wave ? (s_end - s_begin - wave + kWaves - 1) / kWaves : 0;

    const uint32_t row_bytes = (uint32_t)K >> 1;
    const uint32_t nbk = (uint32_t)K >> bs_log2;  // blocks per row
    // Per-lane byte offsets, fixed for the whole walk: rows past N or M
    // take an offset beyond every buffer.  Each segment then views the
    // buffers through a resource whose base is moved to the segment (scalar
    // work): a load reads zeros when its offset falls past the end of the
    // buffer, and a whole resource is emptied for a segment past the wave's
    // last or a half segment past K.
    uint32_t w_off[4], s_off[4], a_off[TM][4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t n = (uint32_t)(n0 + 16 * b + j);
        w_off[b] = n < (uint32_t)N ? n * row_bytes + 16 * (uint32_t)g : kPastEnd;
        s_off[b] = n < (uint32_t)N ? n * nbk * 4 : kPastEnd;
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const uint32_t m = (uint32_t)(m0 + 16 * t + j);
#pragma unroll
        for (int p = 0; p < 4; ++p)
            a_off[t][p] = m < (uint32_t)M ? (m * (uint32_t)K + swapped_k_offset(g, p)) * 2 : kPastEnd;
    }
    // (The start and size are wave-uniform; readfirstlane keeps them in
    // scalar registers, so the resource needs no per-lane handling.)
    auto window = [](const void *base, uint32_t bytes, uint32_t start, bool live) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(start);
        const uint32_t nr = __builtin_amdgcn_readfirstlane(live && start < bytes ? bytes - start : 0u);
        return make_rsrc(static_cast<const char *>(base) + st, nr);
    };
    const uint32_t w_bytes = (uint32_t)N * row_bytes, s_bytes = (uint32_t)N * nbk * 4;
    const uint32_t a_bytes = (uint32_t)M * (uint32_t)K * 2;

    auto load_w = [&](int i, SegW &d) {
        const bool live = i < my;
        const uint32_t seg = (uint32_t)(s_begin + wave + kWaves * i);
        const __amdgpu_buffer_rsrc_t wr = window(Wp, w_bytes, seg * 64, live);
#pragma unroll
        for (int b = 0; b < 4; ++b)
            d.w[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, (int)w_off[b], 0, 0));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t k = seg * 128 + 64 * h;
            const __amdgpu_buffer_rsrc_t sr =
                window(absmax, s_bytes, (k >> bs_log2) * 4, live && k < (uint32_t)K);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                d.s[b][h] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, (int)s_off[b], 0, 0));
        }
    };
    // Activations: the 8 values of each of the lane's 4 code dwords per token
    // block, single-buffered: each half (dwords 2h, 2h+1) is reloaded for the
    // wave's next segment as soon as the MFMAs of this segment's half are
    // issued, a half segment ahead of use.
    uint4 a[TM][4];
    auto load_a = [&](int i, int h) {
        const uint32_t k = (uint32_t)(s_begin + wave + kWaves * i) * 128 + 64 * h;
        const __amdgpu_buffer_rsrc_t ar = window(A, a_bytes, (k - 64 * h) * 2, i < my && k < (uint32_t)K);
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
                a[t][2 * h + pp] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(ar, (int)a_off[t][2 * h + pp], 0, 0));
    };

    floatx4 acc[TM][4];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[t][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Segment i (this wave's i-th) from weights d; reloads the activations
    // for segment i + 1.
    // The 8 blocks of a segment (block q = 4h + b: 64-wide half h of
    // feature block b) each take two steps g = 2q, 2q + 1 (dword p = 2h + g %
    // 2).  Software pipeline, fixed by scheduling barriers: the table reads
    // of step g + 1 are issued before the MFMAs of step g, and the absmax
    // scaling of block q waits until the MFMAs of block q + 1 are issued, so
    // neither the LDS latency nor the MFMA latency stalls the wave.
    auto lookup = [&](const SegW &d, int g, uint4 &bh, uint4 &bl) {
        const int q = g >> 1, p = 2 * (q >> 2) + (g & 1);
        const uint4 &w = d.w[q & 3];
        const uint32_t x = p == 0 ? w.x : p == 1 ? w.y : p == 2 ? w.z : w.w;
        uint32_t vh[4], vl[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // byte c of the dword * 256 + the lane's copy; the lo address is
            // formed separately so the two reads stay single-dword loads into
            // their operand registers
            const uint32_t sel = 0x0c0c0000u | ((4u + c) << 8);
            vh[c] = *reinterpret_cast<const uint32_t *>(tab + __builtin_amdgcn_perm(x, lane_off, sel));
            vl[c] = *reinterpret_cast<const uint32_t *>(tab + __builtin_amdgcn_perm(x, lane_off_lo, sel));
        }
        bh = make_uint4(vh[0], vh[1], vh[2], vh[3]);
        bl = make_uint4(vl[0], vl[1], vl[2], vl[3]);
    };
    auto mfmas = [&](int g, const uint4 &bh, const uint4 &bl, floatx4 (&blk)[TM]) {
        const int p = 2 * (g >> 3) + (g & 1);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const floatx4 c = (g & 1) == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : blk[t];
            blk[t] = mfma_bf16_16x16x32(as_bf16x8(a[t][p]), as_bf16x8(bh), c);
            blk[t] = mfma_bf16_16x16x32(as_bf16x8(a[t][p]), as_bf16x8(bl), blk[t]);
        }
    };
    auto scale = [&](const SegW &d, int q, const floatx4 (&blk)[TM]) {
        const int h = q >> 2, b = q & 3;
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                acc[t][b][rr] = __builtin_fmaf(d.s[b][h], blk[t][rr], acc[t][b][rr]);
    };

    // Segment i (this wave's i-th) from weights d; reloads the activations
    // for segment i + 1, each half once its last MFMAs are issued.
    auto compute_seg = [&](int i, SegW &d) {
#pragma unroll
        for (int b = 0; b < 4; ++b) permlane32_swap_dwords(d.w[b]);
        uint4 bh[2], bl[2];
        floatx4 blk[2][TM];  // block sums of blocks q (even / odd)
        lookup(d, 0, bh[0], bl[0]);
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            if (g + 1 < 16) lookup(d, g + 1, bh[(g + 1) & 1], bl[(g + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(g, bh[g & 1], bl[g & 1], blk[(g >> 1) & 1]);
            if ((g & 1) && g >= 3) scale(d, (g >> 1) - 1, blk[((g >> 1) - 1) & 1]);
            if (g == 7) load_a(i + 1, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        scale(d, 7, blk[1]);
        load_a(i + 1, 1);
    };

    // Prologue: the first segment's activations and two segments' weights,
    // then the table (its codebook loads complete after those, in issue order).
    SegW s0, s1;
    load_a(0, 0);
    load_a(0, 1);
    load_w(0, s0);
    load_w(1, s1);
    {
        const float c0 = codebook[tid & 15], c1 = codebook[tid >> 4];
        const uint2 v = pair_table_entry(c0, c1);
        // Thread t writes the copies of entry t starting at copy t % 32: the
        // 32 lanes of a half-wave write 32 different banks.
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            table[tid * 64 + ((tid + c) & 31)] = v.x;
            table[tid * 64 + 32 + ((tid + c) & 31)] = v.y;
        }
    }
    __syncthreads();

    // Two segments per iteration (ring entries 0 and 1), then a last odd
    // segment.  Every load issued in the loop is consumed both by the next
    // iteration and by the tail, so none is sunk next to its use.
    int i = 0;
    for (; i + 2 <= my; i += 2) {
        compute_seg(i, s0);
        load_w(i + 2, s0);
        compute_seg(i + 1, s1);
        load_w(i + 3, s1);
    }
    if (i < my) compute_seg(i, s0);

    // Cross-wave sum through LDS over the table: red[wave][t][b][lane] float4.
    __syncthreads();
    floatx4 *red = reinterpret_cast<floatx4 *>(table);
    constexpr int kPer = TM * 4 * 64;  // float4 per wave
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int b = 0; b < 4; ++b) red[wave * kPer + (t * 4 + b) * 64 + lane] = acc[t][b];
    __syncthreads();

    const bool partial = gridDim.x > per_part;  // K split: fp32 partial slabs, no bias
    if (partial) C = static_cast<char *>(C) + (size_t)part * (size_t)M * (size_t)N * 4;
#pragma unroll
    for (int u = 0; u < kPer / 256; ++u) {
        const int v = tid + 256 * u;
        floatx4 sum = red[v];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) sum += red[w * kPer + v];
        const int tb = v >> 6, l = v & 63;
        const int n = n0 + 16 * (tb & 3) + (l & 15);
        if (n >= N) continue;
        const float bv = bias && !partial ? load_elem(bias, n, c_dt) : 0.f;
        const int mrow = m0 + 16 * (tb >> 2) + 4 * (l >> 4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int m = mrow + rr;
            if (m < M) store_elem(C, (size_t)m * N + n, sum[rr] + bv, partial ? kF32 : c_dt);
        }
    }
}

int tile_rows(int M) { return M > 32 ? 64 : 32; }

}  // namespace

// 32-bit byte offsets: A, the packed weights and the scales each stay below 2 GiB.
bool q4_fused_tiled_fits(int M, int N, int K) {
    return (uint64_t)M * (uint64_t)K * 2 < (1ull << 31) &&
           (uint64_t)N * (uint64_t)K / 2 < (1ull << 31) &&
           (uint64_t)N * (uint64_t)K / 16 < (1ull << 31);
}

// Parts of K: enough workgroups to give every CU one, keeping at least 8
// segments (two per wave) per part, at most 4 parts.
int q4_fused_tiled_ksplit(int M, int N, int K) {
    const int bm = tile_rows(M);
    const int tiles = ((M + bm - 1) / bm) * ((N + kTileN - 1) / kTileN);
    const int nseg = (K + 127) / 128;
    const int cus = device_info().num_cus;
    int ks = 1;
    while (ks < 4 && tiles * ks < cus && nseg / (ks + 1) >= 8) ++ks;
    return ks;
}

hipError_t launch_q4_fused_tiled(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                                 const float *codebook, const void *bias, int M, int N, int K,
                                 int bs_log2, int ksplit, void *C, int c_dt, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    if (bs_log2 < 6 || ksplit < 1 || (ksplit > 1 && (bias || c_dt != kF32)))
        return hipErrorInvalidValue;
    const int bm = tile_rows(M);
    const int m_blocks = (M + bm - 1) / bm;
    const int n_blocks = (N + kTileN - 1) / kTileN;
    const int n_groups = (n_blocks + 7) / 8;
    const int nseg = (K + 127) / 128;
    const int spp = ((nseg + ksplit - 1) / ksplit + kWaves - 1) / kWaves * kWaves;
    const unsigned grid = (unsigned)(8 * m_blocks * n_groups * ksplit);
    if (bm == 64)
        fused_tiled_kernel<4><<<dim3(grid), dim3(64 * kWaves), 0, s>>>(
            A, Wpacked, absmax, codebook, bias, M, N, K, bs_log2, m_blocks, n_blocks, n_groups,
            spp, C, c_dt);
    else
        fused_tiled_kernel<2><<<dim3(grid), dim3(64 * kWaves), 0, s>>>(
            A, Wpacked, absmax, codebook, bias, M, N, K, bs_log2, m_blocks, n_blocks, n_groups,
            spp, C, c_dt);
    return hipGetLastError();
}

}  // namespace q4
