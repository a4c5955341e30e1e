// Fused 4-bit dequantize + GEMM on the matrix cores for tens to hundreds of
// token rows: C[M,N] = A[M,K] * dequant(W)^T (+ bias), bf16 activations,
// blocksize >= 64.  The packed weights are row-major or in the tile layout
// (wl = 1: 16-row tiles of 1 KiB units); a lane gets the same 16 bytes
// either way: one 128-bit load over rows, two 64-bit loads 512 bytes apart
// over tiles (which hold a row's 16 bytes as two halves in different pieces).
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
// hi + lo is the fp32 value to within 2^-16 relative), 32 copies of each so
// that the lookups of a half-wave never share a bank.  Four lookups give the
// hi parts of a dword's 8 codes and four more the lo parts: two B operands of
// v_mfma_f32_16x16x32_bf16 against the same 8 activations as loaded, so the
// matrix core forms a*hi + a*lo in fp32.  The sum over each 64-wide block is
// kept apart and scaled by the block's absmax once (acc = fma(absmax, block
// sum, acc)).
//
// Two work layouts, chosen per shape by q4_fused_tiled_plan:
//
// Waves split K (64-feature tiles, for shapes with few tiles).  A workgroup
// of 4 waves owns an output tile of 64 (or 32) tokens x 64 features and one
// part of K; the part's 128-wide segments go to the waves in turn (wave w:
// w, w+4, ...), so they read 256 contiguous bytes of each weight row at a
// time, and each wave computes the whole tile over its segments, reading its
// activations from L2.  At the end the 4 waves' fp32 tiles meet in LDS (over
// the decode table) and are summed in wave order.
//
// Waves split N (256-feature tiles, for shapes with many tiles).  A
// workgroup of 8 waves owns 64 (or 32) tokens x 256 features, each wave 32
// features, all waves walking the same segments: each segment's activations
// are staged once through LDS (double-buffered, one barrier per segment)
// and read by all 8 waves, a quarter of the L2 traffic per MFMA of the other
// layout, and no cross-wave sum.
//
// In both, K may also be split over workgroups (up to 4 parts) when the
// tiles cannot fill the GPU; the parts' fp32 partial tiles are summed in
// part order by a separate pass.  A lane loads 16 packed bytes of one
// feature row per segment (one v_permlane32_swap pair regroups them by
// 64-wide block) two segments ahead of use; the loads go through buffer
// resources moved to each segment, whose range check returns zeros for rows
// past M or N, for a half segment past K (K % 128 == 64) and for segments
// past a wave's last, so a zero activation cancels whatever codes sit there.
//
// Placement.  Workgroups are dispatched to the 8 XCDs round-robin by index;
// the token blocks of one feature block run on one XCD, so the later ones
// read the packed weights from that XCD's L2 (tile_of_strided and
// tile_of_balanced below).
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

constexpr int kWaves = 4;                  // waves per workgroup, K-split layout
constexpr int kTileN = 64;                 // features per tile, K-split layout
constexpr int kWavesN = 8;                 // waves per workgroup, N-split layout
constexpr int kTN = 2;                     // 16-feature blocks per wave, N-split layout
constexpr int kTileNN = kWavesN * kTN * 16;  // features per tile, N-split layout
constexpr int kRowU4 = 17;                 // staged activation row: 256 B + 16 B pad, in uint4
constexpr uint32_t kPastEnd = 0x80000000u;  // an offset beyond every buffer: reads zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// A buffer viewed from byte `start` on (empty unless `live`).  The start and
// size are wave-uniform; readfirstlane keeps them in scalar registers, so the
// resource needs no per-lane handling.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const void *base, uint32_t bytes,
                                                         uint32_t start, bool live) {
    const uint32_t st = __builtin_amdgcn_readfirstlane(start);
    const uint32_t nr = __builtin_amdgcn_readfirstlane(live && start < bytes ? bytes - start : 0u);
    return make_rsrc(static_cast<const char *>(base) + st, nr);
}

// The 16 bytes lane (j, g) decodes per segment: bytes 16g..16g+15 of its
// row's segment.  Over tiles those are two 8-byte halves 512 bytes apart
// (the tile layout holds 8 bytes of each 64-wide half of a row's segment per
// piece: the first half of the lane's bytes sits at 16j + 256 (g % 2) +
// 8 (g / 2) of the unit, the second 512 bytes further), so each of the two
// loads still reads 512 contiguous bytes over the wave.
__device__ __forceinline__ uint32_t tile_lane_offset(int lane) {
    const int j = lane & 15, g = lane >> 4;
    return 16u * (uint32_t)j + 256u * (uint32_t)(g & 1) + 8u * (uint32_t)(g >> 1);
}

template <int WL>
__device__ __forceinline__ uint4 load_piece(__amdgpu_buffer_rsrc_t wr, uint32_t off) {
    if constexpr (WL == 1) {
        const auto h0 = __builtin_amdgcn_raw_buffer_load_b64(wr, (int)off, 0, 0);
        const auto h1 = __builtin_amdgcn_raw_buffer_load_b64(wr, (int)(off + 512u), 0, 0);
        return make_uint4(h0[0], h0[1], h1[0], h1[1]);
    }
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, (int)off, 0, 0));
}

// The tile of workgroup b.  The hardware deals workgroups to the 8 XCDs
// round-robin (b % 8).  In both mappings the token blocks of a feature
// block run on one XCD, where the later ones read the packed weights from
// its L2.
struct TileIdx {
    int part, nb, mb;
    bool live;
};
// K-split layout (many 64-feature tiles): feature block f runs on XCD f % 8;
// a part holds 8 * m_blocks * ceil(n_blocks / 8) workgroups (those past the
// last feature block exit at once), and the parts follow one another, so
// the workgroups of an XCD walk different rows at different k.  (A
// contiguous run of tiles per XCD measured 20 % slower at 5120 x 5120,
// M = 64.)
__device__ __forceinline__ TileIdx tile_of_strided(uint32_t b, int m_blocks, int n_blocks) {
    const uint32_t groups = ((uint32_t)n_blocks + 7u) / 8u;
    const uint32_t per_part = 8u * (uint32_t)m_blocks * groups;
    const uint32_t q = b % per_part, r = q >> 3;
    TileIdx t;
    t.part = (int)(b / per_part);
    t.mb = (int)(r % (uint32_t)m_blocks);
    t.nb = (int)(r / (uint32_t)m_blocks) * 8 + (int)(q & 7u);
    t.live = t.nb < n_blocks;
    return t;
}
// N-split layout (few 256-feature tiles): the grid holds 8 * per_xcd
// workgroups and XCD x takes the consecutive tiles x * per_xcd, ... in the
// order K part (fastest), token block, feature block, so every XCD gets the
// same number of tiles to within one (with the mapping above, tile counts
// that are not a multiple of 8 left some XCDs a second round: 5120 x 5120 at
// M = 192 took 70 us, 41 us balanced).
__device__ __forceinline__ TileIdx tile_of_balanced(uint32_t b, int m_blocks, int n_blocks,
                                                    int ksplit, uint32_t per_xcd) {
    const uint32_t L = (b & 7u) * per_xcd + (b >> 3);
    TileIdx t;
    t.live = L < (uint32_t)m_blocks * (uint32_t)n_blocks * (uint32_t)ksplit;
    t.part = (int)(L % (uint32_t)ksplit);
    const uint32_t rem = L / (uint32_t)ksplit;
    t.mb = (int)(rem % (uint32_t)m_blocks);
    t.nb = (int)(rem / (uint32_t)m_blocks);
    return t;
}

// One segment's weights for one wave: 16 packed bytes per feature block and
// the absmax of both 64-wide halves per feature block.
struct SegW {
    uint4 w[4];
    float s[4][2];
};

// K-split layout.  TM: 16-row token blocks per tile (2 or 4).
template <int TM, int WL>
__global__ __launch_bounds__(64 * kWaves, 2) void fused_tiled_ks_kernel(
    const uint16_t *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ absmax, const float *__restrict__ codebook,
    const void *__restrict__ bias, int M, int N, int K, int bs_log2, int m_blocks,
    int n_blocks, int ksplit, int segs_per_part, void *__restrict__ C, int c_dt) {
    // Entry e (a packed byte) fills bytes [256 e, 256 e + 256): 32 copies of
    // its hi pair, then 32 copies of its lo pair; lane l reads copy l % 32.
    // Afterwards the same memory holds the waves' partial tiles.
    __shared__ uint32_t table[256 * 64];
    static_assert(kWaves * TM * 4 * 64 * 16 <= (int)sizeof(table), "partial tiles fit the table");

    const TileIdx ti = tile_of_strided(blockIdx.x, m_blocks, n_blocks);
    if (!ti.live) return;  // uniform over the workgroup
    const int part = ti.part, mb = ti.mb, nb_i = ti.nb;
    const int m0 = mb * 16 * TM, n0 = nb_i * kTileN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
    const int j = lane & 15, g = lane >> 4;
    const uint32_t tile_lane_off = tile_lane_offset(lane);
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
        w_off[b] = n >= (uint32_t)N ? kPastEnd
                   : WL ? (n - (uint32_t)j) * row_bytes + tile_lane_off
                        : n * row_bytes + 16 * (uint32_t)g;
        s_off[b] = n < (uint32_t)N ? n * nbk * 4 : kPastEnd;
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const uint32_t m = (uint32_t)(m0 + 16 * t + j);
#pragma unroll
        for (int p = 0; p < 4; ++p)
            a_off[t][p] = m < (uint32_t)M ? (m * (uint32_t)K + swapped_k_offset(g, p)) * 2 : kPastEnd;
    }
    const uint32_t w_bytes = (uint32_t)N * row_bytes, s_bytes = (uint32_t)N * nbk * 4;
    const int seg_sh = WL ? 10 : 6;  // segment -> byte offset (1 KiB units or 64-byte pieces)
    const uint32_t a_bytes = (uint32_t)M * (uint32_t)K * 2;

    auto load_w = [&](int i, SegW &d) {
        const bool live = i < my;
        const uint32_t seg = (uint32_t)(s_begin + wave + kWaves * i);
        const __amdgpu_buffer_rsrc_t wr = window(Wp, w_bytes, seg << seg_sh, live);
#pragma unroll
        for (int b = 0; b < 4; ++b)
            d.w[b] = load_piece<WL>(wr, w_off[b]);
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

    const bool partial = ksplit > 1;  // K split: fp32 partial slabs, no bias
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

// N-split layout: one segment's weights for one wave (its 2 feature blocks).
struct SegWN {
    uint4 w[kTN];
    float s[kTN][2];
};

// N-split layout.  TM: 16-row token blocks per tile (2 or 4).
template <int TM, int WL>
__global__ __launch_bounds__(64 * kWavesN) void fused_tiled_ns_kernel(
    const uint16_t *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ absmax, const float *__restrict__ codebook,
    const void *__restrict__ bias, int M, int N, int K, int bs_log2, int m_blocks,
    int n_blocks, int ksplit, uint32_t per_xcd, int segs_per_part, void *__restrict__ C,
    int c_dt) {
    __shared__ uint32_t table[256 * 64];                 // as in the K-split layout
    __shared__ uint4 astage[2][TM * 16 * kRowU4];        // the segment's activations, 2 buffers

    const TileIdx ti = tile_of_balanced(blockIdx.x, m_blocks, n_blocks, ksplit, per_xcd);
    if (!ti.live) return;  // uniform over the workgroup
    const int part = ti.part, mb = ti.mb, nb_i = ti.nb;
    const int m0 = mb * 16 * TM, n0 = nb_i * kTileNN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, g = lane >> 4;
    const uint32_t tile_lane_off = tile_lane_offset(lane);
    const char *tab = reinterpret_cast<const char *>(table);
    const uint32_t lane_off = (uint32_t)(lane & 31) * 4;  // hi copies
    const uint32_t lane_off_lo = lane_off + 128;          // lo copies

    const int nseg = (K + 127) >> 7;
    const int s_begin = part * segs_per_part;
    const int s_end = min(nseg, s_begin + segs_per_part);
    const int cnt = s_end > s_begin ? s_end - s_begin : 0;  // segments of this part

    const uint32_t row_bytes = (uint32_t)K >> 1;
    const uint32_t nbk = (uint32_t)K >> bs_log2;
    const uint32_t w_bytes = (uint32_t)N * row_bytes, s_bytes = (uint32_t)N * nbk * 4;
    const int seg_sh = WL ? 10 : 6;  // segment -> byte offset (1 KiB units or 64-byte pieces)
    const uint32_t a_bytes = (uint32_t)M * (uint32_t)K * 2;
    uint32_t w_off[kTN], s_off[kTN];
#pragma unroll
    for (int b = 0; b < kTN; ++b) {
        const uint32_t n = (uint32_t)(n0 + wave * 16 * kTN + 16 * b + j);
        w_off[b] = n >= (uint32_t)N ? kPastEnd
                   : WL ? (n - (uint32_t)j) * row_bytes + tile_lane_off
                        : n * row_bytes + 16 * (uint32_t)g;
        s_off[b] = n < (uint32_t)N ? n * nbk * 4 : kPastEnd;
    }
    // Activation staging: waves 0-3 move the first 64 k of each row of the
    // segment, waves 4-7 the second (one resource per half, so a half past K
    // reads zeros); per half, 256 threads move TM*16 rows x 8 pieces of 16
    // bytes, TM/2 pieces each.  LDS rows are 272 bytes apart, so the 16 rows
    // a quarter-wave reads with ds_read_b128 fall in distinct banks.
    constexpr int kPieces = TM / 2;
    const int sh = wave >> 2;
    uint32_t st_off[kPieces], st_lds[kPieces];
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
        const int idx = (wave & 3) * 64 + lane + 256 * u;
        const int row = idx >> 3, c = idx & 7;
        st_off[u] = (uint32_t)(m0 + row) * (uint32_t)K * 2 + (uint32_t)c * 16;
        st_lds[u] = (uint32_t)(row * kRowU4 + sh * 8 + c);
    }

    auto load_w = [&](int i, SegWN &d) {
        const bool live = i < cnt;
        const uint32_t seg = (uint32_t)(s_begin + i);
        const __amdgpu_buffer_rsrc_t wr = window(Wp, w_bytes, seg << seg_sh, live);
#pragma unroll
        for (int b = 0; b < kTN; ++b)
            d.w[b] = load_piece<WL>(wr, w_off[b]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t k = seg * 128 + 64 * h;
            const __amdgpu_buffer_rsrc_t sr =
                window(absmax, s_bytes, (k >> bs_log2) * 4, live && k < (uint32_t)K);
#pragma unroll
            for (int b = 0; b < kTN; ++b)
                d.s[b][h] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, (int)s_off[b], 0, 0));
        }
    };
    uint4 stv[kPieces];
    auto stage_load = [&](int i) {
        const uint32_t k = (uint32_t)(s_begin + i) * 128 + 64 * sh;
        const __amdgpu_buffer_rsrc_t ar = window(A, a_bytes, k * 2, i < cnt && k < (uint32_t)K);
#pragma unroll
        for (int u = 0; u < kPieces; ++u)
            stv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ar, (int)st_off[u], 0, 0));
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kPieces; ++u) astage[buf][st_lds[u]] = stv[u];
    };
    // LDS-only barrier: waits for this wave's LDS operations, not for its
    // global loads in flight, then synchronises the workgroup.
    auto lds_barrier = []() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    floatx4 acc[TM][kTN];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int b = 0; b < kTN; ++b) acc[t][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    // A segment is 8 steps g: half h = g >> 2, feature block b = (g >> 1) & 1,
    // dword p = 2h + g % 2; block q = g >> 1 collects two steps.  Pipelined
    // as in the K-split layout: table reads one step ahead, the absmax FMA of
    // block q after the MFMAs of block q + 1, the activation operands of the
    // second half read from LDS early in the first.
    auto lookup = [&](const SegWN &d, int gg, uint4 &bh, uint4 &bl) {
        const int p = 2 * (gg >> 2) + (gg & 1);
        const uint4 &w = d.w[(gg >> 1) & 1];
        const uint32_t x = p == 0 ? w.x : p == 1 ? w.y : p == 2 ? w.z : w.w;
        uint32_t vh[4], vl[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t sel = 0x0c0c0000u | ((4u + c) << 8);
            vh[c] = *reinterpret_cast<const uint32_t *>(tab + __builtin_amdgcn_perm(x, lane_off, sel));
            vl[c] = *reinterpret_cast<const uint32_t *>(tab + __builtin_amdgcn_perm(x, lane_off_lo, sel));
        }
        bh = make_uint4(vh[0], vh[1], vh[2], vh[3]);
        bl = make_uint4(vl[0], vl[1], vl[2], vl[3]);
    };
    auto scale = [&](const SegWN &d, int qq, const floatx4 (&blk)[TM]) {
        const int h = qq >> 1, b = qq & 1;
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                acc[t][b][rr] = __builtin_fmaf(d.s[b][h], blk[t][rr], acc[t][b][rr]);
    };
    auto load_ops = [&](int buf, int h, uint4 (&a)[2][TM]) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int t = 0; t < TM; ++t)
                a[pp][t] = astage[buf][(16 * t + j) * kRowU4 + swapped_k_offset(g, 2 * h + pp) / 8];
    };
    auto compute_seg = [&](int buf, SegWN &d) {
#pragma unroll
        for (int b = 0; b < kTN; ++b) permlane32_swap_dwords(d.w[b]);
        uint4 a[2][2][TM];  // [half][dword in half][token block]
        uint4 bh[2], bl[2];
        floatx4 blk[2][TM];
        load_ops(buf, 0, a[0]);
        lookup(d, 0, bh[0], bl[0]);
#pragma unroll
        for (int gg = 0; gg < 8; ++gg) {
            if (gg + 1 < 8) lookup(d, gg + 1, bh[(gg + 1) & 1], bl[(gg + 1) & 1]);
            if (gg == 1) load_ops(buf, 1, a[1]);
            __builtin_amdgcn_sched_barrier(0);
            const int h = gg >> 2, pp = gg & 1, qq = gg >> 1;
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const floatx4 c = pp == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : blk[qq & 1][t];
                blk[qq & 1][t] = mfma_bf16_16x16x32(as_bf16x8(a[h][pp][t]), as_bf16x8(bh[gg & 1]), c);
                blk[qq & 1][t] = mfma_bf16_16x16x32(as_bf16x8(a[h][pp][t]), as_bf16x8(bl[gg & 1]), blk[qq & 1][t]);
            }
            if (pp && qq >= 1) scale(d, qq - 1, blk[(qq - 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        scale(d, 3, blk[1]);
    };

    // Prologue: segment 0's activations, two segments' weights, the table
    // (512 threads: threads e and e + 256 each write 16 of entry e's copies),
    // segment 0 staged, segment 1's activations in flight.
    SegWN s0, s1;
    stage_load(0);
    load_w(0, s0);
    load_w(1, s1);
    {
        const int e = tid & 255;
        const float c0 = codebook[e & 15], c1 = codebook[e >> 4];
        const uint2 v = pair_table_entry(c0, c1);
        const int half = tid >> 8;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int cp = (e + half * 16 + c) & 31;
            table[e * 64 + cp] = v.x;
            table[e * 64 + 32 + cp] = v.y;
        }
    }
    stage_store(0);
    stage_load(1);
    lds_barrier();

    // Segment i from staging buffer buf; then stage segment i + 1 into the
    // other buffer (every wave finished reading it before the last barrier)
    // and start loading segment i + 2's activations.  The loop runs two
    // segments per iteration and a last odd one after it, so every load in
    // the loop is consumed on both exits.
    auto seg = [&](int i, int buf, SegWN &d) {
        compute_seg(buf, d);
        stage_store(buf ^ 1);
        stage_load(i + 2);
        lds_barrier();
    };
    int i = 0;
    for (; i + 2 <= cnt; i += 2) {
        seg(i, 0, s0);
        load_w(i + 2, s0);
        seg(i + 1, 1, s1);
        load_w(i + 3, s1);
    }
    if (i < cnt) compute_seg(0, s0);

    const bool partial = ksplit > 1;  // K split: fp32 partial slabs, no bias
    if (partial) C = static_cast<char *>(C) + (size_t)part * (size_t)M * (size_t)N * 4;
#pragma unroll
    for (int b = 0; b < kTN; ++b) {
        const int n = n0 + wave * 16 * kTN + 16 * b + j;
        if (n >= N) continue;
        const float bv = bias && !partial ? load_elem(bias, n, c_dt) : 0.f;
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int m = m0 + 16 * t + 4 * g + rr;
                if (m < M) store_elem(C, (size_t)m * N + n, acc[t][b][rr] + bv, partial ? kF32 : c_dt);
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

// Layout and K split.  The N-split layout (a quarter of the L2 traffic per
// MFMA) when its 256-feature tiles, times the smallest K split of 1, 2 or 4
// that reaches it, give at least 3/5 of the CUs a workgroup; otherwise the
// K-split layout, its parts chosen to give every CU a workgroup (at least 8
// segments per part).  Measured on MI355X at M = 64 .. 256 on the decode
// shapes: the N-split layout is 1.2x to 1.5x faster wherever it fills the
// GPU, 1.2x to 4x slower where it cannot.  layout 0 or 1 forces one.
TiledPlan q4_fused_tiled_plan(int M, int N, int K, int max_ks, int layout) {
    const int bm = tile_rows(M);
    const int mb = (M + bm - 1) / bm;
    const int nseg = (K + 127) / 128;
    const int cus = device_info().num_cus;
    if (max_ks < 1) max_ks = 1;
    if (layout != 0) {
        const int tiles = mb * ((N + kTileNN - 1) / kTileNN);
        int best = 0;
        for (int ks = 1; ks <= 4 && ks <= max_ks; ks *= 2) {
            if (ks > 1 && nseg / ks < 4) break;
            best = ks;
            if (tiles * ks * 5 >= cus * 3) return TiledPlan{1, ks};
        }
        if (layout == 1) return TiledPlan{1, best > 0 ? best : 1};
    }
    const int tiles = mb * ((N + kTileN - 1) / kTileN);
    int ks = 1;
    while (ks < 4 && ks < max_ks && tiles * ks < cus && nseg / (ks + 1) >= 8) ++ks;
    return TiledPlan{0, ks};
}

hipError_t launch_q4_fused_tiled(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                                 const float *codebook, const void *bias, int M, int N, int K,
                                 int bs_log2, int wl, const TiledPlan &plan, void *C, int c_dt,
                                 hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    const int ksplit = plan.ksplit;
    if (bs_log2 < 6 || ksplit < 1 || (ksplit > 1 && (bias || c_dt != kF32)) ||
        (wl && (N % 16 != 0 || K % 128 != 0)))
        return hipErrorInvalidValue;
    const int bm = tile_rows(M);
    const int m_blocks = (M + bm - 1) / bm;
    const int nseg = (K + 127) / 128;
    if (plan.layout == 1) {
        const int n_blocks = (N + kTileNN - 1) / kTileNN;
        const uint32_t per_xcd = (uint32_t)(((int64_t)m_blocks * n_blocks * ksplit + 7) / 8);
        const int spp = (nseg + ksplit - 1) / ksplit;
        const unsigned grid = 8u * per_xcd;
#define Q4_TILED_NS(T, L)                                                                     \
    fused_tiled_ns_kernel<T, L><<<dim3(grid), dim3(64 * kWavesN), 0, s>>>(                  \
        A, Wpacked, absmax, codebook, bias, M, N, K, bs_log2, m_blocks, n_blocks, ksplit, per_xcd, \
        spp, C, c_dt)
        if (bm == 64) {
            if (wl) Q4_TILED_NS(4, 1);
            else Q4_TILED_NS(4, 0);
        } else {
            if (wl) Q4_TILED_NS(2, 1);
            else Q4_TILED_NS(2, 0);
        }
#undef Q4_TILED_NS
        return hipGetLastError();
    }
    const int n_blocks = (N + kTileN - 1) / kTileN;
    const int spp = ((nseg + ksplit - 1) / ksplit + kWaves - 1) / kWaves * kWaves;
    const unsigned grid = (unsigned)(8 * m_blocks * ((n_blocks + 7) / 8) * ksplit);
#define Q4_TILED_KS(T, L)                                                                    \
    fused_tiled_ks_kernel<T, L><<<dim3(grid), dim3(64 * kWaves), 0, s>>>(                  \
        A, Wpacked, absmax, codebook, bias, M, N, K, bs_log2, m_blocks, n_blocks, ksplit, spp, C, \
        c_dt)
    if (bm == 64) {
        if (wl) Q4_TILED_KS(4, 1);
        else Q4_TILED_KS(4, 0);
    } else {
        if (wl) Q4_TILED_KS(2, 1);
        else Q4_TILED_KS(2, 0);
    }
#undef Q4_TILED_KS
    return hipGetLastError();
}

}  // namespace q4
