// Fused 4-bit dequantize + skinny GEMM on the matrix cores (blocksize >= 64).
//
// C[M,N] = A[M,K] * dequant(W)^T for M <= 16: the fused path of the
// bitsandbytes pull request "[ROCm] Optimize kgemm_4bit_inference_naive for
// ROCm, use it for batch sizes other than 1" (sections "Kernel optimization"
// and "Fused path support for M > 1"), laid out for CDNA4 rather than after
// the SIMT kernel of the pages.  Each packed byte is read from HBM once.
//
// Decode.  A 256-entry LDS table maps one packed byte (two codes c0, c1) to
// two dwords: (hi(c0), hi(c1)) and (lo(c0), lo(c1)) in bf16, where
// hi = bf16(cb) and lo = bf16(cb - hi), so hi + lo equals the fp32 codebook
// value to within 2^-16 relative (exactly for values of at most 16
// significant bits).  One ds_read_b64 decodes two weights.  Two
// such reads form one B operand of v_mfma_f32_16x16x32_bf16 laid out
// [hi(c0) hi(c1) lo(c0) lo(c1) hi(c2) hi(c3) lo(c2) lo(c3)] against the A
// operand [a0 a1 a0 a1 a2 a3 a2 a3], so the matrix core forms a*hi + a*lo
// exactly and accumulates in fp32, and the loaded registers are the operand
// registers.  The absmax of each 64-wide block scales the block's partial
// sum (acc += absmax * D_block).
//
// The table is stored 32 times, interleaved so that entry b of lane l sits
// at byte b*256 + 8*(l % 32): every lane reads its own pair of LDS banks
// whatever byte it decodes, so the random lookups never conflict (a single
// copy loses about half its LDS cycles to bank conflicts).  One v_perm_b32
// builds that address from the packed byte and the lane's offset.
//
// Tiles.  A tile is 16 output features (the B-operand columns, lane % 16)
// over all of K, walked in 128-wide segments: each lane takes 16 bytes (32
// codes) of its feature's row per segment, 8 from the segment's first
// 64-wide block (dwords 0, 1) and 8 from the second (dwords 2, 3), so that
// every MFMA step draws from a single 64-wide block, which keeps the absmax
// scaling exact per block; one load instruction brings 1 KiB.  The tile
// layout stores the bytes in that order.  Over rows lane group g = lane / 16
// reads the 16 bytes at byte 16*g of the segment (groups 0,1 hold the first
// block, groups 2,3 the second) and half of each lane's dwords are exchanged
// with the lane 32 away by one v_permlane32_swap pair.
// Tokens feed the A operand, one per row; rows without a token read zeros
// and their outputs are discarded.  Output row 4g + r of an MFMA lands in
// lane group g, accumulator r, so with one token block token t takes row
// 4 (t % 4) + t / 4: up to 4 tokens then need one accumulator per lane
// (SR = 1), up to 8 two, up to 16 four, which saves the scaling and the
// cross-wave sums of the empty rows.  Two token blocks (up to 32 tokens)
// keep token t at row t of block t / 16.  fp16 / fp32 activations arrive as
// NP = 2 / 3 exact bf16 planes ([NP][M][K]); plane p of token t then takes
// row 4 (t % 4) + NP (t / 4) + p, so a token's planes land in one lane and
// are added there, in plane order, before the bias and the rounding.
//
// Schedule.  One persistent 8-wave workgroup per CU.  Tiles form groups of
// TB (1..8, the tiles each CU must cover, chosen per shape so that only the
// last group holds fewer live tiles); workgroup b computes groups b, b+G, ...
// as chunks.  The waves of a workgroup interleave each chunk's 128-wide
// segments, so together they read 64*KW contiguous bytes of every row at a
// time, and walk their work as (slot = segment) x (tile), so the activation
// operand of a segment (read from L2 one slot ahead) serves TB tiles.  Block
// scales are staged through LDS one slot ahead by whole-line cooperative
// loads.  Weight loads run RS slots ahead in a register ring of about 8
// units per wave that continues across chunks, and use buffer loads, whose
// hardware range check returns zeros past the end of a buffer: slots past
// the last segment or past the workgroup's last chunk take an offset beyond
// every buffer, so the loop has no bounds branches and reads nothing it does
// not use.  At the end of a chunk every wave writes its fp32 partials to LDS;
// after a barrier that leaves global loads in flight, each output is summed
// over the waves in wave order (deterministic, no atomics) and stored as
// bf16.
//
// K parts.  When the tile groups would leave compute units idle (320 tiles
// of a 5120-row matrix on 256 CUs give 160 groups of two), K is cut into KS
// parts of SPP segments and workgroup b computes part b / groups of group
// b % groups, one chunk per workgroup.  Each part's fp32 sums go to its own
// slab of a buffer, and a second kernel adds the slabs in part order, adds
// the bias and rounds once (deterministic).  Combining inside this kernel
// (the last workgroup of a group to arrive adds the parts) needs an
// agent-scope release per workgroup, an L2 write-back, which measured far
// slower than the second launch.
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

// LDS-only barrier: waits for this wave's LDS operations, not for its global
// loads still in flight, then synchronises the workgroup.
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr uint32_t kPastEnd = 0x80000000u;  // an offset beyond every buffer: reads zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kBufferFlags);
}

constexpr int KW = 8;  // waves per workgroup

// Activations are bf16 (fp16 and fp32 activations reach this kernel as
// exact bf16 planes).  SR: accumulator rows kept per lane
// (ceil(M / 4) rounded up to 1, 2 or 4).  TB: tiles per chunk.  RS:
// segment slots the weight ring runs ahead, so every wave keeps TB*RS weight
// loads in flight.  UF: slots per loop iteration, a multiple of RS with UF*TB
// even, which makes the ring entry and the decode double-buffer index of
// every unit compile-time constants.  P: slots per scale-staging period (a
// divisor of UF).  MB: blocks of 16 token rows per pass (1, or 2 for up to 32
// tokens): the decoded weights of a unit feed the MFMAs of every block.
template <int SR, int TB, int RS, int UF, int P, int MB, bool BS64, int WL>
__global__ __launch_bounds__(64 * KW) void fused_mfma_kernel(
    const uint16_t *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ absmax, const float *__restrict__ codebook,
    const void *__restrict__ bias, int M, int N, int K, int bs_log2, int groups, int ks,
    int spp, float *__restrict__ kpart, void *__restrict__ C, int c_dt, int np) {
    static_assert(UF % RS == 0 && (UF * TB) % 2 == 0, "static ring and decode-buffer indices");
    static_assert(64 * KW == 512, "two threads per table entry");
    static_assert(MB == 1 || (MB == 2 && SR == 4), "two blocks of full rows");
    __shared__ uint2 table[256 * 32];  // [byte][lane % 32]
    __shared__ float red[KW][TB * SR][64];
    // Raw block scales of the current and the next period of P slots, one
    // row per weight row of the chunk: the P*KW*128/bs blocks the KW = 8
    // waves cover in P slots (16*P at bs = 64).  Each thread stages SP
    // 16-byte pieces per period; there are SP*128/P rows, at least TB*16:
    // the threads past the chunk's rows write to spare rows, so the staging
    // code has no branches.  Rows are P*16 + 2 floats apart so the 16 rows a
    // wave reads at once fall in distinct banks.
    static_assert(P == 1 || P == 2 || P == 4 || P == 8, "4*P divides the workgroup");
    static_assert(UF % P == 0, "periods end inside a loop iteration");
    constexpr int SP = (TB * P + 7) / 8;
    constexpr int kScaleRows = SP * 128 / P;
    static_assert(kScaleRows >= TB * 16, "the chunk's rows fit the staging rows");
    constexpr int kScaleStride = P * 16 + 2;
    __shared__ float scl[2][kScaleRows * kScaleStride];
    const int G = gridDim.x;
    // With K parts the grid is exactly groups * ks workgroups of one chunk.
    const int my_chunks = ks > 1 ? 1 : (groups - (int)blockIdx.x + G - 1) / G;
    if (my_chunks <= 0) return;  // uniform over the workgroup
    const int kpart_ix = ks > 1 ? (int)blockIdx.x / groups : 0;
    const uint32_t grp0 = (uint32_t)blockIdx.x - (uint32_t)(kpart_ix * groups);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // The codebook is read first: loads complete in issue order, so the
    // table can be built while the first weight loads are still in flight.
    const int e_tab = tid & 255;
    const float cb0 = codebook[e_tab & 15], cb1 = codebook[e_tab >> 4];
    const char *tab_bytes = reinterpret_cast<const char *>(table);
    const uint32_t lane_off = (uint32_t)(lane & 31) * 8;

    const int j = lane & 15;
    const int g = lane >> 4;
    const int nseg = (K + 127) >> 7;
    // This workgroup's part: segments seg0 .. seg0 + seg_lim - 1 of each row
    // (all of them without K parts, spp == nseg).  Slots index segments of
    // the part; slots at or past seg_lim read zeros.
    const int seg0 = kpart_ix * spp;
    const int seg_lim = nseg - seg0 < spp ? nseg - seg0 : spp;
    const int spw = (spp + KW - 1) / KW;  // segment slots per wave per chunk
    const uint32_t row_bytes = (uint32_t)K >> 1;
    // Over rows, workgroups start their walk along K at different slots
    // (whole scale periods), chosen by b / 8 so that the workgroups on one XCD
    // do too: neighbouring workgroups then read different parts of their rows
    // at any time, which spreads the loads over more DRAM banks and channels
    // than a walk in lockstep, where every CU reads the same 64-byte column
    // window of rows K/2 bytes apart (measured 10 % faster at 28672 x 8192).
    // Slot q of a chunk is slot (q + rot) % spw of the row.  Over tiles,
    // where each unit is 1 KiB of contiguous memory, the lockstep walk
    // measured 3-4 % faster than the rotated one (same shape, M = 1..16), so
    // tiles walk from slot 0.
    const int nper = spw / P;  // whole periods per chunk
    const int rot = WL == 0 && spw % P == 0 ? (int)((blockIdx.x / 8u) % (uint32_t)nper) * P : 0;
    const uint32_t nb = (uint32_t)K >> bs_log2;

    const __amdgpu_buffer_rsrc_t wres = make_rsrc(Wp, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t sres = make_rsrc(absmax, (uint32_t)N * nb * 4);
    const __amdgpu_buffer_rsrc_t ares = make_rsrc(A, (uint32_t)(np * M) * (uint32_t)K * 2);

    // Chunk c of this workgroup is tile group blockIdx.x + c*G; tile tr of
    // group q is q + tr*groups, so at any time neighbouring workgroups read
    // neighbouring 16-row tiles.  Slot q of wave w is segment w + q*KW (the
    // waves of a workgroup read 64*KW contiguous bytes of each row at a time).
    auto group_of = [&](int c) { return grp0 + (uint32_t)c * (uint32_t)G; };
    const uint32_t w_tile_step = 16u * (uint32_t)groups * row_bytes;
    // The lane's part of a weight offset, and the shift from a segment to its
    // offset.  Row-major: segment s of row n is the 64 bytes at
    // n*row_bytes + 64*s, lane (j, g) reads 16 of them at 16*g.  Tile layout:
    // the 16 rows x 64 bytes of (tile, segment) are one 1 KiB unit at
    // (tile*nseg + s) * 1024 that holds lane l's 16 bytes at 16*l, already in
    // the order the MFMA steps use (8 bytes of the segment's first 64-wide
    // block, then 8 of its second): one 128-bit load per lane and unit, 1 KiB
    // of contiguous memory per instruction, no lane exchange (measured 3-4 %
    // faster at M = 1..4 than two 64-bit loads of 512 bytes each from the
    // earlier tile order).  Over rows each lane loads its own 16 bytes (half
    // from each block would make each instruction read 32-byte pieces of 16
    // rows, which measured 40 against 28 us at M = 1 on the FFN) and one
    // v_permlane32_swap pair regroups them.  A tile spans 16*row_bytes bytes
    // in both layouts.
    const uint32_t w_lane = (WL ? 16u * (uint32_t)lane : (uint32_t)j * row_bytes + 16u * (uint32_t)g) +
                            ((uint32_t)seg0 << (WL ? 10 : 6));
    const int seg_sh = WL ? 10 : 6;

    // Weight issue cursor: the (chunk, slot) whose loads are issued next.
    // Slots past this workgroup's last chunk and segments past the end of a
    // row take an offset beyond the buffer: they read zeros without touching
    // memory.
    int ic = 0, iq = 0;
    uint32_t w_row0 = group_of(0) * 16 * row_bytes + w_lane;
    bool w_live = true;
    int iqr = rot;  // (iq + rot) % spw, kept incrementally (no division per slot)
    auto w_seek = [&]() {
        const int seg = wave + iqr * KW;
        w_live = ic < my_chunks && seg < seg_lim;
        w_row0 = group_of(ic) * 16 * row_bytes + ((uint32_t)seg << seg_sh) + w_lane;
    };
    auto w_advance = [&]() {
        if (++iqr == spw) iqr = 0;
        if (++iq == spw) {
            iq = 0;
            ++ic;
        }
        w_seek();
    };
    w_seek();
    // Each weight byte is read once: the loads carry the non-temporal hint
    // (cache policy bit 1), which measured 2-5 % faster over the tile layout
    // at M = 1..8 (neutral over rows).
    auto issue = [&](uint4 &dst, int tr) {
        const uint32_t wo = w_live ? w_row0 + (uint32_t)tr * w_tile_step : kPastEnd;
        dst = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wres, (int)wo, 0, 2));
    };

    // Scales are staged through LDS one period (P slots) ahead: per period
    // the workgroup needs the P*KW*128/bs consecutive block scales of each of
    // its TB*16 rows (64*P bytes per row at bs = 64), which thread t fetches
    // as 16-byte piece t % (4*P) of chunk rows t / (4*P) + i*128/P, i < SP:
    // whole cache lines with no duplicates.
    const int s_row = tid / (4 * P);
    const uint32_t s_piece = (uint32_t)(tid % (4 * P)) * 16;
    const uint32_t s_win = (uint32_t)(P * KW * 128 * 4) >> bs_log2;  // bytes per row per period
    // The part's scales: from its first block to the end of its last one.
    const uint32_t s_first = ((uint32_t)seg0 * 128 >> bs_log2) * 4;
    const uint32_t s_blocks_end = ((uint32_t)(seg0 + seg_lim) * 128 + (1u << bs_log2) - 1) >> bs_log2;
    const uint32_t s_end = (s_blocks_end < nb ? s_blocks_end : nb) * 4;
    int sc = 0, sq = 0;  // scale cursor: the first slot of the period loaded next
    int sqr = rot;       // (sq + rot) % spw
    // Bytes of this thread's piece that lie inside the row (a piece may run
    // past the row's last block when K / bs is not a multiple of 4: those
    // scales belong to the next row and are zeroed at staging, so that a
    // non-finite scale there cannot turn the 0 * scale of the padded blocks
    // into NaN).
    int s_rem = 16;
    // Byte offset of this thread's pieces in their rows' scales for the chunk
    // being loaded (kPastEnd for the spare rows past the chunk's tiles); set
    // once per chunk, so a period adds only its window start.
    uint32_t s_rowoff[SP];
    auto scale_rows = [&]() {
#pragma unroll
        for (int i = 0; i < SP; ++i) {
            const int row = s_row + i * (128 / P);
            const uint32_t ns = (group_of(sc) + (uint32_t)(row >> 4) * (uint32_t)groups) * 16 +
                                (uint32_t)(row & 15);
            s_rowoff[i] = row < TB * 16 && s_piece < s_win ? ns * nb * 4 + s_piece : kPastEnd;
        }
    };
    scale_rows();
    auto load_scales = [&](floatx4 (&out)[SP]) {
        const uint32_t w0 = s_first + ((uint32_t)sqr * KW * 128 >> bs_log2) * 4;  // window start
        const bool live = sc < my_chunks && w0 + s_piece < s_end;
        s_rem = (int)s_end - (int)(w0 + s_piece);
#pragma unroll
        for (int i = 0; i < SP; ++i) {
            const uint32_t so = live ? s_rowoff[i] + w0 : kPastEnd;
            out[i] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(sres, (int)so, 0, 0));
        }
        sq += P;
        sqr += P;
        if (sqr >= spw) sqr -= spw;
        if (sq >= spw) {
            sq = 0;
            sqr = rot;
            ++sc;
            scale_rows();
        }
    };
    // Writes the pieces into the staging buffer; every thread writes, so the
    // compiler has no branch to sink the scale loads into and they stay a
    // period ahead of their use.
    auto stage_scales = [&](const floatx4 (&v)[SP], int buf) {
#pragma unroll
        for (int i = 0; i < SP; ++i) {
            float *row = &scl[buf][(s_row + i * (128 / P)) * kScaleStride + (s_piece >> 2)];
            const float x0 = s_rem > 0 ? v[i][0] : 0.f, x1 = s_rem > 4 ? v[i][1] : 0.f;
            const float x2 = s_rem > 8 ? v[i][2] : 0.f, x3 = s_rem > 12 ? v[i][3] : 0.f;
            *reinterpret_cast<floatx2 *>(row) = floatx2{x0, x1};
            *reinterpret_cast<floatx2 *>(row + 2) = floatx2{x2, x3};
        }
    };
    // In slot u of a period, wave w applies the scales of the 64-wide blocks
    // e = 16u + 2w and e + 1 of the period window, which lie in bs-wide blocks
    // e >> sh and (e + 1) >> sh: one 8-byte read at the even block below, then
    // a select (both halves for bs = 64, one half twice for bs = 128 and 256).
    const int sh = BS64 ? 0 : bs_log2 - 6;
    auto read_scales = [&](const float *p) { return *reinterpret_cast<const floatx2 *>(p); };
    auto pick_scales = [&](const floatx2 &a2, int pick, float (&out)[2]) {
        out[0] = pick == 1 ? a2[1] : a2[0];
        out[1] = pick == 0 ? a2[0] : a2[1];
    };

    // Activation operand of slot q: token j's 8 activations for each of the
    // lane's 4 dwords of codes.  Rows of tokens >= M lie past the end of A,
    // and k >= K (a ragged last segment, or a slot past the last segment)
    // takes an offset past every buffer: both read zeros without touching
    // memory, which cancels whatever codes sit there.
    //
    // Lane (j, g) reads at k = kk + L + T(t) with L = 32 (g & 1) + 16 (g >> 1)
    // its own part and T(t) = 8 (t & 1) + 64 (t >> 1) (swapped_k_offset), so
    // one per-lane base per slot and immediate offsets 0, 16, 128, 144 give
    // the four loads.  K is a multiple of 64 here: dwords 0, 1 (k < kk + 64)
    // are live when kk + 64 <= K and dwords 2, 3 when kk + 128 <= K, the same
    // for every lane.
    // A row j = 4 (t % 4) + np q + p holds plane p of token t (q = t / 4);
    // rows without a token read past the end of A
    const int j_r = j & 3, j_q = j_r / np, j_p = j_r - j_q * np, tok_j = 4 * j_q + (j >> 2);
    const uint32_t a_rowoff = MB == 2 ? (uint32_t)j * (uint32_t)K * 2
                              : tok_j < M ? (uint32_t)(j_p * M + tok_j) * (uint32_t)K * 2 : kPastEnd;
    const uint32_t a_lane = a_rowoff +
                            2u * (32u * (uint32_t)(g & 1) + 16u * (uint32_t)(g >> 1));
    uint4 anext[MB][4];
    auto load_a = [&](int qr) {  // qr: the slot's index along the part, (q + rot) % spw
        const int ls = wave + qr * KW;  // segment of the part
        const uint32_t kk = (uint32_t)(seg0 + ls) * 128;
        const uint32_t base = a_lane + 2u * kk;
        const bool in = ls < seg_lim;
        const uint32_t lo = in && kk + 64 <= (uint32_t)K ? base : kPastEnd;
        const uint32_t hi = in && kk + 128 <= (uint32_t)K ? base : kPastEnd;
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            const uint32_t bo = (uint32_t)(16 * b) * (uint32_t)K * 2;
            anext[b][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, (int)(lo + bo), 0, 0));
            anext[b][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, (int)(lo + bo + 16), 0, 0));
            anext[b][2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, (int)(hi + bo + 128), 0, 0));
            anext[b][3] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, (int)(hi + bo + 144), 0, 0));
        }
    };

    // Table lookups of one tile: 16 packed bytes -> 32 bf16 hi/lo pairs,
    // with the codes of the segment's first 64-wide block in dwords 0, 1 and
    // those of the second in dwords 2, 3 (as loaded over tiles; over rows
    // after the exchange).
    auto swap_w = [&](const uint4 &wv, uint32_t (&x)[4]) {
        x[0] = wv.x; x[1] = wv.y; x[2] = wv.z; x[3] = wv.w;
        if constexpr (WL == 0) {
            // lanes 0-31 keep dwords 0,1 and take dwords 0,1 of lane+32;
            // lanes 32-63 take dwords 2,3 of lane-32 and keep dwords 2,3
            const auto s02 = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
            x[0] = s02[0]; x[2] = s02[1];
            x[1] = s13[0]; x[3] = s13[1];
        }
    };
    auto lookups = [&](const uint32_t (&x)[4], uint2 (&ev)[16], int i0, int i1) {
#pragma unroll
        for (int i = i0; i < i1; ++i) {
            // address = byte * 256 + lane_off: byte 1 from the packed
            // dword, byte 0 from lane_off, bytes 2-3 zero
            const uint32_t addr = __builtin_amdgcn_perm(x[i >> 2], lane_off, 0x0c0c0000u | ((4 + (i & 3)) << 8));
            ev[i] = *reinterpret_cast<const uint2 *>(tab_bytes + addr);
        }
    };
    auto decode = [&](const uint4 &wv, uint2 (&ev)[16]) {
        uint32_t x[4];
        swap_w(wv, x);
        lookups(x, ev, 0, 16);
    };

    // Prologue: the scales and activations of slot 0, RS slots of weights,
    // then the table, then the first decode.
    uint4 wbuf[RS][TB];
    {
        floatx4 s0[SP];
        load_scales(s0);
        load_a(rot);
#pragma unroll
        for (int r = 0; r < RS; ++r) {
#pragma unroll
            for (int tr = 0; tr < TB; ++tr) issue(wbuf[r][tr], tr);
            w_advance();
        }
        {
            // Threads t and t + 256 write entry t & 255 into 16 copies each.
            // Lane l of a wave starts at copy l % 32, so the 32 lanes of a
            // half-wave write 32 different bank pairs (writing copy c from
            // every lane at once would put all 64 lanes on one bank pair).
            const uint2 v = pair_table_entry(cb0, cb1);
            const int c0 = (tid >> 8) * 16 + e_tab;
#pragma unroll
            for (int c = 0; c < 16; ++c) table[e_tab * 32 + ((c0 + c) & 31)] = v;
        }
        stage_scales(s0, 0);
        lds_barrier();
    }
    // Decoded units: double-buffered with one token block, so the table
    // reads of the next unit fly while this unit's MFMAs run; with two
    // blocks the 16 MFMAs of a unit cover that latency and the registers go
    // to the second block's activations.
    constexpr int DB = MB == 1 ? 2 : 1;
    uint2 e[DB][16];
    // Scale pairs of the current and the next unit: with the double-buffered
    // decode raw (the pick is applied where they are used), else picked at
    // the read (fewer live registers for two token blocks).
    floatx2 am[2];
    decode(wbuf[0][0], e[0]);
    issue(wbuf[0][0], 0);

    const floatx4 zerof = floatx4{0.f, 0.f, 0.f, 0.f};
    float acc[TB][MB][SR];
#pragma unroll
    for (int tr = 0; tr < TB; ++tr)
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int r = 0; r < SR; ++r) acc[tr][b][r] = 0.f;
    int pqr = rot;  // the slot being computed, as its index along the row
    int qp = 0;   // periods done, for the staging buffer parity
    floatx4 snext[SP];  // the next period's scale pieces

    // One slot: TB units (tiles) of 16 rows x 128 k, software-pipelined one
    // unit ahead: the table reads of unit u+1 (the next tile, or tile 0 of
    // the next slot) are in flight while the MFMAs of unit u run, and each
    // ring entry is refilled RS slots ahead right after its decode.  The slot
    // loop starts every chunk at ring entry 0 and decode buffer 0, which holds
    // when a workgroup has one chunk, or when a chunk is a whole number of
    // loop iterations (spw a multiple of UF).
    auto slot = [&](auto us_c) {
        constexpr int us = decltype(us_c)::value;
        constexpr int r_cur = us % RS, r_next = (us + 1) % RS;
        // Activation operand, each pair of activations duplicated (fp16
        // activations as two bf16 operands, hi and lo).  Built once per slot
        // and pinned in registers: an MFMA whose operand a VALU instruction has
        // just written stalls for the hazard, so the compiler must not rebuild
        // these next to every MFMA.
        uint4 adup[MB][8];
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 &an = anext[b][t];
                adup[b][2 * t] = make_uint4(an.x, an.x, an.y, an.y);
                adup[b][2 * t + 1] = make_uint4(an.z, an.z, an.w, an.w);
            }
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int s = 0; s < 8; ++s)
                __asm__ volatile("" : "+v"(adup[b][s].x), "+v"(adup[b][s].y), "+v"(adup[b][s].z),
                                 "+v"(adup[b][s].w));
        load_a(pqr + 1 == spw ? 0 : pqr + 1);  // the activations of the next slot
        if constexpr (us % P == 0) load_scales(snext);  // and the next period's scales
        const int s_blk = (16 * (us % P) + 2 * wave) >> sh;
        const int s_pick = BS64 || sh == 0 ? -1 : (s_blk & 1);
        auto picked = [&](const floatx2 &a2) {
            float o[2];
            pick_scales(a2, s_pick, o);
            return floatx2{o[0], o[1]};
        };
        const float *scs = &scl[qp & 1][j * kScaleStride + (s_blk & ~1)];
        am[(us * TB) & 1] = DB == 2 ? read_scales(scs) : picked(read_scales(scs));
        // Block sums of the previous tile and their scales: with one token
        // block a tile's sums are scaled into its accumulators one unit
        // later, after the next tile's MFMAs are issued, so the wave does not
        // wait for its own MFMAs to finish (measured 2-3 % at M = 1..4; same
        // values, same order).  Two token blocks have no registers to spare
        // for it and scale at once.
        floatx4 P0[MB], P1[MB];
        float psc[2];
        auto scale_into = [&](float (&a)[MB][SR]) {
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
                for (int r = 0; r < SR; ++r)
                    a[b][r] = fmaf(psc[1], P1[b][r], fmaf(psc[0], P0[b][r], a[b][r]));
        };
#pragma unroll
        for (int tr = 0; tr < TB; ++tr) {
            const int cur = (us * TB + tr) & 1;
            const int ecur = DB == 2 ? cur : 0, enext = DB == 2 ? cur ^ 1 : 0;
            const uint2 *ev = e[ecur];
            // two independent chains per token block, one per 64-wide block
            floatx4 D0[MB], D1[MB];
#pragma unroll
            for (int b = 0; b < MB; ++b) D0[b] = D1[b] = zerof;
            auto mfma_steps = [&](int s0, int s1) {
#pragma unroll
                for (int s = s0; s < s1; ++s) {
                    const uint4 b0 = make_uint4(ev[2 * s].x, ev[2 * s].y, ev[2 * s + 1].x, ev[2 * s + 1].y);
                    const uint4 b1 = make_uint4(ev[8 + 2 * s].x, ev[8 + 2 * s].y, ev[9 + 2 * s].x, ev[9 + 2 * s].y);
#pragma unroll
                    for (int b = 0; b < MB; ++b) {
                        D0[b] = mfma_bf16_16x16x32(as_bf16x8(adup[b][s]), as_bf16x8(b0), D0[b]);
                        D1[b] = mfma_bf16_16x16x32(as_bf16x8(adup[b][4 + s]), as_bf16x8(b1), D1[b]);
                    }
                }
            };
            if constexpr (DB == 2) {
                // The next unit's decode interleaved with this unit's MFMAs,
                // so its table reads fly while the MFMAs run.
                uint32_t xn[4];
                if (tr + 1 < TB) {
                    swap_w(wbuf[r_cur][tr + 1], xn);
                } else {
                    // tile 0 of the next slot: its weights are in the ring;
                    // its scales are read at the start of that slot
                    w_advance();
                    swap_w(wbuf[r_next][0], xn);
                }
                lookups(xn, e[enext], 0, 16);
                if (tr + 1 < TB) {
                    am[cur ^ 1] = read_scales(scs + (tr + 1) * 16 * kScaleStride);
                    issue(wbuf[r_cur][tr + 1], tr + 1);
                } else {
                    issue(wbuf[r_next][0], 0);
                }
                mfma_steps(0, 4);
                // Each MFMA followed by four VALU instructions and two table
                // reads of the next unit, so one wave keeps the matrix core,
                // the VALU and the LDS busy together (the compiler otherwise
                // clusters the dependent MFMAs of a chain).
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
                }
                __builtin_amdgcn_sched_barrier(0);
            } else {
                // One decode buffer: the next unit's table reads follow this
                // unit's MFMAs.
                mfma_steps(0, 4);
                __builtin_amdgcn_sched_barrier(0);
                if (tr + 1 < TB) {
                    decode(wbuf[r_cur][tr + 1], e[enext]);
                    am[cur ^ 1] = picked(read_scales(scs + (tr + 1) * 16 * kScaleStride));
                    issue(wbuf[r_cur][tr + 1], tr + 1);
                } else {
                    w_advance();
                    decode(wbuf[r_next][0], e[enext]);
                    issue(wbuf[r_next][0], 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // With the double-buffered decode the pick (for blocksizes above
            // 64) runs here, not next to the read: a use right after the read
            // would wait for it, and LDS reads complete in order, so also for
            // the table reads of the next unit issued just before it.
            float sc[2] = {am[cur][0], am[cur][1]};
            if constexpr (DB == 2) pick_scales(am[cur], s_pick, sc);
            if constexpr (MB == 1) {
                if (tr > 0) scale_into(acc[tr > 0 ? tr - 1 : 0]);
            }
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                P0[b] = D0[b];
                P1[b] = D1[b];
                // Keep all four MFMA result registers live until here: the
                // rows past SR are unused, and reusing their registers right
                // after the MFMA makes the wave wait for its write-back.
                if constexpr (MB == 1) __asm__ volatile("" ::"v"(D0[b]), "v"(D1[b]));
            }
            psc[0] = sc[0];
            psc[1] = sc[1];
            if constexpr (MB == 2) scale_into(acc[tr]);
        }
        if constexpr (MB == 1) scale_into(acc[TB - 1]);
        // At the end of a period, publish the next period's scales.  The
        // buffer written here was last read in the previous period, which
        // every wave finished before the previous barrier.
        if constexpr (us % P == P - 1) {
            stage_scales(snext, (qp + 1) & 1);
            lds_barrier();
            ++qp;
        }
        if (++pqr == spw) pqr = 0;
    };

    // Chunk end: combine the KW partials of the chunk's tiles.  Output (tile,
    // token row) pair p is summed by wave p % KW in wave order (no atomics:
    // the result is deterministic).  The buffer is rewritten at the next
    // chunk end, after at least one more period barrier (every chunk holds
    // at least one period end).  The stores of C sit
    // outside the unrolled slot loop: a store makes the compiler wait for
    // every outstanding load before the next use of a loaded register, which
    // here happens once per chunk instead of once per slot.
    for (int pc = 0;;) {
        for (int q0 = 0; q0 < spw; q0 += UF) {
            slot(std::integral_constant<int, 0>{});
            if constexpr (UF > 1) { if (q0 + 1 < spw) slot(std::integral_constant<int, 1 % UF>{}); }
            if constexpr (UF > 2) { if (q0 + 2 < spw) slot(std::integral_constant<int, 2 % UF>{}); }
            if constexpr (UF > 3) { if (q0 + 3 < spw) slot(std::integral_constant<int, 3 % UF>{}); }
            if constexpr (UF > 4) { if (q0 + 4 < spw) slot(std::integral_constant<int, 4 % UF>{}); }
            if constexpr (UF > 5) { if (q0 + 5 < spw) slot(std::integral_constant<int, 5 % UF>{}); }
            if constexpr (UF > 6) { if (q0 + 6 < spw) slot(std::integral_constant<int, 6 % UF>{}); }
            if constexpr (UF > 7) { if (q0 + 7 < spw) slot(std::integral_constant<int, 7 % UF>{}); }
        }
        const uint32_t grp = group_of(pc);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            // token block b reuses the buffer: wait until every wave has read
            // block b - 1
            if (b > 0) lds_barrier();
#pragma unroll
            for (int tr = 0; tr < TB; ++tr)
#pragma unroll
                for (int r = 0; r < SR; ++r) {
                    red[wave][tr * SR + r][lane] = acc[tr][b][r];
                    acc[tr][b][r] = 0.f;
                }
            lds_barrier();
            if (MB == 1 && np > 1) {
                // output (tile, token group q): each plane's row summed over
                // the waves in wave order, then the planes in plane order
                const int qg = SR / np;
                for (int o0 = 0; o0 < TB * qg; o0 += KW) {
                    const int o = o0 + wave;
                    if (o < TB * qg) {
                        const int tr = o / qg, q = o - tr * qg;
                        float v = 0.f;
                        for (int pl = 0; pl < np; ++pl) {
                            const int p = tr * SR + q * np + pl;
                            float vp = red[0][p][lane];
#pragma unroll
                            for (int w2 = 1; w2 < KW; ++w2) vp += red[w2][p][lane];
                            v = pl == 0 ? vp : v + vp;
                        }
                        const int n = (int)((grp + (uint32_t)tr * (uint32_t)groups) * 16) + j;
                        const int tok = 4 * q + g;
                        if (n < N && tok < M) {
                            if (bias) v += load_elem(bias, n, c_dt);  // before the single rounding
                            store_elem(C, (size_t)tok * N + n, v, c_dt);
                        }
                    }
                }
            } else {
#pragma unroll
            for (int p0 = 0; p0 < TB * SR; p0 += KW) {
                const int p = p0 + wave;
                if (p < TB * SR) {
                    const int tr = p / SR, r = p % SR;
                    float v = red[0][p][lane];
#pragma unroll
                    for (int w2 = 1; w2 < KW; ++w2) v += red[w2][p][lane];
                    const int n = (int)((grp + (uint32_t)tr * (uint32_t)groups) * 16) + j;
                    const int tok = MB == 1 ? 4 * r + g : 16 * b + 4 * g + r;
                    if (n < N && tok < M) {
                        if (ks > 1) {
                            kpart[((size_t)kpart_ix * M + tok) * N + n] = v;  // this part's sum
                        } else {
                            if (bias) v += load_elem(bias, n, c_dt);  // before the single rounding
                            store_elem(C, (size_t)tok * N + n, v, c_dt);
                        }
                    }
                }
            }
            }
        }
        if (++pc == my_chunks) break;
    }
}

// Tiles per chunk: the tiles each CU must cover, at most 8.
int tiles_per_chunk(int N) {
    const int tiles = (N + 15) / 16;
    const int cus = device_info().num_cus;
    const int tb = (tiles + cus - 1) / cus;
    return tb > 8 ? 8 : tb;
}

// Work plan: tiles per chunk (tb), K parts (ks) of spp segments each.
struct SkinnyPlan {
    int tb, ks, spp;
};

// Without K parts a workgroup walks ceil(groups / CUs) chunks of tb tiles
// times ceil(segments / 8) slots.  With up to 32 token rows in one pass, K
// parts are used when some (tb, ks) with groups * ks <= CUs (one chunk per
// workgroup) saves at least 8 units per wave and 20 % of them: the second
// launch that adds the parts costs about as much as 4 units (a unit is
// ~0.42 us at 17408 x 5120 with one token block), so 17408 x 5120 goes from
// 34 to 24 units per wave while 5120 x 5120 (10 to 7) keeps one part.  Two
// token blocks (17..32 rows) take the same plans without 8-tile chunks
// (which run as two 16-row passes).  Parts are whole slots of the 8 waves
// (spp a multiple of 8 segments), so every part starts on a scale block
// boundary for blocksizes up to 1024.
SkinnyPlan skinny_plan(int M, int N, int K) {
    const int tb0 = tiles_per_chunk(N);
    const int nseg = (K + 127) / 128;
    SkinnyPlan plan{tb0, 1, nseg};
    if (M > 32 || (M > 16 && tb0 >= 8)) return plan;  // 8-tile chunks run 16-row passes
    const int tiles = (N + 15) / 16;
    const int cus = device_info().num_cus;
    const long groups0 = (tiles + tb0 - 1) / tb0;
    const long base = (groups0 + cus - 1) / cus * tb0 * ((nseg + KW - 1) / KW);
    long best = base;
    for (int tb = 1; tb <= (M > 16 ? 7 : 8); ++tb)
        for (int ks = 2; ks <= 8; ++ks) {
            const int per = (nseg + ks - 1) / ks;
            const int spp = (per + KW - 1) / KW * KW;
            if ((nseg + spp - 1) / spp != ks) continue;  // fewer parts than asked
            const long groups = (tiles + tb - 1) / tb;
            if (groups * ks > cus) continue;
            const long units = (long)tb * (spp / KW);
            if (units + 8 <= base && units * 100 <= base * 80 && units < best) {
                best = units;
                plan = SkinnyPlan{tb, ks, spp};
            }
        }
    return plan;
}

template <int SR, int MB, int TB>
hipError_t launch_tb(const uint16_t *A, const uint8_t *Wp, const float *absmax,
                     const float *codebook, const void *bias, int M, int N, int K, int bs_log2,
                     void *C, int c_dt, int groups, int G, const SkinnyPlan &plan, float *kpart,
                     int np, int wl, hipStream_t s) {
    // Ring depth TB*RS of about 8 units (8 KiB of weights in flight per wave).
    constexpr int RS = TB == 1 ? 8 : TB == 2 ? 4 : TB <= 4 ? 2 : 1;
    constexpr int UF = (RS * TB) % 2 == 0 ? RS : 2 * RS;
    // Scales are staged once per ring period: with one slot (TB >= 5) every
    // slot, which lets workgroups start their walk at any slot; a barrier
    // every slot costs more than it gains for shapes of one or two tiles per
    // chunk (measured), which stage every RS slots.
    constexpr int P = RS;
    // The ring entry and decode buffer of a chunk's first unit are fixed at
    // compile time: a workgroup with several chunks needs chunks of whole
    // loop iterations.
    const int spw = (plan.spp + KW - 1) / KW;
    if (groups > G && spw % UF != 0) return hipErrorInvalidValue;
    if (plan.ks > 1 && (G != groups * plan.ks || !kpart || np != 1))
        return hipErrorInvalidValue;
    if (np > 1 && MB != 1) return hipErrorInvalidValue;
#define Q4_LAUNCH_KERNEL(B, L)                                                          \
    fused_mfma_kernel<SR, TB, RS, UF, P, MB, B, L><<<dim3(G), dim3(64 * KW), 0, s>>>( \
        A, Wp, absmax, codebook, bias, M, N, K, bs_log2, groups, plan.ks, plan.spp, kpart, C, \
        c_dt, np)
    if (bs_log2 == 6) {
        if (wl) Q4_LAUNCH_KERNEL(true, 1);
        else Q4_LAUNCH_KERNEL(true, 0);
    } else {
        if (wl) Q4_LAUNCH_KERNEL(false, 1);
        else Q4_LAUNCH_KERNEL(false, 0);
    }
#undef Q4_LAUNCH_KERNEL
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.ks == 1) return e;
    return launch_sum_planes(kpart, plan.ks, M, N, bias, C, c_dt, s);
}

template <int SR, int MB>
hipError_t launch_sr(const uint16_t *A, const uint8_t *Wp, const float *absmax,
                     const float *codebook, const void *bias, int M, int N, int K, int bs_log2,
                     void *C, int c_dt, float *kpart, int np, int wl, hipStream_t s) {
    // One 8-wave workgroup per CU (the replicated table takes 64 KiB of LDS).
    // TB = the tiles each CU must cover, up to 8, so that every chunk but the
    // last holds TB live tiles; a workgroup loops over ceil(groups / CUs)
    // chunks.  With K parts (a buffer given and the plan asks for them) the
    // grid is groups * ks workgroups of one chunk each.
    SkinnyPlan plan = SkinnyPlan{tiles_per_chunk(N), 1, (K + 127) / 128};
    if (kpart) plan = skinny_plan(M, N, K);
    const int tb = plan.tb;
    const int tiles = (N + 15) / 16;
    const int cus = device_info().num_cus;
    const int groups = (tiles + tb - 1) / tb;
    const int G = plan.ks > 1 ? groups * plan.ks : groups < cus ? groups : cus;
#define Q4_LAUNCH_TB(T) \
    return launch_tb<SR, MB, T>(A, Wp, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt, groups, G, plan, kpart, np, wl, s)
    switch (tb) {
    case 1: Q4_LAUNCH_TB(1);
    case 2: Q4_LAUNCH_TB(2);
    case 3: Q4_LAUNCH_TB(3);
    case 4: Q4_LAUNCH_TB(4);
    case 5: Q4_LAUNCH_TB(5);
    case 6: Q4_LAUNCH_TB(6);
    case 7: Q4_LAUNCH_TB(7);
    default: Q4_LAUNCH_TB(8);
    }
#undef Q4_LAUNCH_TB
}

}  // namespace

// The kernel's byte offsets are 32-bit.  Weight and scale offsets reach the
// rows of the last tile group, at most 8 tiles (128 rows) past the last row,
// so the matrix plus 256 rows must stay below 4 GiB; activation offsets reach
// 32 rows of K (the lanes of absent tokens read past the end of A), which must
// stay below 4 GiB as well.
// One launch takes two token blocks unless 8 tiles per chunk leave no
// registers for the second (then 17..32 rows run as two 16-row launches).
bool q4_fused_mfma_two_blocks(int N) { return tiles_per_chunk(N) < 8; }

int q4_fused_tiles_per_chunk(int N) { return tiles_per_chunk(N); }

int q4_fused_kparts(int M, int N, int K) { return skinny_plan(M, N, K).ks; }

bool q4_fused_mfma_fits(int M, int N, int K) {
    (void)M;
    return ((uint64_t)N + 256) * (uint64_t)K / 2 < (1ull << 32) &&
           32ull * (uint64_t)K * 2 < (1ull << 32);
}

hipError_t launch_q4_fused_mfma(const void *A, int a_dt, const uint8_t *Wpacked,
                                const float *absmax, const float *codebook, const void *bias,
                                int M, int N, int K, int bs_log2, void *C, int c_dt, int wl,
                                hipStream_t s, float *kpart, int np) {
    if (a_dt != kBf16 || M > 32 || (wl && (N % 16 != 0 || K % 128 != 0)))
        return hipErrorInvalidValue;
    // accumulator rows a lane needs: np planes per group of 4 tokens
    const int rows = np * ((M + 3) / 4);
    if (np < 1 || np > 3 || (np > 1 && (rows > 4 || kpart))) return hipErrorInvalidValue;
    const uint16_t *A16 = static_cast<const uint16_t *>(A);
#define Q4_LAUNCH_SR(R, B) \
    return launch_sr<R, B>(A16, Wpacked, absmax, codebook, bias, M, N, K, bs_log2, C, c_dt, kpart, np, wl, s)
    if (rows <= 1) Q4_LAUNCH_SR(1, 1);
    if (rows <= 2) Q4_LAUNCH_SR(2, 1);
    if (rows <= 4) Q4_LAUNCH_SR(4, 1);
    Q4_LAUNCH_SR(4, 2);
#undef Q4_LAUNCH_SR
}

// Up to Q4_FUSED_PASS_M (32) token rows.  bf16 activations with blocksize
// >= 64 run on the matrix cores in one pass (two token blocks), except where a
// chunk holds 8 tiles: there the second block's registers spill and two
// 16-row passes are faster (measured at 248320 x 2560).  Other activations
// reaching this point (blocksize 32, or offsets beyond 32 bits) take the
// vector-ALU kernel in passes of 16 rows.
hipError_t launch_q4_fused(const void *A, int a_dt, const uint8_t *Wpacked, const float *absmax,
                           const float *codebook, const void *bias, int M, int N, int K,
                           int bs_log2, void *C, int c_dt, int wl, hipStream_t s, float *kpart) {
    const bool mfma = a_dt == kBf16 && bs_log2 >= 6 && q4_fused_mfma_fits(M, N, K);
    if (wl && !mfma) return hipErrorInvalidValue;  // the vector-ALU kernel reads rows
    if (mfma && (M <= 16 || tiles_per_chunk(N) < 8))
        return launch_q4_fused_mfma(A, a_dt, Wpacked, absmax, codebook, bias, M, N, K, bs_log2,
                                    C, c_dt, wl, s, kpart, 1);
    const size_t a_row = (size_t)K * (a_dt == kF32 ? 4 : 2);
    const size_t c_row = (size_t)N * (c_dt == kF32 ? 4 : 2);
    for (int m0 = 0; m0 < M; m0 += 16) {
        const int mm = M - m0 < 16 ? M - m0 : 16;
        const void *Am = static_cast<const char *>(A) + (size_t)m0 * a_row;
        void *Cm = static_cast<char *>(C) + (size_t)m0 * c_row;
        const hipError_t e =
            mfma ? launch_q4_fused_mfma(Am, a_dt, Wpacked, absmax, codebook, bias, mm, N, K, bs_log2,
                                        Cm, c_dt, wl, s, nullptr, 1)
                 : launch_q4_fused_simt(Am, a_dt, Wpacked, absmax, codebook, bias, mm, N, K, bs_log2,
                                        Cm, c_dt, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4
