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
// value to within 2^-18 relative.  One ds_read_b64 decodes two weights.  Two
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
// over all of K, walked in 128-wide segments: lane group g = lane / 16 reads
// 16 bytes (32 codes) of its feature's row at byte 16*g of the segment, so a
// feature row is read 64 contiguous bytes per segment and one load
// instruction brings 1 KiB.  Groups 0,1 hold the segment's first 64-wide
// block and groups 2,3 the second; one v_permlane32_swap exchanges half of
// each lane's dwords with the lane 32 away so that every MFMA step draws from
// a single 64-wide block, which keeps the absmax scaling exact per block.
// Tokens feed the A operand (lane % 16 = token; lanes of tokens >= M are
// computed and discarded).
//
// Schedule.  Workgroups are persistent and take every G-th tile; the KW
// waves of a workgroup interleave each tile's segments, so together they read
// 64*KW contiguous bytes of a row at a time.  Per tile and slot a wave
// fetches the two block scales of each of the tile's 16 rows with one 8-byte
// load per lane, straight into the lanes that apply them.  A wave walks its
// work as
// (chunk of TB tiles) x (segment slot) x (tile in chunk), so the activation
// operand of a segment (read from L2 one slot ahead) serves TB tiles.
// Weight loads run one slot (TB units) ahead in a register ring and use
// buffer loads, whose hardware range check returns zeros past the end of a
// buffer, so the loop has no branches.  After each chunk every wave writes its
// fp32 partials to an LDS slot; after a barrier that leaves global loads in
// flight, wave 0 sums the KW partials in wave order (deterministic, no
// atomics) and stores bf16.
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

// Table entry e (a packed byte): x = (hi(cb[e & 15]), hi(cb[e >> 4])),
// y = (lo(cb[e & 15]), lo(cb[e >> 4])), low nibble = even k = low half.
__device__ __forceinline__ uint2 pair_table_entry(float c0, float c1) {
    const uint32_t h0 = f32_to_bf16_rne(c0), h1 = f32_to_bf16_rne(c1);
    const uint32_t l0 = f32_to_bf16_rne(c0 - __uint_as_float(h0 << 16));
    const uint32_t l1 = f32_to_bf16_rne(c1 - __uint_as_float(h1 << 16));
    return make_uint2(h0 | (h1 << 16), l0 | (l1 << 16));
}

// Offset (in k) of the 8 codes in dword t of lane group g's 16 bytes after
// the permlane32 swap.
__device__ __forceinline__ uint32_t k_offset(int g, int t) {
    return 32 * (g & 1) + 16 * (g >> 1) + 8 * (t & 1) + 64 * (t >> 1);
}

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

// SR: accumulator rows kept per lane (min(M, 4)); KW: waves per workgroup;
// TB: tiles per chunk (also the weight loads in flight per wave); NBUF:
// partial buffers (2 lets the next chunk's partials land while wave 0 reads).
template <int SR, int KW, int TB, int NBUF>
__global__ __launch_bounds__(64 * KW) void fused_mfma_kernel(
    const uint16_t *__restrict__ A, const uint8_t *__restrict__ Wp,
    const float *__restrict__ absmax, const float *__restrict__ codebook, int M, int N, int K,
    int bs_log2, int tiles, uint16_t *__restrict__ C) {
    __shared__ uint2 table[256 * 32];  // [byte][lane % 32]
    __shared__ float red[NBUF][KW][TB * SR][64];
    // Block scales of the current and the next slot for the chunk's TB*16
    // rows: 16 entries per row (the 16 64-wide blocks the KW = 8 waves cover
    // in one slot; a larger block is repeated over the entries it spans).
    // Rows are 18 floats apart so the 16 rows a wave reads at once fall in
    // distinct banks.
    constexpr int kScaleStride = 18;
    __shared__ float scl[2][TB * 16 * kScaleStride];
    static_assert(KW == 8 && 64 * KW == TB * 64, "one 16-byte scale load per thread per slot");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // The codebook is read first: loads complete in issue order, so the
    // table can be built while the first weight loads are still in flight.
    static_assert(64 * KW >= 256, "one table entry per thread");
    const int e_tab = tid & 255;
    const float cb0 = codebook[e_tab & 15], cb1 = codebook[e_tab >> 4];
    const char *tab_bytes = reinterpret_cast<const char *>(table);
    const uint32_t lane_off = (uint32_t)(lane & 31) * 8;

    const int j = lane & 15;
    const int g = lane >> 4;
    const int nseg = (K + 127) >> 7;
    const int spw = (nseg + KW - 1) / KW;  // segment slots per wave per tile
    const int G = gridDim.x;
    const int my_tiles = (tiles - (int)blockIdx.x + G - 1) / G;
    const int nchunks = (my_tiles + TB - 1) / TB;
    const uint32_t row_bytes = (uint32_t)K >> 1;
    const uint32_t nb = (uint32_t)K >> bs_log2;

    const __amdgpu_buffer_rsrc_t wres = make_rsrc(Wp, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t sres = make_rsrc(absmax, (uint32_t)N * nb * 4);
    const __amdgpu_buffer_rsrc_t ares = make_rsrc(A, (uint32_t)M * (uint32_t)K * 2);

    // Slot q of wave w is segment w + q*KW of every tile (the waves of a
    // workgroup read 64*KW contiguous bytes of each row at a time).  Byte
    // offsets advance incrementally in (chunk, slot, tile) order.
    const uint32_t w_tile_step = 16u * (uint32_t)G * row_bytes;
    const uint32_t w_lane = (uint32_t)wave * 64 + 16 * g;
    // Scales are staged through LDS one slot ahead: per slot the workgroup
    // needs the KW*128/bs consecutive block scales of each of its TB*16 rows
    // (64 bytes per row at bs = 64), which thread t fetches as 16-byte piece
    // t % 4 of chunk row t / 4, whole cache lines with no duplicates.
    const int s_row = tid >> 2;
    const uint32_t s_piece = (uint32_t)(tid & 3) * 16;
    const uint32_t s_win = (uint32_t)(KW * 128 * 4) >> bs_log2;  // bytes per row per slot

    // Issue cursor: the (chunk, slot) whose loads are issued next.  Byte
    // offsets advance incrementally in (chunk, slot) order.
    int ic = 0, iq = 0;
    uint32_t wo_q = 0, so_q = 0;
    auto chunk_base = [&](int c) {
        const uint32_t n0 = ((uint32_t)blockIdx.x + (uint32_t)(c * TB) * (uint32_t)G) * 16 + j;
        wo_q = n0 * row_bytes + w_lane;
        const uint32_t ns = ((uint32_t)blockIdx.x + (uint32_t)(c * TB + (s_row >> 4)) * (uint32_t)G) * 16 +
                            (uint32_t)(s_row & 15);
        so_q = ns * nb * 4;
    };
    auto advance = [&]() {
        if (++iq == spw) {
            iq = 0;
            chunk_base(++ic);
        } else {
            wo_q += 64u * KW;
        }
    };
    chunk_base(0);

    // Load ring: one weight register quad per tile.  The load of tile tr of
    // the next slot is issued as soon as tile tr of the current slot has been
    // decoded, so every wave keeps TB loads in flight at all times instead of
    // draining its queue once per slot.
    uint4 wbuf[TB];
    auto issue_tile = [&](int tr) {
        const uint32_t wo = wo_q + tr * w_tile_step;
        wbuf[tr] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wres, (int)wo, 0, 0));
    };
    // This thread's piece of the scales of the cursor's slot; pieces past the
    // slot's window or past the end of the row read zeros.
    auto load_scales = [&]() -> floatx4 {
        const uint32_t w0 = ((uint32_t)iq * KW * 128 >> bs_log2) * 4;  // window start in the row
        const bool live = s_piece < s_win && w0 + s_piece < nb * 4;
        const uint32_t so = live ? so_q + w0 + s_piece : kPastEnd;
        return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(sres, (int)so, 0, 0));
    };
    // Writes a piece into the staging buffer, repeating each scale over the
    // 64-wide entries its block spans.
    auto stage_scales = [&](const floatx4 &v, int buf) {
        float *row = &scl[buf][s_row * kScaleStride];
        const int e = (int)s_piece >> 2;  // first block of the piece in the window
        if (bs_log2 == 6) {
            *reinterpret_cast<floatx2 *>(row + e) = floatx2{v[0], v[1]};
            *reinterpret_cast<floatx2 *>(row + e + 2) = floatx2{v[2], v[3]};
        } else if (bs_log2 == 7) {
            if (e < 8) {
#pragma unroll
                for (int i = 0; i < 4; ++i) *reinterpret_cast<floatx2 *>(row + 2 * (e + i)) = floatx2{v[i], v[i]};
            }
        } else if (e < 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                *reinterpret_cast<floatx2 *>(row + 4 * (e + i)) = floatx2{v[i], v[i]};
                *reinterpret_cast<floatx2 *>(row + 4 * (e + i) + 2) = floatx2{v[i], v[i]};
            }
        }
    };

    // Activation operand of slot q: token j's 8 activations for each of the
    // lane's 4 dwords of codes.  Rows of tokens >= M lie past the end of A,
    // and k >= K (a ragged last segment, or a slot past the last segment)
    // takes an offset past every buffer: both read zeros without touching
    // memory, which cancels whatever codes sit there.
    const uint32_t a_row = (uint32_t)j * (uint32_t)K * 2;  // past the end of A for j >= M
    uint4 anext[4];
    auto load_a = [&](int q) {
        const uint32_t kk = ((uint32_t)wave + (uint32_t)q * KW) * 128;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t k = kk + k_offset(g, t);
            const uint32_t off = k < (uint32_t)K ? a_row + k * 2 : kPastEnd;
            anext[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, (int)off, 0, 0));
        }
    };

    {
        const floatx4 s0 = load_scales();
        load_a(0);
#pragma unroll
        for (int tr = 0; tr < TB; ++tr) issue_tile(tr);
        advance();
        if (tid < 256) {
            const uint2 v = pair_table_entry(cb0, cb1);
#pragma unroll 8
            for (int c = 0; c < 32; ++c) table[e_tab * 32 + c] = v;
        }
        stage_scales(s0, 0);
        lds_barrier();
    }
    int qs = 0;  // slots done, for the staging buffer parity

    // Table lookups of one tile: 16 packed bytes -> 32 bf16 hi/lo pairs.
    auto decode = [&](const uint4 &wv, uint2 (&ev)[16]) {
        uint32_t x[4] = {wv.x, wv.y, wv.z, wv.w};
        // lanes 0-31 keep dwords 0,1 and take dwords 0,1 of lane+32;
        // lanes 32-63 take dwords 2,3 of lane-32 and keep dwords 2,3
        const auto s02 = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
        x[0] = s02[0]; x[2] = s02[1];
        x[1] = s13[0]; x[3] = s13[1];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            // address = byte * 256 + lane_off: byte 1 from the packed
            // dword, byte 0 from lane_off, bytes 2-3 zero
            const uint32_t addr = __builtin_amdgcn_perm(x[i >> 2], lane_off, 0x0c0c0000u | ((4 + (i & 3)) << 8));
            ev[i] = *reinterpret_cast<const uint2 *>(tab_bytes + addr);
        }
    };

    const floatx4 zerof = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nchunks; ++c) {
        float acc[TB][SR];
#pragma unroll
        for (int tr = 0; tr < TB; ++tr)
#pragma unroll
            for (int r = 0; r < SR; ++r) acc[tr][r] = 0.f;

        for (int q = 0; q < spw; ++q) {
            // Activation operand, each pair of activations duplicated.  Built
            // once per slot and pinned in registers: an MFMA whose operand a
            // VALU instruction has just written stalls for the hazard, so the
            // compiler must not rebuild these next to every MFMA.
            uint4 adup[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                adup[2 * t] = make_uint4(anext[t].x, anext[t].x, anext[t].y, anext[t].y);
                adup[2 * t + 1] = make_uint4(anext[t].z, anext[t].z, anext[t].w, anext[t].w);
            }
#pragma unroll
            for (int s = 0; s < 8; ++s)
                __asm__ volatile("" : "+v"(adup[s].x), "+v"(adup[s].y), "+v"(adup[s].z), "+v"(adup[s].w));
            load_a(iq);  // the activations and scales of the slot issued next
            const floatx4 snext = load_scales();
            const float *sc = &scl[qs & 1][j * kScaleStride + 2 * wave];

            // Decode is software-pipelined one tile ahead: the 16 table reads
            // of tile tr+1 are in flight while the MFMAs of tile tr run.  Each
            // tile's ring entry is refilled with the next slot's loads right
            // after its decode.
            uint2 e[2][16];
            float am[2][2];
            decode(wbuf[0], e[0]);
            {
                const floatx2 a2 = *reinterpret_cast<const floatx2 *>(sc);
                am[0][0] = a2[0];
                am[0][1] = a2[1];
            }
            issue_tile(0);
#pragma unroll
            for (int tr = 0; tr < TB; ++tr) {
                // Per tile: its MFMAs, then the next tile's decode and loads
                // (VALU, LDS and memory work that runs under the matrix
                // cores), then the scale FMAs that consume the MFMA results.
                // Tiles past the end of a partial last chunk are computed too
                // (their loads read zeros past the buffer end and their
                // outputs are never stored), which keeps this loop one block.
                const uint2 *ev = e[tr & 1];
                // two independent chains, one per 64-wide block
                floatx4 D0 = zerof, D1 = zerof;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint4 b0 = make_uint4(ev[2 * s].x, ev[2 * s].y, ev[2 * s + 1].x, ev[2 * s + 1].y);
                    const uint4 b1 = make_uint4(ev[8 + 2 * s].x, ev[8 + 2 * s].y, ev[9 + 2 * s].x, ev[9 + 2 * s].y);
                    D0 = mfma_bf16_16x16x32(as_bf16x8(adup[s]), as_bf16x8(b0), D0);
                    D1 = mfma_bf16_16x16x32(as_bf16x8(adup[4 + s]), as_bf16x8(b1), D1);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (tr + 1 < TB) {
                    decode(wbuf[tr + 1], e[(tr + 1) & 1]);
                    const floatx2 a2 = *reinterpret_cast<const floatx2 *>(sc + (tr + 1) * 16 * kScaleStride);
                    am[(tr + 1) & 1][0] = a2[0];
                    am[(tr + 1) & 1][1] = a2[1];
                    issue_tile(tr + 1);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < SR; ++r)
                    acc[tr][r] = fmaf(am[tr & 1][1], D1[r], fmaf(am[tr & 1][0], D0[r], acc[tr][r]));
            }
            advance();
            // Publish the next slot's scales.  The buffer written here was
            // last read in the previous slot, which every wave finished before
            // the previous barrier.
            stage_scales(snext, (qs + 1) & 1);
            lds_barrier();
            ++qs;
        }

        // combine the KW partials of this chunk's tiles
        const int buf = NBUF == 2 ? (c & 1) : 0;
#pragma unroll
        for (int tr = 0; tr < TB; ++tr)
#pragma unroll
            for (int r = 0; r < SR; ++r) red[buf][wave][tr * SR + r][lane] = acc[tr][r];
        lds_barrier();
        if (wave == 0) {
#pragma unroll
            for (int tr = 0; tr < TB; ++tr) {
                const int n = ((int)blockIdx.x + (c * TB + tr) * G) * 16 + j;
#pragma unroll
                for (int r = 0; r < SR; ++r) {
                    float v = red[buf][0][tr * SR + r][lane];
                    for (int w2 = 1; w2 < KW; ++w2) v += red[buf][w2][tr * SR + r][lane];
                    const int tok = 4 * g + r;
                    if (n < N && tok < M) C[(size_t)tok * N + n] = (uint16_t)f32_to_bf16_rne(v);
                }
            }
        }
        if constexpr (NBUF == 1) lds_barrier();
    }
}

template <int SR, int KW, int TB, int NBUF>
hipError_t launch_cfg(const uint16_t *A, const uint8_t *Wp, const float *absmax,
                      const float *codebook, int M, int N, int K, int bs_log2, uint16_t *C,
                      int wg_per_cu, hipStream_t s) {
    const int tiles = (N + 15) / 16;
    const DeviceInfo info = device_info();
    int G = info.num_cus * wg_per_cu;
    if (G > tiles) G = tiles;
    fused_mfma_kernel<SR, KW, TB, NBUF><<<dim3(G), dim3(64 * KW), 0, s>>>(
        A, Wp, absmax, codebook, M, N, K, bs_log2, tiles, C);
    return hipGetLastError();
}

template <int SR>
hipError_t launch_sr(const uint16_t *A, const uint8_t *Wp, const float *absmax,
                     const float *codebook, int M, int N, int K, int bs_log2, uint16_t *C,
                     hipStream_t s) {
    // One 8-wave workgroup per CU (the replicated table takes 64 KiB of LDS),
    // 8 tiles per chunk so each wave keeps 8 KiB of weights in flight; for
    // more than two tokens the partial tiles share a single buffer.
    constexpr int NBUF = SR <= 2 ? 2 : 1;
    return launch_cfg<SR, 8, 8, NBUF>(A, Wp, absmax, codebook, M, N, K, bs_log2, C, 1, s);
}

}  // namespace

// The kernel's byte offsets are 32-bit.  The weight offsets run up to two
// chunks of every workgroup past the last tile (at most 2 * 4 * 1024 tiles of
// 16 rows on a 256-CU part), so the matrix plus that margin must stay below
// 4 GiB; activation offsets reach 16 rows of K (the lanes of absent tokens
// read past the end of A), which must stay below 4 GiB as well.
bool q4_fused_mfma_fits(int M, int N, int K) {
    (void)M;
    const uint64_t margin_rows = 2ull * 4 * 1024 * 16;
    return ((uint64_t)N + margin_rows) * (uint64_t)K / 2 < (1ull << 32) &&
           16ull * (uint64_t)K * 2 < (1ull << 32);
}

hipError_t launch_q4_fused_mfma(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                                const float *codebook, int M, int N, int K, int bs_log2,
                                uint16_t *C, hipStream_t s) {
    if (M <= 1) return launch_sr<1>(A, Wpacked, absmax, codebook, M, N, K, bs_log2, C, s);
    if (M <= 2) return launch_sr<2>(A, Wpacked, absmax, codebook, M, N, K, bs_log2, C, s);
    return launch_sr<4>(A, Wpacked, absmax, codebook, M, N, K, bs_log2, C, s);
}

hipError_t launch_q4_fused(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                           const float *codebook, int M, int N, int K, int bs_log2,
                           uint16_t *C, hipStream_t s) {
    if (bs_log2 >= 6 && q4_fused_mfma_fits(M, N, K))
        return launch_q4_fused_mfma(A, Wpacked, absmax, codebook, M, N, K, bs_log2, C, s);
    return launch_q4_fused_simt(A, Wpacked, absmax, codebook, M, N, K, bs_log2, C, s);
}

}  // namespace q4
