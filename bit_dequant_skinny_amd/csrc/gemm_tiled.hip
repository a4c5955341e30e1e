// Tiled bf16 GEMM on the matrix cores for the split path at larger M:
// C[M,N] = A[M,K] * W[N,K]^T (+ bias), fp32 accumulation.
//
// The GEMM half of the split path (dequantize to bf16, then GEMM) of the
// bitsandbytes pull request "[ROCm] Optimize kgemm_4bit_inference_naive for
// ROCm, use it for batch sizes other than 1" (section "Fused path support for
// M > 1"), for token counts where the weights must be reused from on-chip
// memory instead of streamed once per 16-row slab.
//
// A workgroup of 4 waves computes a 128 x 128 tile of C (tokens x features),
// each wave a 64 x 64 quarter as 4 x 4 v_mfma_f32_16x16x32_bf16 tiles.  K is
// walked in steps of 64: the next step's A and W tiles (16 KiB each) are
// loaded into registers while the current step's tiles are multiplied from
// LDS, then written to the other half of a double-buffered LDS stage.  LDS
// rows are 64 bf16 plus 16 bytes of padding (144 bytes), so the 16 rows a
// quarter-wave reads with ds_read_b128 fall in distinct banks.  Loads are
// buffer loads whose range check returns zeros past the end of A or W (rows
// past M or N); k past K is masked per 16-byte piece (K % 8 == 0).  The grid
// runs the token blocks of one feature block next to each other, so a W tile
// is fetched from HBM once and the other token blocks find it in L2.  When
// there are too few tiles to give every CU two workgroups, K is split into up
// to 4 parts whose fp32 partial outputs a separate pass sums in part order.
#include "device.h"
#include "launch.h"

namespace q4 {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kRowBytes = BK * 2 + 16;
constexpr int kTileBytes = BM * kRowBytes;
constexpr uint32_t kPastEnd = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

__global__ __launch_bounds__(kThreads, 2) void gemm_tiled_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ W,
    const void *__restrict__ bias, int M, int N, int K, int m_blocks, int mn_blocks,
    int k_steps, void *__restrict__ C, int c_dt) {
    __shared__ __attribute__((aligned(16))) char lds[2][2][kTileBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // Block b: token block b % m_blocks, feature block (b % mn_blocks) /
    // m_blocks, and K part b / mn_blocks (k_steps steps of 64 from
    // part * k_steps); part p writes its own fp32 output slab C + p*M*N.
    const uint32_t blk = blockIdx.x % (uint32_t)mn_blocks;
    const int part = (int)(blockIdx.x / (uint32_t)mn_blocks);
    const int m0 = (int)(blk % (uint32_t)m_blocks) * BM;
    const int n0 = (int)(blk / (uint32_t)m_blocks) * BN;
    const int kt0 = part * k_steps;
    const int j = lane & 15, g = lane >> 4;

    const __amdgpu_buffer_rsrc_t ares = make_rsrc(A, (uint32_t)M * (uint32_t)K * 2);
    const __amdgpu_buffer_rsrc_t wres = make_rsrc(W, (uint32_t)N * (uint32_t)K * 2);
    // Global -> LDS mapping: thread t moves the 16-byte piece t % 8 of rows
    // t / 8 + 32r (r < 4) of each tile.
    const int lrow = tid >> 3, lcol = tid & 7;
    auto gload = [&](int k0, uint4 (&ra)[4], uint4 (&rw)[4]) {
        const uint32_t k = (uint32_t)(k0 + lcol * 8);
        const bool kin = k < (uint32_t)K;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t row = (uint32_t)(lrow + 32 * r);
            const uint32_t oa = kin && m0 + row < (uint32_t)M ? ((m0 + row) * (uint32_t)K + k) * 2 : kPastEnd;
            const uint32_t ow = kin && n0 + row < (uint32_t)N ? ((n0 + row) * (uint32_t)K + k) * 2 : kPastEnd;
            ra[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ares, (int)oa, 0, 0));
            rw[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wres, (int)ow, 0, 0));
        }
    };
    auto lstore = [&](int buf, const uint4 (&ra)[4], const uint4 (&rw)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int off = (lrow + 32 * r) * kRowBytes + lcol * 16;
            *reinterpret_cast<uint4 *>(&lds[buf][0][off]) = ra[r];
            *reinterpret_cast<uint4 *>(&lds[buf][1][off]) = rw[r];
        }
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nk_all = (K + BK - 1) / BK;
    const int nk = nk_all - kt0 < k_steps ? nk_all - kt0 : k_steps;
    if (part > 0) C = static_cast<char *>(C) + (size_t)part * (size_t)M * (size_t)N * 4;
    uint4 ra[4], rw[4];
    gload(kt0 * BK, ra, rw);
    lstore(0, ra, rw);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt0 + kt + 1) * BK, ra, rw);
        const char *as = lds[cur][0];
        const char *ws = lds[cur][1];
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int kb = (ks * 32 + g * 8) * 2;
            uint4 af[4], bf[4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
                af[a] = *reinterpret_cast<const uint4 *>(as + (wm * 64 + a * 16 + j) * kRowBytes + kb);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                bf[b] = *reinterpret_cast<const uint4 *>(ws + (wn * 64 + b * 16 + j) * kRowBytes + kb);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = mfma_bf16_16x16x32(as_bf16x8(af[a]), as_bf16x8(bf[b]), acc[a][b]);
        }
        if (kt + 1 < nk) lstore(cur ^ 1, ra, rw);
        __syncthreads();
    }

    // D layout: lane holds feature j of each 16-wide block and tokens 4g + r.
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int n = n0 + wn * 64 + b * 16 + j;
        if (n >= N) continue;
        const float bv = bias ? load_elem(bias, n, c_dt) : 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = m0 + wm * 64 + a * 16 + 4 * g + r;
                if (tok < M) store_elem(C, (size_t)tok * N + n, acc[a][b][r] + bv, c_dt);
            }
    }
}

}  // namespace

// 32-bit byte offsets: A and W must each stay below 2 GiB.
bool gemm_tiled_fits(int M, int N, int K) {
    return (uint64_t)M * (uint64_t)K * 2 < (1ull << 31) && (uint64_t)N * (uint64_t)K * 2 < (1ull << 31);
}

int gemm_tiled_ksplit(int M, int N, int K) {
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int want = 2 * device_info().num_cus;  // two workgroups per CU
    const int nk = (K + BK - 1) / BK;
    int ks = 1;
    while (ks < 4 && tiles * ks < want && nk >= 4 * (ks + 1)) ++ks;
    return ks;
}

hipError_t launch_gemm_tiled(const uint16_t *A, const uint16_t *W, const void *bias, int M,
                             int N, int K, int ksplit, void *C, int c_dt, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    if (ksplit < 1 || (ksplit > 1 && (bias || c_dt != kF32))) return hipErrorInvalidValue;
    const int m_blocks = (M + BM - 1) / BM;
    const int n_blocks = (N + BN - 1) / BN;
    const int nk = (K + BK - 1) / BK;
    const int k_steps = (nk + ksplit - 1) / ksplit;
    gemm_tiled_kernel<<<dim3((unsigned)(m_blocks * n_blocks * ksplit)), dim3(kThreads), 0, s>>>(
        A, W, bias, M, N, K, m_blocks, m_blocks * n_blocks, k_steps, C, c_dt);
    return hipGetLastError();
}

}  // namespace q4
