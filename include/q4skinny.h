/*
 * q4skinny: small-batch weight-streaming GEMMs of LLM decode on MI355X (gfx950).
 *
 * C ABI.  Callers need neither HIP nor torch headers: device buffers are
 * passed as plain pointers, a HIP stream as `void *` (NULL = the default
 * stream), sizes as int.
 *
 * Notation: M = token rows of A and C, N = output features (rows of W),
 * K = reduction length.  Every matrix is row-major and contiguous.  The
 * product is the "TN" inference layout C[M,N] = A[M,K] * W[N,K]^T named in
 * the maintainer's comment on the bitsandbytes pull request "[ROCm] Optimize
 * kgemm_4bit_inference_naive for ROCm, use it for batch sizes other than 1".
 *
 * Common conventions
 *  - Pointers are device pointers owned by the caller; the library never
 *    frees them.  Outputs must not alias inputs.
 *  - Calls are asynchronous: they enqueue work on `stream` and return.
 *  - Arguments are validated before anything is launched.  On any error
 *    status nothing has been launched and the outputs are untouched.
 *  - Empty shapes (M == 0 or N == 0) return Q4_OK and launch nothing.
 *  - A HIP launch failure returns Q4_ERR_HIP; the sticky HIP error is read
 *    and cleared with hipGetLastError() so that the next call starts clean.
 *  - q4_last_error() returns a message for the last failing call on the
 *    calling thread (empty after a successful call).
 *  - Results are deterministic: the same inputs, shape and path give
 *    bit-identical outputs (no atomics; fixed reduction orders).
 *  - Thread safety: every entry point may be called from several threads;
 *    the crossover setter changes a process-wide value.
 */
#ifndef Q4SKINNY_H
#define Q4SKINNY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum q4_status {
    Q4_OK = 0,
    Q4_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, negative size, misalignment, K not a multiple */
    Q4_ERR_UNSUPPORTED = 2,      /* a legal request this library has no kernel for */
    Q4_ERR_HIP = 3               /* the HIP runtime reported an error (see q4_last_error) */
} q4_status;

/* Element types: bfloat16, IEEE binary32, IEEE binary16. */
enum { Q4_DTYPE_BF16 = 0, Q4_DTYPE_FP32 = 1, Q4_DTYPE_FP16 = 2 };
enum { Q4_PATH_AUTO = 0, Q4_PATH_FUSED = 1, Q4_PATH_SPLIT = 2 };

/* Token rows one pass of the skinny fused kernels handles.  Where the tiled
 * kernel cannot run (blocksize 32, shapes beyond its 32-bit offsets), the
 * fused path runs larger M in passes over slabs of this many rows, each pass
 * streaming the packed weights again (as launches of 16 rows for other
 * element types than bf16, blocksize 32 and matrices of more than 2048 * 16
 * rows per 256 CUs). */
#define Q4_FUSED_PASS_M 32
/* Largest crossover value q4_set_crossover_m accepts. */
#define Q4_CROSSOVER_MAX 65536

/*
 * q4_gemm_skinny: C = A * dequant(W)^T with W blockwise 4-bit quantized.
 *
 * Defined by the bitsandbytes pull request "[ROCm] Optimize
 * kgemm_4bit_inference_naive for ROCm, use it for batch sizes other than 1"
 * (sections "Technical details" and "Fused path support for M > 1"): a fused
 * dequantize + matmul for small multi-row inputs, falling back to dequantize
 * + GEMM above a per-GPU crossover M.
 *
 *  A        bf16 [M, K]   activations.
 *  Wpacked  uint8 [N, K/2] two 4-bit codes per byte; byte j of a row holds
 *           k = 2j in its low nibble and k = 2j + 1 in its high nibble.
 *  absmax   fp32 [N, K/blocksize]  one scale per block of `blocksize`
 *           consecutive k inside a row.
 *  codebook fp32 [16]     the value of each code (device memory).
 *  C        bf16 [M, N]   output, round-to-nearest-even of the fp32 result.
 *
 *  The weight of element (n, k) is codebook[code] * absmax[n, k / blocksize]
 *  (an fp32 product); products with A accumulate in fp32.
 *
 *  Q4_ERR_INVALID_ARGUMENT: NULL A/Wpacked/absmax/codebook/C, M/N/K < 0,
 *    K == 0, blocksize <= 0 or odd, K % blocksize != 0, A, Wpacked or absmax
 *    not 16-byte aligned, codebook not 4-byte aligned, C not 2-byte aligned.
 *  Q4_ERR_UNSUPPORTED: blocksize not in {32, 64, 128, 256}; M or N above
 *    2^30/K-sized limits (N * K / 2 must fit in 2^40 bytes).
 *  Which kernel runs: M <= the crossover (q4_get_crossover_shape(N, K)) take
 *  the fused path: up to 32 rows (16 on shapes of more than 2048 weight rows
 *  per CU) the skinny matrix-core kernel, above that the tiled matrix-core
 *  kernel (output tiles of 64 tokens x 64 or 256 features, K split over
 *  workgroups into fp32 partials in the workspace when its tiles cannot
 *  fill the GPU).  Blocksize 32 (and shapes beyond the kernels' 32-bit
 *  offsets) take the vector-ALU kernel in passes of Q4_FUSED_PASS_M rows.
 *  Other M take the split path (dequantize to bf16 into a library-owned
 *  workspace of N*K*2 bytes, then an MFMA bf16 GEMM).
 */
q4_status q4_gemm_skinny(const void *A, const uint8_t *Wpacked, const float *absmax,
                         const float *codebook, int M, int N, int K, int blocksize,
                         void *C, void *stream);

/*
 * q4_gemm_skinny_path: q4_gemm_skinny with the path forced (Q4_PATH_AUTO,
 * Q4_PATH_FUSED or Q4_PATH_SPLIT).
 *
 * The two paths are those the bitsandbytes pull request "[ROCm] Optimize
 * kgemm_4bit_inference_naive for ROCm, use it for batch sizes other than 1"
 * times against each other (section "Fused path support for M > 1" and its
 * split-versus-fused table): the fused dequantize + GEMM kernel, and the split
 * dequantize-to-bf16 then GEMM.  Forcing one is how the crossover is measured
 * and how the tests reach both.  Arguments, outputs and errors are those of
 * q4_gemm_skinny; an unknown path value is Q4_ERR_INVALID_ARGUMENT.
 */
q4_status q4_gemm_skinny_path(const void *A, const uint8_t *Wpacked, const float *absmax,
                              const float *codebook, int M, int N, int K, int blocksize,
                              void *C, void *stream, int path);

/*
 * q4_gemm_skinny_ex: q4_gemm_skinny with a bias and other element types.
 *
 * Defined by the maintainer's comment on the bitsandbytes pull request
 * "[ROCm] Optimize kgemm_4bit_inference_naive for ROCm, use it for batch
 * sizes other than 1", which lists a fused bias epilogue (C += bias) and
 * fp32 / fp16 / bf16 variants that all accumulate in fp32.
 *
 *  A        [M, K] of a_dtype (Q4_DTYPE_BF16, Q4_DTYPE_FP16 or Q4_DTYPE_FP32).
 *  Wpacked, absmax, codebook: as in q4_gemm_skinny.
 *  bias     [N] of c_dtype, or NULL.
 *  C        [M, N] of c_dtype (Q4_DTYPE_BF16, Q4_DTYPE_FP16 or Q4_DTYPE_FP32).
 *  path     Q4_PATH_AUTO, Q4_PATH_FUSED or Q4_PATH_SPLIT, as in
 *           q4_gemm_skinny_path.
 *
 *  C[m, n] = round_c(sum_k a[m, k] * w(n, k) + bias[n]): the products are
 *  exact, the sum is fp32, the bias is added to the fp32 sum and the result
 *  is rounded once to c_dtype (nearest even).  fp16 and fp32 activations are
 *  exact in the kernels (fp16 as an exact bf16 hi + lo pair on the matrix
 *  cores, fp32 on the vector ALUs).  The split path rounds the weights to
 *  bf16 first, as q4_gemm_skinny does.
 *
 *  Q4_ERR_INVALID_ARGUMENT: as q4_gemm_skinny, plus an unknown dtype or
 *    path, C or bias not aligned to their element size.
 *  Q4_ERR_UNSUPPORTED: as q4_gemm_skinny; fp32 activations on the split
 *    path (above the crossover, or forced).
 */
q4_status q4_gemm_skinny_ex(const void *A, int a_dtype, const uint8_t *Wpacked,
                            const float *absmax, const float *codebook, const void *bias, int M,
                            int N, int K, int blocksize, void *C, int c_dtype, void *stream,
                            int path);

/*
 * q4_gemm_skinny_ex_noalloc: q4_gemm_skinny_ex that allocates nothing.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Arguments,
 * results (bit for bit), dispatch and errors are those of q4_gemm_skinny_ex,
 * except that the scratch some paths need (the bf16 weights of the split
 * path, the activation planes of fp16 / fp32 inputs, the fp32 partial
 * outputs of K splits) comes from a fixed device array of
 * Q4_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends, instead of the per-stream workspace.
 *  - A call whose path needs more scratch than that returns
 *    Q4_ERR_UNSUPPORTED (nothing launched); q4_gemm_skinny_ex has no limit.
 *  - No hipMalloc / hipFree / allocating library call is made, so the call
 *    can be captured into a HIP graph from its first use.
 *  - Every call on a device shares that device's array: calls that overlap
 *    on one device (different streams or threads) race; serialise them.
 *    Each call writes the scratch it reads, so nothing carries over.
 *  - The array's device address is looked up once per device, at the
 *    device's first call (Q4_ERR_HIP if that lookup fails).
 */
#define Q4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
q4_status q4_gemm_skinny_ex_noalloc(const void *A, int a_dtype, const uint8_t *Wpacked,
                                    const float *absmax, const float *codebook, const void *bias,
                                    int M, int N, int K, int blocksize, void *C, int c_dtype,
                                    void *stream, int path);

/*
 * The tile layout of the packed weights.
 *
 * The same bytes as the row-major Wpacked [N, K/2], reordered so that the
 * 16 rows x 64 bytes a wave's matrix-core lanes decode together for one
 * 128-wide segment of K are 1 KiB of contiguous memory.  This is the
 * "packed-weight layout" part that the bitsandbytes pull request "[ROCm]
 * Optimize kgemm_4bit_inference_naive ..." leaves to the kernel (its kernel
 * reads whole packed rows with 128-bit loads, section on the kernel's
 * optimizations); the arrangement below is this library's.
 *
 *   Tile t = rows 16t .. 16t+15; segment s = bytes 64s .. 64s+63 of a row
 *   (k = 128s .. 128s+127), cut into quarters of 8 bytes (quarter c = bytes
 *   64s + 8c .. +8, k = 128s + 16c .. +16).  Unit (t, s) is the 1024 bytes at
 *   offset (t * K/128 + s) * 1024; its 16-byte piece l (l = 0..63) holds
 *   quarter a then quarter a + 4 of row 16t + l % 16, with a = 0, 2, 1, 3
 *   for l / 16 = 0, 1, 2, 3: 16 weights of each 64-wide half of the segment,
 *   the order in which matrix-core lane l consumes them.
 *
 * Within a quarter the bytes, nibble order and codes are those of the
 * row-major layout, and absmax keeps its row-major [N, K/blocksize] layout.
 * Requires N % 16 == 0, K % 128 == 0 and N*K/2 below 4 GiB.  Reading each
 * tile as one contiguous run gives the DRAM longer bursts than 64-byte
 * pieces of 16 rows 4 KiB or more apart (a read-only pattern test on MI355X:
 * 22.2 against 24.4 us for 117 MB), and the piece order lets each lane of the
 * skinny kernel load its 16 bytes with one 128-bit load.
 */

/*
 * q4_repack_tiles: Wtiles = the tile layout of the row-major Wpacked.
 *
 *  Wpacked  uint8 [N, K/2] (device), Wtiles uint8 [N*K/2] (device), both
 *           16-byte aligned and not overlapping.  A pure byte permutation,
 *           bit-exact.
 *
 *  Q4_ERR_INVALID_ARGUMENT: NULL pointer, N/K < 0, K == 0, N % 16 != 0,
 *    K % 128 != 0, misalignment, overlapping buffers.
 *  Q4_ERR_UNSUPPORTED: N*K/2 >= 4 GiB.
 */
q4_status q4_repack_tiles(const uint8_t *Wpacked, uint8_t *Wtiles, int N, int K, void *stream);

/*
 * q4_gemm_skinny_tiles: q4_gemm_skinny_ex over weights in the tile layout.
 *
 * Arguments, dispatch (fused kernels up to the crossover, split path above)
 * and results are those of q4_gemm_skinny_ex on the row-major weights the
 * tiles were made from.  Above 32 token rows and on the split path the
 * outputs are bit-identical to it (every kernel sees the same bytes in the
 * same registers and sums in the same order); up to 32 rows the skinny
 * kernel walks K from the first segment over tiles but from a rotated
 * segment per workgroup over rows (which spreads row-major loads over the
 * DRAM channels), so the fp32 sums of the same products may round
 * differently; both meet the same tolerance and each is deterministic.
 *
 *  Q4_ERR_INVALID_ARGUMENT: as q4_gemm_skinny_ex, plus N % 16 != 0 or
 *    K % 128 != 0.
 *  Q4_ERR_UNSUPPORTED: as q4_gemm_skinny_ex, plus blocksize 32 (whose
 *    vector-ALU kernel reads rows) and N*K/2 beyond the matrix-core kernels'
 *    32-bit offsets.
 */
q4_status q4_gemm_skinny_tiles(const void *A, int a_dtype, const uint8_t *Wtiles,
                               const float *absmax, const float *codebook, const void *bias,
                               int M, int N, int K, int blocksize, void *C, int c_dtype,
                               void *stream, int path);

/*
 * bf16_gemm_skinny: C = A * W^T (+ bias) for unquantized bf16 weights.
 *
 * Defined by the report on vLLM pull request 40687 "Support N=5 in wvSplitK
 * skinny GEMM kernels for speculative decoding" (section "关键源码片段"): the
 * skinny bf16 GEMM serves 1..5 token rows (one token plus four draft tokens
 * of speculative-decode verification), needs K % 8 == 0, takes an optional
 * bias and rejects token counts it has no kernel for.  (That page calls the
 * token count n and the output features m; here they are M and N.)
 *
 *  A    bf16 [M, K], W bf16 [N, K], bias bf16 [N] or NULL, C bf16 [M, N].
 *  Accumulates in fp32; the bias is added to the fp32 sum before the single
 *  rounding to bf16.
 *
 *  Q4_ERR_INVALID_ARGUMENT: NULL A/W/C, M/N/K < 0, K == 0, K % 8 != 0,
 *    A or W not 16-byte aligned, C or bias not 2-byte aligned.
 *  Q4_ERR_UNSUPPORTED: M > 5.
 */
q4_status bf16_gemm_skinny(const void *A, const void *W, const void *bias, int M, int N,
                           int K, void *C, void *stream);

/*
 * Tile layout of bf16 weights (a layout of this library; the GEMM of the
 * report on vLLM pull request 40687, section "关键源码片段", reads W [N, K]
 * row-major, which bf16_gemm_skinny keeps).  Rows form tiles of 16 (tile t =
 * rows 16t..16t+15) and a row's elements form steps of 32 (step s = k
 * 32s..32s+31: the k one matrix-core instruction consumes).  The 16 x 32
 * elements of (t, s) are one 1 KiB unit at element (t * K/32 + s) * 512;
 * piece l = 0..63 of a unit (8 elements) holds k = 32s + 8*(l/16) .. +7 of
 * row 16t + l % 16, the 16 bytes matrix-core lane l takes for that step.
 * Each load instruction then reads 1 KiB of contiguous memory in operand
 * order, with no reordering pass (the row-major call reorders its loads
 * through LDS; on MI355X the tile layout is 3-9 % faster on the K = 2560
 * shapes).  Requires N % 16 == 0, K % 32 == 0 and (N + 64)*K*2 below 2 GiB.
 */

/*
 * bf16_repack_tiles: Wtiles = the tile layout of the row-major bf16 W.
 *
 *  W bf16 [N, K] (device), Wtiles bf16 [N*K] (device), both 16-byte aligned
 *  and not overlapping.  A pure permutation of 16-byte pieces, bit-exact.
 *
 *  Q4_ERR_INVALID_ARGUMENT: NULL pointer, N/K < 0, K == 0, N % 16 != 0,
 *    K % 32 != 0, misalignment, overlapping buffers.
 *  Q4_ERR_UNSUPPORTED: (N + 64)*K*2 >= 2 GiB.
 */
q4_status bf16_repack_tiles(const void *W, void *Wtiles, int N, int K, void *stream);

/*
 * bf16_gemm_skinny_tiles: bf16_gemm_skinny over weights in the tile layout.
 * Arguments and results are those of bf16_gemm_skinny on the row-major
 * weights the tiles were made from; the outputs are bit-identical to it
 * (each lane receives the same values and the sums run in the same order).
 *
 *  Q4_ERR_INVALID_ARGUMENT: as bf16_gemm_skinny, plus N % 16 != 0 or
 *    K % 32 != 0.
 *  Q4_ERR_UNSUPPORTED: as bf16_gemm_skinny, plus (N + 64)*K*2 >= 2 GiB.
 */
q4_status bf16_gemm_skinny_tiles(const void *A, const void *Wtiles, const void *bias, int M,
                                 int N, int K, void *C, void *stream);

/*
 * q4_dequant: out[n, k] = codebook[code(n, k)] * absmax[n, k / blocksize].
 *
 * The dequantize step of the split path in the bitsandbytes pull request
 * "[ROCm] Optimize kgemm_4bit_inference_naive ..." (section "Fused path
 * support for M > 1": "split dequantize + GEMM").  Same packed layout as
 * q4_gemm_skinny.  out_dtype Q4_DTYPE_FP32 writes the fp32 product,
 * Q4_DTYPE_BF16 and Q4_DTYPE_FP16 write it rounded once to bf16 or fp16
 * (nearest-even; NaN stays NaN; fp16 overflows to infinity).
 * Bit-exact: one fp32 multiply per element, denormals kept.
 *
 *  Q4_ERR_INVALID_ARGUMENT: NULL pointer, N/K < 0, K == 0, bad blocksize
 *    (as above), out_dtype unknown, Wpacked/absmax/out not 16-byte aligned,
 *    codebook not 4-byte aligned.
 *  Q4_ERR_UNSUPPORTED: blocksize not in {32, 64, 128, 256}.
 */
q4_status q4_dequant(const uint8_t *Wpacked, const float *absmax, const float *codebook,
                     int N, int K, int blocksize, void *out, int out_dtype, void *stream);

/*
 * q4_dequant_tiles: q4_dequant over weights in the tile layout; `out` is
 * row-major [N, K] and bit-identical to q4_dequant of the row-major weights.
 *  Errors: as q4_dequant, plus those of the tile layout in
 *  q4_gemm_skinny_tiles.
 */
q4_status q4_dequant_tiles(const uint8_t *Wtiles, const float *absmax, const float *codebook,
                           int N, int K, int blocksize, void *out, int out_dtype, void *stream);

/*
 * q4_quantize: blockwise 4-bit quantization, the inverse of q4_dequant.
 *
 * Produces the packed weights and block scales of the fused kernels: the
 * blockwise absmax quantization to a 16-entry NF4/FP4 table, blocksize 64 by
 * default, that the maintainer's comment on the bitsandbytes pull request
 * "[ROCm] Optimize kgemm_4bit_inference_naive ..." describes.  The pages do
 * not spell out the rounding; this library's reading:
 *   absmax[n, b] = max |W[n, k]| over the block (exact);
 *   code(n, k)   = the index of the codebook entry nearest to the exact ratio
 *                  W[n, k] / absmax[n, b], a tie going to the lower entry;
 *                  a block of zeros stores absmax 0 and the entry nearest 0.
 *
 *  W        [N, K] of w_dtype (Q4_DTYPE_BF16, Q4_DTYPE_FP16 or Q4_DTYPE_FP32),
 *           device memory, finite values.
 *  codebook fp32 [16] in HOST memory, strictly increasing (the thresholds
 *           between entries are derived on the host).
 *  Wpacked  uint8 [N, K/2] output, layout as in q4_gemm_skinny.
 *  absmax   fp32 [N, K/blocksize] output.
 *
 *  Q4_ERR_INVALID_ARGUMENT: NULL pointer, unknown w_dtype, N/K < 0, K == 0,
 *    K % blocksize != 0, blocksize <= 0 or odd, a codebook that is not finite
 *    and strictly increasing, W or Wpacked not 16-byte aligned, absmax not
 *    4-byte aligned.
 *  Q4_ERR_UNSUPPORTED: blocksize not in {32, 64, 128, 256}.
 */
q4_status q4_quantize(const void *W, int w_dtype, const float *codebook, int N, int K,
                      int blocksize, uint8_t *Wpacked, float *absmax, void *stream);

/*
 * q4_codebook_preset: writes a 16-entry table to host memory.  The pages name
 * NF4 and FP4 tables but print no values, so the presets follow rules of this
 * library:
 *  Q4_CODEBOOK_NF4_STYLE  8 positive entries at the standard-normal quantiles
 *    of 0.5 + (i/8)(0.97 - 0.5), i = 1..8, 7 negative entries at
 *    0.5 - (i/7)(0.97 - 0.5), i = 1..7, each side divided by its largest
 *    magnitude (so the extremes are exactly -1 and 1), plus 0; sorted.
 *  Q4_CODEBOOK_INT4       the uniform grid (i - 8) / 8, i = 0..15.
 * Both are strictly increasing and hold -1 and 0, so they suit q4_quantize.
 * Q4_ERR_INVALID_ARGUMENT for an unknown preset or a NULL pointer.
 */
enum { Q4_CODEBOOK_NF4_STYLE = 0, Q4_CODEBOOK_INT4 = 1 };
q4_status q4_codebook_preset(int which, float *codebook);

/*
 * Crossover control.  The fused-versus-split threshold (fused when
 * M <= crossover) of the bitsandbytes pull request "[ROCm] Optimize
 * kgemm_4bit_inference_naive ..." (section "Fused path support for M > 1":
 * the crossover M differs per GPU, and one threshold is chosen so that the
 * fused path is kept wherever it wins on the slowest-crossing GPU).  Here
 * it starts at the value measured on MI355X and compiled in, unless the
 * environment variable Q4_CROSSOVER_M holds an integer at the first call.
 *  q4_get_crossover_m  the process-wide value (shapes without an entry of
 *                      their own use it).
 *  q4_set_crossover_m  sets it; 0..Q4_CROSSOVER_MAX (0 = always split), else
 *                      Q4_ERR_INVALID_ARGUMENT and the value is unchanged.
 */
int q4_get_crossover_m(void);
q4_status q4_set_crossover_m(int m);

/*
 * Per-shape crossovers: the crossover can be set for one weight shape (N
 * rows, K columns), which then overrides the process-wide value for calls
 * with that shape; the pull request above tunes its threshold per GPU and
 * notes that the best switch point depends on the problem (section "Fused
 * path support for M > 1" and the crossover table), and measured per-shape
 * values on MI355X can be recorded here.  The table starts from the values
 * measured on MI355X for the decode layer shapes compiled into the library,
 * then the environment variable Q4_CROSSOVER_TABLE at first use:
 * comma-separated "N:K:m" items (malformed items are skipped).
 *  q4_set_crossover_shape   m in 0..Q4_CROSSOVER_MAX sets the entry, m < 0
 *                           removes it; Q4_ERR_INVALID_ARGUMENT for N <= 0,
 *                           K <= 0 or m > Q4_CROSSOVER_MAX.
 *  q4_get_crossover_shape   the crossover calls of shape (N, K) use: the
 *                           entry if present; else the smallest entry of
 *                           the shapes in the same bucket (K rounded up to
 *                           a power of two, and 16-row tiles per compute
 *                           unit in the class 1, 2, 3-4 or 5+), the exact-
 *                           then-bucket lookup of the bitsandbytes pull
 *                           request "Cache the hipBLASLt int8 matmul algo per
 *                           problem on ROCm"; else q4_get_crossover_m().
 *  q4_clear_crossover_shapes removes every entry, the measured ones
 *                           included (neither they nor the environment's
 *                           table are read again).
 * Thread-safe (one mutex); a change applies to calls made after it returns.
 */
q4_status q4_set_crossover_shape(int N, int K, int m);
int q4_get_crossover_shape(int N, int K);

/*
 * q4_skinny_kparts: how many parts the fused skinny kernel cuts K into for
 * M bf16 token rows (1..32) and an N x K weight on the current device (1 =
 * none; 1 for arguments outside those ranges, and for 17..32 rows where
 * they run as two 16-row passes).  The pages' kernel gives each
 * output row to one thread group over all of K (bitsandbytes pull request
 * "[ROCm] Optimize kgemm_4bit_inference_naive ...", section "Technical
 * details"); here a row's K may be split over workgroups when the 16-row
 * tiles alone would leave compute units idle (N = 5120: 320 tiles on 256
 * CUs) and the split saves enough of each workgroup's walk to pay for a
 * second launch: the parts' fp32 sums go to the per-stream workspace (or
 * the fixed scratch of the allocation-free entry point) and a second kernel
 * adds them in part order, adds the bias and rounds once (deterministic).
 */
int q4_skinny_kparts(int M, int N, int K);
q4_status q4_clear_crossover_shapes(void);

/*
 * q4_release_workspace: frees the library-owned scratch of every device and
 * stream.  The split path of the bitsandbytes pull request "[ROCm] Optimize
 * kgemm_4bit_inference_naive ..." (section "Fused path support for M > 1")
 * dequantizes W to bf16 before the GEMM, so that path needs an N*K*2-byte
 * buffer; it also holds the activation planes of fp16 / fp32 inputs and the
 * fp32 partial outputs of K splits.  The library keeps one buffer per
 * (device, stream), grown on demand: a growth frees the previous buffer, so
 * HIP graphs captured with calls that used it must not be replayed after a
 * call that grows it, or after this call.  A growth is refused while its
 * stream is being captured (Q4_ERR_HIP; run the call once eagerly first).
 * Each device that owns a buffer is synchronised before its buffers are
 * freed.  Returns Q4_ERR_HIP (and still forgets every buffer) if a
 * synchronisation or free fails.
 */
q4_status q4_release_workspace(void);

/*
 * q4_last_error: the message of the last failing call on the calling thread
 * ("" after a successful call); valid until the thread's next call into the
 * library.  Every entry point returns a status the caller acts on and drains
 * the HIP runtime's last-error flag after a failed launch, the convention of
 * the bitsandbytes pull request "Cache the hipBLASLt int8 matmul algo per
 * problem on ROCm" (its csrc/ops.cu change); this accessor carries the
 * runtime's or the validator's message to the caller.
 */
const char *q4_last_error(void);

/*
 * q4_copy_probe: dst[i] = src[i] for `bytes` bytes (a multiple of 16, both
 * pointers 16-byte aligned) with the same 128-bit streaming loads as the
 * GEMM kernels.  A measurement aid: it gives the achievable HBM copy rate
 * and scales hardware byte counters against a transfer of known size.
 */
q4_status q4_copy_probe(const void *src, void *dst, size_t bytes, void *stream);

/*
 * q4_read_probe: reads `bytes` bytes at `src` once with 128-bit buffer loads
 * and writes (almost) nothing.  A measurement aid: the achievable HBM read
 * rate of one launch over a buffer of that size, the ceiling of kernels that
 * stream their weights once, against which the bitsandbytes pull request
 * "[ROCm] Optimize kgemm_4bit_inference_naive for ROCm, use it for batch
 * sizes other than 1" also quotes a measured peak (table
 * "kgemm_4bit_inference_naive benchmark").
 *
 *  src         device buffer, 16-byte aligned; bytes a multiple of 16, below
 *              4 GiB.
 *  sink        device buffer of one uint32, written only when the folded
 *              data equals a fixed value (it keeps every load live).
 *  threads     lanes per workgroup: 256, 512 or 1024 (0 = the default below).
 *  unroll      16-byte loads per lane per batch: 2, 4 or 8 (0 = default);
 *              about twice that many are in flight per lane.
 *  wgs_per_cu  workgroups per compute unit, 1..32 (0 = default).
 *  flags       Q4_PROBE_NONTEMPORAL: the loads carry the non-temporal hint
 *              of the fused kernels' weight loads; Q4_PROBE_INTERLEAVE:
 *              batches are dealt round robin to the workgroups instead of
 *              one contiguous share each.
 *
 *  Q4_ERR_INVALID_ARGUMENT: NULL pointer, misalignment, a launch shape or
 *    flag outside the sets above.  Q4_ERR_UNSUPPORTED: bytes >= 4 GiB.
 */
/* The fastest shape of a sweep over 132 MB (9 rotating buffers) on MI355X:
 * 256 lanes, 4 loads per batch, 2 workgroups per CU (with both flags set,
 * 19.6 us = 6.7 TB/s; 512 lanes x 8 loads x 1 workgroup took 21.7 us). */
#define Q4_READ_PROBE_THREADS 256
#define Q4_READ_PROBE_UNROLL 4
#define Q4_READ_PROBE_WGS_PER_CU 2
enum { Q4_PROBE_NONTEMPORAL = 1, Q4_PROBE_INTERLEAVE = 2 };
q4_status q4_read_probe(const void *src, size_t bytes, uint32_t *sink, int threads, int unroll,
                        int wgs_per_cu, int flags, void *stream);

/* Library version string. */
const char *q4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4SKINNY_H */
