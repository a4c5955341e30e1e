/*
 * Plain CPU oracle for the blockwise 4-bit skinny GEMM and its bf16 sibling.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  The GPU
 * library never links, includes or calls it, and it shares no code with the
 * GPU library (no headers, tables or helpers).
 *
 * Everything here is written for obviousness, not speed: scalar loops, fp64
 * accumulation in increasing k, one output element at a time.  The only
 * concession to run time is an OpenMP loop over output columns, which does not
 * change any result (each element is still one sequential sum).
 *
 * Sources (web pages, by title and section):
 *  - "[ROCm] Optimize kgemm_4bit_inference_naive for ROCm, use it for batch
 *    sizes other than 1" (bitsandbytes pull request 1920), sections "Technical
 *    details" and the maintainer's comment on the replacement kernel: the
 *    computation is a fused dequantize + matmul over blockwise 4-bit weights
 *    looked up in a 16-entry NF4/FP4 table, blocksize 64 by default, fp32
 *    accumulation, "TN" inference layout A[M,K] * W[N,K]^T.
 *  - "Support N=5 in wvSplitK skinny GEMM kernels for speculative decoding"
 *    (vLLM pull request 40687 report), section "关键源码片段": bf16 skinny GEMM of
 *    a weight W[out,K] with 1..5 token rows and an optional bias.
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes):
 *  - nibble order: the low nibble of byte j holds even k = 2j, the high nibble
 *    holds odd k = 2j + 1;
 *  - a quantization block runs along K inside one row (K % blocksize == 0), so
 *    block b of row n covers k in [b*bs, (b+1)*bs) and its scale is
 *    absmax[n * (K/bs) + b];
 *  - a dequantized weight is one IEEE binary32 product codebook[code]*absmax;
 *    the bf16 dequantized weight is that product rounded to bf16 with
 *    round-to-nearest-even;
 *  - activations, weights and bias in bf16, fp16 or fp32 are widened exactly
 *    to fp64; a bias is added to the sum of products;
 *  - fp16 is IEEE binary16, rounded to from fp32 to nearest even.
 *
 * Compiled with -O2 -ffp-contract=off (no fused multiply-add anywhere) and
 * without -ffast-math, so fp32 denormals are kept.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

/* A bf16 value is the top half of an fp32 bit pattern: widening is exact. */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---- O1: unpack one 4-bit code ------------------------------------------ */
/* Row n of the packed matrix holds K/2 bytes.  Byte j carries k = 2j in its
 * low nibble and k = 2j + 1 in its high nibble. */
int oracle_code(const uint8_t *Wpacked, int64_t K, int64_t n, int64_t k)
{
    uint8_t byte = Wpacked[n * (K / 2) + k / 2];
    if (k % 2 == 0)
        return byte & 0x0F;
    return (byte >> 4) & 0x0F;
}

void oracle_unpack(const uint8_t *Wpacked, int64_t N, int64_t K, uint8_t *codes)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            codes[n * K + k] = (uint8_t)oracle_code(Wpacked, K, n, k);
}

/* ---- O2: which absmax scales element (n, k) ----------------------------- */
int64_t oracle_block_index(int64_t K, int64_t bs, int64_t n, int64_t k)
{
    return n * (K / bs) + k / bs;
}

/* ---- O3: fp32 dequantized weight ---------------------------------------- */
/* One binary32 multiply, rounded to nearest even (the C default).  The
 * volatile store keeps the product a separate, rounded fp32 value. */
float oracle_w32(const uint8_t *Wpacked, const float *absmax, const float *codebook,
                 int64_t K, int64_t bs, int64_t n, int64_t k)
{
    int code = oracle_code(Wpacked, K, n, k);
    float scale = absmax[oracle_block_index(K, bs, n, k)];
    volatile float w = codebook[code] * scale;
    return w;
}

void oracle_dequant_f32(const uint8_t *Wpacked, const float *absmax, const float *codebook,
                        int64_t N, int64_t K, int64_t bs, float *out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            out[n * K + k] = oracle_w32(Wpacked, absmax, codebook, K, bs, n, k);
}

/* ---- O4: fp32 -> bf16, round to nearest, ties to even ------------------- */
/* Keep the top 16 bits of the fp32 pattern.  The discarded low half decides:
 * above half an ulp rounds up, below rounds down, exactly half rounds to the
 * even neighbour.  A NaN stays a NaN (quiet bit forced).  Rounding up may
 * carry into the exponent, which correctly yields the next binade or inf. */
uint16_t oracle_f32_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint32_t exp_bits = (u >> 23) & 0xFF;
    uint32_t man_bits = u & 0x7FFFFF;
    if (exp_bits == 0xFF && man_bits != 0)
        return (uint16_t)((u >> 16) | 0x0040);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xFFFF;
    if (lower > 0x8000 || (lower == 0x8000 && (upper & 1) != 0))
        upper += 1;
    return (uint16_t)upper;
}

void oracle_f32_to_bf16_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f32_to_bf16(x[i]);
}

void oracle_dequant_bf16(const uint8_t *Wpacked, const float *absmax, const float *codebook,
                         int64_t N, int64_t K, int64_t bs, uint16_t *out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            out[n * K + k] = oracle_f32_to_bf16(oracle_w32(Wpacked, absmax, codebook, K, bs, n, k));
}

/* ---- O5: the fused 4-bit GEMM, the reference of the tolerance ------------ */
/* C[m, j] = sum over k of a[m,k] * w32(cols[j], k), summed in fp64 in
 * increasing k.  Every product is exact in fp64 (8-bit by 24-bit
 * significands), so the only rounding is in the running fp64 sum.  S[m, j] is
 * the same sum over absolute values, the scale of the tolerance.  cols lists
 * the output columns to compute (NULL = all N, in order); C and S are
 * [M, ncols] row-major. */
void oracle_q4_gemm(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                    const float *codebook, int64_t M, int64_t N, int64_t K, int64_t bs,
                    const int64_t *cols, int64_t ncols, double *C, double *S)
{
    if (cols == NULL)
        ncols = N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < ncols; j++) {
        int64_t n = cols ? cols[j] : j;
        for (int64_t m = 0; m < M; m++) {
            double sum = 0.0, sum_abs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double a = bf16_to_double(A[m * K + k]);
                double w = (double)oracle_w32(Wpacked, absmax, codebook, K, bs, n, k);
                double p = a * w;
                sum += p;
                sum_abs += fabs(p);
            }
            C[m * ncols + j] = sum;
            if (S)
                S[m * ncols + j] = sum_abs;
        }
    }
}

/* ---- O7: the same GEMM on bf16-rounded weights (split-path diagnostic) --- */
void oracle_q4_gemm_w16(const uint16_t *A, const uint8_t *Wpacked, const float *absmax,
                        const float *codebook, int64_t M, int64_t N, int64_t K, int64_t bs,
                        const int64_t *cols, int64_t ncols, double *C, double *S)
{
    if (cols == NULL)
        ncols = N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < ncols; j++) {
        int64_t n = cols ? cols[j] : j;
        for (int64_t m = 0; m < M; m++) {
            double sum = 0.0, sum_abs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double a = bf16_to_double(A[m * K + k]);
                uint16_t w16 = oracle_f32_to_bf16(
                    oracle_w32(Wpacked, absmax, codebook, K, bs, n, k));
                double p = a * bf16_to_double(w16);
                sum += p;
                sum_abs += fabs(p);
            }
            C[m * ncols + j] = sum;
            if (S)
                S[m * ncols + j] = sum_abs;
        }
    }
}

/* ---- O6: bf16 GEMM with optional bias ----------------------------------- */
/* C[m, j] = sum over k of a[m,k] * W[cols[j], k] (+ bias[cols[j]]), fp64 in
 * increasing k, bias added last.  S includes |bias|. */
void oracle_bf16_gemm(const uint16_t *A, const uint16_t *W, const uint16_t *bias,
                      int64_t M, int64_t N, int64_t K, const int64_t *cols, int64_t ncols,
                      double *C, double *S)
{
    if (cols == NULL)
        ncols = N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < ncols; j++) {
        int64_t n = cols ? cols[j] : j;
        for (int64_t m = 0; m < M; m++) {
            double sum = 0.0, sum_abs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = bf16_to_double(A[m * K + k]) * bf16_to_double(W[n * K + k]);
                sum += p;
                sum_abs += fabs(p);
            }
            if (bias) {
                double b = bf16_to_double(bias[n]);
                sum += b;
                sum_abs += fabs(b);
            }
            C[m * ncols + j] = sum;
            if (S)
                S[m * ncols + j] = sum_abs;
        }
    }
}

/* ---- O8 building block: plain fp64 GEMM over an fp32 weight matrix ------ */
/* Used to check that dequantize-then-multiply equals the fused oracle. */
void oracle_gemm_f32w(const uint16_t *A, const float *W, int64_t M, int64_t N, int64_t K,
                      double *C)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; k++)
                sum += bf16_to_double(A[m * K + k]) * (double)W[n * K + k];
            C[m * N + n] = sum;
        }
}

/* ---- O9: IEEE binary16 <-> binary32 -------------------------------------- */
/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.  A
 * normal value is (1 + f/1024) * 2^(e - 15), a subnormal (e = 0) is
 * f * 2^-24, e = 31 is infinity (f = 0) or NaN. */
double oracle_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + f / 1024.0, e - 15);
    return sign ? -v : v;
}

/* Nearest binary16 to a binary32 value, ties to the even fraction.  The
 * 24-bit significand is shifted right to the binary16 precision at the
 * value's exponent (11 bits for normals, fewer for subnormals); the bits
 * shifted out decide the rounding exactly as in the bf16 case.  A carry out
 * of the fraction moves to the next binade; past 65504 the result is
 * infinity. */
uint16_t oracle_f32_to_f16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    int E = (int)((u >> 23) & 0xFF);
    uint32_t m = u & 0x7FFFFF;
    if (E == 0xFF)
        return (uint16_t)(sign | (m ? 0x7E00 : 0x7C00));
    if (E == 0)
        return sign; /* binary32 subnormals are below half the smallest binary16 subnormal */
    uint32_t sig = (1u << 23) | m; /* value = sig * 2^(E - 150) */
    int e16 = E - 127 + 15;       /* biased binary16 exponent for a normal result */
    int shift = e16 >= 1 ? 13 : 13 + (1 - e16);
    if (shift > 24)
        return sign;
    uint32_t q = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1)))
        q += 1;
    if (e16 >= 1) {
        if (q == 2048) { /* carried into the next binade */
            q = 1024;
            e16 += 1;
        }
        if (e16 >= 31)
            return (uint16_t)(sign | 0x7C00);
        return (uint16_t)(sign | (e16 << 10) | (q & 0x3FF));
    }
    /* subnormal result: q counts units of 2^-24; q == 1024 is the smallest normal */
    return (uint16_t)(sign | q);
}

void oracle_f32_to_f16_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f32_to_f16(x[i]);
}

void oracle_dequant_f16(const uint8_t *Wpacked, const float *absmax, const float *codebook,
                        int64_t N, int64_t K, int64_t bs, uint16_t *out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            out[n * K + k] = oracle_f32_to_f16(oracle_w32(Wpacked, absmax, codebook, K, bs, n, k));
}

/* ---- O10: the fused 4-bit GEMM with any activation type and a bias ------- */
/* Element types: 0 bf16, 1 binary32, 2 binary16 (the library's codes).
 * Each element is widened exactly to fp64. */
static double elem(const void *p, int64_t i, int dtype)
{
    if (dtype == 1)
        return (double)((const float *)p)[i];
    uint16_t b = ((const uint16_t *)p)[i];
    return dtype == 2 ? oracle_f16_to_double(b) : bf16_to_double(b);
}

/* C[m, j] = sum over k of a[m,k] * w32(cols[j], k) + bias[cols[j]], fp64 in
 * increasing k, bias added last; every product is exact in fp64 (at most 24
 * by 24 significant bits).  S adds |bias| to the sum of |a*w|.  bias may be
 * NULL. */
void oracle_q4_gemm_ex(const void *A, int a_dtype, const uint8_t *Wpacked, const float *absmax,
                       const float *codebook, const void *bias, int bias_dtype, int64_t M,
                       int64_t N, int64_t K, int64_t bs, const int64_t *cols, int64_t ncols,
                       double *C, double *S)
{
    if (cols == NULL)
        ncols = N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < ncols; j++) {
        int64_t n = cols ? cols[j] : j;
        for (int64_t m = 0; m < M; m++) {
            double sum = 0.0, sum_abs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double a = elem(A, m * K + k, a_dtype);
                double w = (double)oracle_w32(Wpacked, absmax, codebook, K, bs, n, k);
                double p = a * w;
                sum += p;
                sum_abs += fabs(p);
            }
            if (bias) {
                double b = elem(bias, n, bias_dtype);
                sum += b;
                sum_abs += fabs(b);
            }
            C[m * ncols + j] = sum;
            if (S)
                S[m * ncols + j] = sum_abs;
        }
    }
}

/* ---- O11: blockwise 4-bit quantization (the inverse of O3) ---------------- */
/* For a strictly increasing codebook c[0] < ... < c[15] and each block of bs
 * consecutive k of a row: absmax = max |w| over the block (exact), and each
 * weight takes the code of the entry nearest to the exact ratio w / absmax,
 * a tie between two entries going to the lower one.  Entries i and i+1 are
 * separated by their midpoint m_i = (c[i] + c[i+1]) / 2 (exact in fp64), so
 * the nearest entry is the number of midpoints strictly below the ratio; with
 * absmax > 0, m_i < w / absmax is the same as m_i * absmax < w, and that
 * product of two 24-bit significands is exact in fp64, so every comparison is
 * exact.  A block of zeros (absmax = 0) takes the ratio 0.  Weights are
 * bf16, fp16 or fp32 (element types as in O10), widened exactly. */
void oracle_quantize(const void *W, int w_dtype, const float *codebook, int64_t N, int64_t K,
                     int64_t bs, uint8_t *codes, float *absmax)
{
    double mid[15];
    for (int i = 0; i < 15; i++)
        mid[i] = ((double)codebook[i] + (double)codebook[i + 1]) / 2.0;
    for (int64_t n = 0; n < N; n++)
        for (int64_t b = 0; b < K / bs; b++) {
            double a = 0.0;
            for (int64_t k = b * bs; k < (b + 1) * bs; k++) {
                double w = fabs(elem(W, n * K + k, w_dtype));
                if (w > a)
                    a = w;
            }
            absmax[n * (K / bs) + b] = (float)a; /* a is one of the inputs: exact */
            for (int64_t k = b * bs; k < (b + 1) * bs; k++) {
                double w = a > 0.0 ? elem(W, n * K + k, w_dtype) : 0.0;
                double scale = a > 0.0 ? a : 1.0;
                int code = 0;
                for (int i = 0; i < 15; i++)
                    if (mid[i] * scale < w)
                        code++;
                codes[n * K + k] = (uint8_t)code;
            }
        }
}

/* O12  The tile layout of the packed weights (a layout of this library, not
 * of the pages; the pages leave the packed-weight layout to the kernel).
 * Rows form tiles of 16 (tile t = rows 16t..16t+15); a row's bytes form
 * segments of 64 (segment s = bytes 64s..64s+63, i.e. k = 128s..128s+127);
 * the 16 rows x 64 bytes of (t, s) become one unit of 1024 bytes, stored
 * unit after unit in the order (t, s) with s fastest.  Inside a unit, the
 * 64 bytes of a row's segment are 8 quarters of 8 bytes (quarter c = bytes
 * 8c..8c+7, k = 128s + 16c .. +15); piece p = 0..63 of 16 bytes belongs to
 * row 16t + p % 16 and holds quarter a then quarter a + 4 (one piece of each
 * 64-wide half of the segment), where a = 0, 2, 1, 3 for p / 16 = 0, 1, 2,
 * 3.  Requires N % 16 == 0 and K % 128 == 0.
 * oracle_tile_offset gives where byte j of row n goes; oracle_repack_tiles
 * moves every byte there. */
int64_t oracle_tile_offset(int64_t N, int64_t K, int64_t n, int64_t j)
{
    (void)N;
    int64_t segs = K / 128;     /* segments per row */
    int64_t t = n / 16, r = n % 16;
    int64_t s = j / 64, q = j % 64;
    int64_t quarter = q / 8, half = quarter / 4, a = quarter % 4;
    int64_t piece = r + 16 * (2 * (a % 2) + a / 2);
    return (t * segs + s) * 1024 + piece * 16 + half * 8 + q % 8;
}

void oracle_repack_tiles(const uint8_t *Wpacked, int64_t N, int64_t K, uint8_t *out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t j = 0; j < K / 2; j++)
            out[oracle_tile_offset(N, K, n, j)] = Wpacked[n * (K / 2) + j];
}

/* O13  The tile layout of unquantized bf16 weights (again a layout of this
 * library; the bf16 skinny GEMM of the pages reads W [N, K] row-major).
 * Rows form tiles of 16 as in O12; a row's elements form steps of 32
 * (step s = k 32s..32s+31, the k one matrix-core instruction consumes);
 * the 16 rows x 32 elements of (t, s) become one unit of 512 elements,
 * stored unit after unit in the order (t, s) with s fastest; inside a unit,
 * piece p = 0..63 of 8 elements holds k = 32s + 8*(p / 16) .. +7 of row
 * 16t + p % 16.  Requires N % 16 == 0 and K % 32 == 0.
 * oracle_bf16_tile_index gives the element index that W[n][k] moves to;
 * oracle_bf16_repack_tiles moves every element there. */
int64_t oracle_bf16_tile_index(int64_t N, int64_t K, int64_t n, int64_t k)
{
    (void)N;
    int64_t steps = K / 32;     /* steps per row */
    int64_t t = n / 16, r = n % 16;
    int64_t s = k / 32, q = k % 32;
    int64_t piece = r + 16 * (q / 8);
    return (t * steps + s) * 512 + piece * 8 + q % 8;
}

void oracle_bf16_repack_tiles(const uint16_t *W, int64_t N, int64_t K, uint16_t *out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            out[oracle_bf16_tile_index(N, K, n, k)] = W[n * K + k];
}

/* Thread count of the OpenMP loops from here on (the benchmark's CPU baseline
 * times the oracle single-threaded and on all cores); n < 1 leaves it as is. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
