// C-ABI layer of q4skinny: argument validation, path dispatch, split-path
// workspace, HIP error capture.  Declared in include/q4skinny.h.
//
// Error convention (after the bitsandbytes int8 pull request "Cache the
// hipBLASLt int8 matmul algo per problem on ROCm", which returns a status code
// the caller acts on and drains the sticky HIP error after a failed launch):
// every entry point validates all arguments before touching the runtime,
// returns a q4_status, and leaves a message for q4_last_error().
#include "q4skinny.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "launch.h"

namespace {

// Fused-versus-split threshold on MI355X (fused when M <= value) for weight
// shapes without an entry of their own.  Timed at M = 33 .. 512 on the decode
// layer shapes (K, N) = (5120, 8192), (5120, 5120), (17408, 5120),
// (8192, 8192), the 28672 x 8192 FFN, the 4096 x 4096 GEMV and the 248320 x
// 2560 output projection: the fused path (the tiled kernel above 32 rows)
// wins on every shape up to M = 192 (1.4x to 3x at M = 64), and dequantize +
// tiled GEMM first wins between M = 256 and M = 512 depending on the shape.
// The smallest of those switch points is the default: the routing principle
// of the bitsandbytes pull request "[ROCm] Optimize
// kgemm_4bit_inference_naive for ROCm, use it for batch sizes other than 1"
// (maintainer's comment) prefers a missed win to a regression.
constexpr int kDefaultCrossoverM = 192;

// Measured crossovers of those shapes: (N, K) -> the largest M the fused path
// takes.  They seed the per-shape table, which the caller can change or clear.
struct ShapeEntry {
    int n, k, m;
};
constexpr ShapeEntry kMeasuredCrossovers[] = {
    {8192, 5120, 384}, {5120, 5120, 384}, {5120, 17408, 192}, {8192, 8192, 384},
    {28672, 8192, 384}, {4096, 4096, 512}, {248320, 2560, 384},
};

thread_local std::string tl_error;

q4_status fail(q4_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    tl_error = buf;
    return st;
}

q4_status ok() {
    tl_error.clear();
    return Q4_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---- test hook: Q4_TEST_FAIL_LAUNCH=<kernel>[:count] --------------------------
// kernel: fused, dequant, gemm, planes, plane sum, quantize, copy or read.  Makes the
// next `count` launches of that kernel report a launch failure without
// launching, so tests can check the error path and the recovery.
std::once_flag g_hook_once;
std::string g_hook_kernel;
std::atomic<int> g_hook_left{0};

bool injected_failure(const char *kernel) {
    std::call_once(g_hook_once, [] {
        const char *v = std::getenv("Q4_TEST_FAIL_LAUNCH");
        if (!v || !*v) return;
        std::string s(v);
        int count = 1;
        const size_t colon = s.find(':');
        if (colon != std::string::npos) {
            count = std::atoi(s.c_str() + colon + 1);
            s.resize(colon);
        }
        g_hook_kernel = s;
        g_hook_left.store(count);
    });
    if (g_hook_left.load() <= 0 || g_hook_kernel != kernel) return false;
    return g_hook_left.fetch_sub(1) > 0;
}

q4_status check_launch(hipError_t e, const char *kernel) {
    if (e != hipSuccess) {
        (void)hipGetLastError();  // drain the sticky error so the next call starts clean
        return fail(Q4_ERR_HIP, "%s: %s", kernel, hipGetErrorString(e));
    }
    return Q4_OK;
}

// Runs one launcher and checks its status; the test hook fails it before it
// launches anything.
template <class F>
q4_status launch_checked(const char *kernel, F &&launch) {
    if (injected_failure(kernel))
        return fail(Q4_ERR_HIP, "%s: injected launch failure (Q4_TEST_FAIL_LAUNCH)", kernel);
    return check_launch(launch(), kernel);
}

// ---- crossover -------------------------------------------------------------
std::atomic<int> g_crossover{-1};

int crossover() {
    int v = g_crossover.load();
    if (v >= 0) return v;
    int init = kDefaultCrossoverM;
    if (const char *e = std::getenv("Q4_CROSSOVER_M")) {
        char *end = nullptr;
        const long x = std::strtol(e, &end, 10);
        if (end != e && *end == '\0' && x >= 0 && x <= Q4_CROSSOVER_MAX) init = (int)x;
    }
    int expected = -1;
    g_crossover.compare_exchange_strong(expected, init);
    return g_crossover.load();
}

// Per-shape crossovers: an entry for (N, K) overrides the process-wide value
// for that weight shape.  The table starts from the measured entries above,
// then the environment variable Q4_CROSSOVER_TABLE ("N:K:m" items separated
// by commas) at first use; a malformed item is skipped.
std::mutex g_shape_mutex;
std::map<std::pair<int, int>, int> g_shape_crossover;
bool g_shape_loaded = false;

void load_shape_table_locked() {
    if (g_shape_loaded) return;
    g_shape_loaded = true;
    for (const ShapeEntry &x : kMeasuredCrossovers) g_shape_crossover[{x.n, x.k}] = x.m;
    const char *e = std::getenv("Q4_CROSSOVER_TABLE");
    if (!e) return;
    const std::string text(e);
    size_t pos = 0;
    while (pos <= text.size()) {
        size_t end = text.find(',', pos);
        if (end == std::string::npos) end = text.size();
        const std::string item = text.substr(pos, end - pos);
        long n = 0, k = 0, m = 0;
        char extra = 0;
        if (std::sscanf(item.c_str(), "%ld:%ld:%ld%c", &n, &k, &m, &extra) == 3 && n > 0 &&
            k > 0 && n <= INT32_MAX && k <= INT32_MAX && m >= 0 && m <= Q4_CROSSOVER_MAX)
            g_shape_crossover[{(int)n, (int)k}] = (int)m;
        pos = end + 1;
    }
}

// Shapes without an entry of their own take the entry of a shape in the same
// bucket, the convention of the bitsandbytes pull request "Cache the
// hipBLASLt int8 matmul algo per problem on ROCm" (an exact key first, then a
// bucket key).  A bucket groups shapes on which the fused kernel runs the
// same schedule and the split path does about as much work per weight: the
// same K rounded up to a power of two, and the same class of 16-row tiles per
// compute unit (1, 2, 3-4 or 5 and more; the skinny kernel's ring and scale
// period change at those points).  Several entries in one bucket: the
// smallest crossover, which prefers a missed win to a regression.
int bucket_of(int N, int K) {
    int kb = 0;
    while (kb < 31 && (1 << kb) < K) ++kb;
    const int tb = q4::q4_fused_tiles_per_chunk(N);
    const int tc = tb <= 1 ? 0 : tb == 2 ? 1 : tb <= 4 ? 2 : 3;
    return kb * 4 + tc;
}

int crossover_for(int N, int K) {
    std::lock_guard<std::mutex> lock(g_shape_mutex);
    load_shape_table_locked();
    const auto it = g_shape_crossover.find({N, K});
    if (it != g_shape_crossover.end()) return it->second;
    const int b = bucket_of(N, K);
    int best = -1;
    for (const auto &kv : g_shape_crossover)
        if (bucket_of(kv.first.first, kv.first.second) == b && (best < 0 || kv.second < best))
            best = kv.second;
    return best >= 0 ? best : crossover();
}

// ---- workspace: one buffer per (device, stream) -------------------------------
// The split path's bf16 weights, the activation planes of fp16 / fp32 inputs
// and the fp32 partial outputs of K splits.  One buffer per stream, so that
// calls on different streams never share scratch; grown on demand.  Growing
// frees the old buffer: HIP graphs captured earlier with calls that used it
// must not be replayed after a call that grows it.  Growing during a stream
// capture is refused (an allocation cannot be captured): the first call of a
// shape runs eagerly, later calls of the same or a smaller size reuse the
// buffer and can be captured.
struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// A call made through q4_gemm_skinny_ex_noalloc brings its own scratch (the
// device's fixed array) for the duration of the call on this thread; every
// workspace request of that call is served from it or refused.
thread_local void *tl_fixed_scratch = nullptr;
thread_local size_t tl_fixed_bytes = 0;

q4_status refuse_under_capture(hipStream_t s, const char *what, size_t bytes) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(s, &cap);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(Q4_ERR_HIP, "%s: hipStreamIsCapturing: %s", what, hipGetErrorString(e));
    }
    if (cap != hipStreamCaptureStatusNone)
        return fail(Q4_ERR_HIP,
                    "%s of %zu bytes needed while the stream is being captured: run the call "
                    "once outside the capture first",
                    what, bytes);
    return Q4_OK;
}

q4_status workspace(int device, hipStream_t s, size_t bytes, void **out) {
    if (tl_fixed_scratch) {
        if (bytes > tl_fixed_bytes)
            return fail(Q4_ERR_UNSUPPORTED,
                        "this call needs %zu bytes of scratch, above the %zu bytes of the "
                        "allocation-free entry point",
                        bytes, tl_fixed_bytes);
        *out = tl_fixed_scratch;
        return Q4_OK;
    }
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace &w = g_ws[{device, s}];
    if (w.bytes < bytes) {
        q4_status st = refuse_under_capture(s, "workspace", bytes);
        if (st != Q4_OK) return st;
        hipError_t e = hipSuccess;
        if (w.ptr) {
            // The old buffer may still be read by work queued on `s`; it is
            // freed even if that wait fails.
            hipError_t se = hipStreamSynchronize(s);
            hipError_t fe = hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
            if (se != hipSuccess || fe != hipSuccess) {
                (void)hipGetLastError();
                return fail(Q4_ERR_HIP, "workspace release: %s",
                            hipGetErrorString(se != hipSuccess ? se : fe));
            }
        }
        void *p = nullptr;
        e = hipMalloc(&p, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(Q4_ERR_HIP, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
        }
        w.ptr = p;
        w.bytes = bytes;
    }
    *out = w.ptr;
    return Q4_OK;
}

// ---- validation ---------------------------------------------------------------
int log2_exact(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return ((1 << l) == v) ? l : -1;
}

q4_status check_q4_shape(int N, int K, int blocksize, int *bs_log2) {
    if (N < 0 || K < 0) return fail(Q4_ERR_INVALID_ARGUMENT, "negative size (N=%d, K=%d)", N, K);
    if (K == 0) return fail(Q4_ERR_INVALID_ARGUMENT, "K must be positive");
    if (blocksize <= 0 || (blocksize & 1))
        return fail(Q4_ERR_INVALID_ARGUMENT, "blocksize %d must be positive and even", blocksize);
    if (K % blocksize)
        return fail(Q4_ERR_INVALID_ARGUMENT, "K=%d is not a multiple of blocksize %d", K, blocksize);
    if (blocksize != 32 && blocksize != 64 && blocksize != 128 && blocksize != 256)
        return fail(Q4_ERR_UNSUPPORTED, "blocksize %d not in {32, 64, 128, 256}", blocksize);
    if ((int64_t)N * (int64_t)K > (int64_t(1) << 41))
        return fail(Q4_ERR_UNSUPPORTED, "N*K=%lld too large", (long long)N * K);
    *bs_log2 = log2_exact(blocksize);
    return Q4_OK;
}

q4_status drain_prior_error() {
    (void)hipGetLastError();
    return Q4_OK;
}

bool known_dtype(int dt) { return dt == Q4_DTYPE_BF16 || dt == Q4_DTYPE_FP16 || dt == Q4_DTYPE_FP32; }
size_t dtype_size(int dt) { return dt == Q4_DTYPE_FP32 ? 4 : 2; }

// Token rows above which the fused path takes the tiled matrix-core kernel
// (each decoded weight serves a 64-row token block) instead of the skinny
// kernel, which reads the packed weights once per pass of up to 32 rows: 32,
// or 16 on shapes where the skinny kernel runs 17..32 rows as two 16-row
// launches (8 tiles per chunk; measured at 248320 x 2560, M = 32: 174 us
// tiled, 210 us in two launches).  Test hooks, read once:
// Q4_FUSED_TILED_MIN_M (0 .. Q4_CROSSOVER_MAX) replaces the threshold,
// Q4_FUSED_TILED_LAYOUT (0 or 1) forces the tiled kernel's work layout.
constexpr int kFusedTiledMinM = 32;

int env_int(const char *name, int lo, int hi, int dflt) {
    if (const char *e = std::getenv(name)) {
        char *end = nullptr;
        const long x = std::strtol(e, &end, 10);
        if (end != e && *end == '\0' && x >= lo && x <= hi) return (int)x;
    }
    return dflt;
}

int fused_tiled_min_m(int N) {
    static const int env = env_int("Q4_FUSED_TILED_MIN_M", 0, Q4_CROSSOVER_MAX, -1);
    if (env >= 0) return env;
    return q4::q4_fused_mfma_two_blocks(N) ? kFusedTiledMinM : 16;
}

int fused_tiled_layout() {
    static const int v = env_int("Q4_FUSED_TILED_LAYOUT", 0, 1, -1);
    return v;
}

bool fused_tiled(int rows, int N, int K, int bs_log2) {
    return bs_log2 >= 6 && rows > fused_tiled_min_m(N) && q4::q4_fused_tiled_fits(rows, N, K);
}

q4_status current_device(int *device) {
    const hipError_t e = hipGetDevice(device);
    if (e == hipSuccess) return Q4_OK;
    (void)hipGetLastError();
    return fail(Q4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
}

// The tiled fused kernel on bf16 activations (rows = token rows, or np*M rows
// of activation planes).  When K is split over workgroups (ksplit > 1) the
// kernel writes ksplit fp32 partial outputs to `parts` for the caller to sum.
q4_status run_fused_tiled(const uint16_t *A, const uint8_t *Wp, const float *am, const float *cb,
                          const void *bias, int rows, int N, int K, int bs_log2, int wl,
                          const q4::TiledPlan &plan, float *parts, void *C, int c_dt,
                          hipStream_t s) {
    if (plan.ksplit == 1)
        return launch_checked("fused", [&] {
            return q4::launch_q4_fused_tiled(A, Wp, am, cb, bias, rows, N, K, bs_log2, wl, plan, C,
                                             c_dt, s);
        });
    return launch_checked("fused", [&] {
        return q4::launch_q4_fused_tiled(A, Wp, am, cb, nullptr, rows, N, K, bs_log2, wl, plan,
                                         parts, Q4_DTYPE_FP32, s);
    });
}

q4_status run_fused_planes(const void *A, int a_dt, const uint8_t *Wp, const float *am,
                           const float *cb, const void *bias, int M, int N, int K, int bs_log2,
                           int wl, void *C, int c_dt, hipStream_t s);

// bf16 activations: the tiled kernel above fused_tiled_min_m rows, else the
// skinny kernels in passes of up to Q4_FUSED_PASS_M token rows over
// consecutive row slabs, each streaming the packed weights once more (more
// than one pass only where the tiled kernel cannot run).  Up to 32 rows (one
// pass) the skinny kernel may split K over workgroups (kparts_ok: the
// workspace is free for its partial sums, i.e. not holding activation
// planes).
q4_status run_fused(const void *A, int a_dt, const uint8_t *Wp, const float *am, const float *cb,
                    const void *bias, int M, int N, int K, int bs_log2, int wl, void *C, int c_dt,
                    hipStream_t s, bool kparts_ok = true) {
    if (a_dt != Q4_DTYPE_BF16 && bs_log2 >= 6 && q4::q4_fused_mfma_fits(M, N, K))
        return run_fused_planes(A, a_dt, Wp, am, cb, bias, M, N, K, bs_log2, wl, C, c_dt, s);
    if (a_dt == Q4_DTYPE_BF16 && fused_tiled(M, N, K, bs_log2)) {
        const q4::TiledPlan plan = q4::q4_fused_tiled_plan(M, N, K, 4, fused_tiled_layout());
        const int ks = plan.ksplit;
        float *parts = nullptr;
        if (ks > 1) {
            int device = 0;
            q4_status st = current_device(&device);
            if (st != Q4_OK) return st;
            void *ws = nullptr;
            st = workspace(device, s, (size_t)ks * (size_t)M * (size_t)N * 4, &ws);
            if (st != Q4_OK) return st;
            parts = static_cast<float *>(ws);
        }
        q4_status st = run_fused_tiled(static_cast<const uint16_t *>(A), Wp, am, cb, bias, M, N,
                                       K, bs_log2, wl, plan, parts, C, c_dt, s);
        if (st != Q4_OK || ks == 1) return st;
        return launch_checked("plane sum", [&] {
            return q4::launch_sum_planes(parts, ks, M, N, bias, C, c_dt, s);
        });
    }
    float *kpart = nullptr;
    if (kparts_ok && a_dt == Q4_DTYPE_BF16 && bs_log2 >= 6 && M <= 32 &&
        q4::q4_fused_mfma_fits(M, N, K)) {
        const int ks = q4::q4_fused_kparts(M, N, K);
        if (ks > 1) {
            int device = 0;
            q4_status st = current_device(&device);
            if (st != Q4_OK) return st;
            void *ws = nullptr;
            st = workspace(device, s, (size_t)ks * (size_t)M * (size_t)N * 4, &ws);
            if (st != Q4_OK) return st;
            kpart = static_cast<float *>(ws);
        }
    }
    const size_t a_row = (size_t)K * dtype_size(a_dt), c_row = (size_t)N * dtype_size(c_dt);
    for (int m0 = 0; m0 < M; m0 += Q4_FUSED_PASS_M) {
        const int mm = M - m0 < Q4_FUSED_PASS_M ? M - m0 : Q4_FUSED_PASS_M;
        q4_status st = launch_checked("fused", [&] {
            return q4::launch_q4_fused(static_cast<const char *>(A) + (size_t)m0 * a_row, a_dt,
                                       Wp, am, cb, bias, mm, N, K, bs_log2,
                                       static_cast<char *>(C) + (size_t)m0 * c_row, c_dt, wl, s,
                                       kpart);
        });
        if (st != Q4_OK) return st;
    }
    return Q4_OK;
}

// fp16 / fp32 activations with blocksize >= 64: the exact split of each
// activation row into 2 / 3 bf16 planes (planes.hip) runs through the
// matrix-core kernels as np*M bf16 rows with fp32 partial outputs (times the
// K parts of the tiled kernel, at most 4 slabs in all), then one pass sums
// the partials of each output, adds the bias and rounds once.  Planes and
// partials live in the per-stream workspace.
q4_status run_fused_planes(const void *A, int a_dt, const uint8_t *Wp, const float *am,
                           const float *cb, const void *bias, int M, int N, int K, int bs_log2,
                           int wl, void *C, int c_dt, hipStream_t s) {
    int device = 0;
    q4_status st = current_device(&device);
    if (st != Q4_OK) return st;
    const int np = q4::activation_planes(a_dt);
    const int rows = np * M;
    // Few tokens (np planes per group of 4 tokens fit one lane's 4 output
    // rows): the skinny kernel adds each token's planes itself, so no fp32
    // partials and no second pass.
    if (np * ((M + 3) / 4) <= 4 && q4::q4_fused_mfma_fits(rows, N, K)) {
        void *ws = nullptr;
        st = workspace(device, s, (size_t)rows * (size_t)K * 2, &ws);
        if (st != Q4_OK) return st;
        uint16_t *planes = static_cast<uint16_t *>(ws);
        st = launch_checked("planes", [&] {
            return q4::launch_split_planes(A, a_dt, (size_t)M * (size_t)K, planes, s);
        });
        if (st != Q4_OK) return st;
        return launch_checked("fused", [&] {
            return q4::launch_q4_fused_mfma(planes, Q4_DTYPE_BF16, Wp, am, cb, bias, M, N, K,
                                            bs_log2, C, c_dt, wl, s, nullptr, np);
        });
    }
    const bool tiled = fused_tiled(rows, N, K, bs_log2);
    // at most 4 partial slabs in all (planes times K parts)
    const q4::TiledPlan plan =
        tiled ? q4::q4_fused_tiled_plan(rows, N, K, 4 / np, fused_tiled_layout()) : q4::TiledPlan{0, 1};
    const int ks = plan.ksplit;
    const size_t plane_bytes = (size_t)rows * (size_t)K * 2;
    const size_t part_off = (plane_bytes + 255) & ~(size_t)255;
    void *ws = nullptr;
    st = workspace(device, s, part_off + (size_t)(ks * np) * (size_t)M * (size_t)N * 4, &ws);
    if (st != Q4_OK) return st;
    uint16_t *planes = static_cast<uint16_t *>(ws);
    float *parts = reinterpret_cast<float *>(static_cast<char *>(ws) + part_off);
    st = launch_checked("planes", [&] {
        return q4::launch_split_planes(A, a_dt, (size_t)M * (size_t)K, planes, s);
    });
    if (st != Q4_OK) return st;
    st = tiled ? run_fused_tiled(planes, Wp, am, cb, nullptr, rows, N, K, bs_log2, wl, plan,
                                 parts, parts, Q4_DTYPE_FP32, s)
               : run_fused(planes, Q4_DTYPE_BF16, Wp, am, cb, nullptr, rows, N, K, bs_log2, wl,
                           parts, Q4_DTYPE_FP32, s, false);
    if (st != Q4_OK) return st;
    return launch_checked("plane sum", [&] {
        return q4::launch_sum_planes(parts, ks * np, M, N, bias, C, c_dt, s);
    });
}

// Token rows above which the split path's GEMM takes the tiled kernel (which
// reuses each weight tile from LDS for 128 tokens) instead of the streaming
// kernel (which reads the weights once per 16-row slab).
constexpr int kTiledGemmMinM = 16;

q4_status run_split(const void *A, int a_dt, const uint8_t *Wp, const float *am, const float *cb,
                    const void *bias, int M, int N, int K, int bs_log2, int wl, void *C, int c_dt,
                    hipStream_t s) {
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(Q4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    }
    // Workspace: the bf16 weights, then (on the tiled GEMM) the bf16 planes of
    // fp16 activations and the fp32 partial outputs of the planes and K parts.
    const bool tiled = M > kTiledGemmMinM && q4::gemm_tiled_fits(2 * M, N, K);
    const int np = tiled && a_dt == Q4_DTYPE_FP16 ? 2 : 1;
    int ks = tiled ? q4::gemm_tiled_ksplit(np * M, N, K) : 1;
    if (np * ks > 4) ks = 4 / np;
    const bool partials = np * ks > 1;
    const size_t w_bytes = ((size_t)N * (size_t)K * 2 + 255) & ~(size_t)255;
    const size_t p_bytes = np > 1 ? ((np * (size_t)M * (size_t)K * 2 + 255) & ~(size_t)255) : 0;
    const size_t s_bytes = partials ? (size_t)(np * ks) * (size_t)M * (size_t)N * 4 : 0;
    void *ws = nullptr;
    q4_status st = workspace(device, s, w_bytes + p_bytes + s_bytes, &ws);
    if (st != Q4_OK) return st;
    const uint16_t *Wd = static_cast<const uint16_t *>(ws);
    st = launch_checked("dequant", [&] {
        return q4::launch_dequant(Wp, am, cb, N, K, bs_log2, wl, ws, Q4_DTYPE_BF16, s);
    });
    if (st != Q4_OK) return st;
    if (!tiled)
        return launch_checked("gemm", [&] {
            return q4::launch_bf16_gemm(A, a_dt, Wd, bias, M, N, K, C, c_dt, s);
        });
    if (!partials)
        return launch_checked("gemm", [&] {
            return q4::launch_gemm_tiled(static_cast<const uint16_t *>(A), Wd, bias, M, N, K, 1,
                                         C, c_dt, s);
        });
    const uint16_t *Ab = static_cast<const uint16_t *>(A);
    if (np > 1) {
        uint16_t *pl = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + w_bytes);
        st = launch_checked("planes", [&] {
            return q4::launch_split_planes(A, a_dt, (size_t)M * (size_t)K, pl, s);
        });
        if (st != Q4_OK) return st;
        Ab = pl;
    }
    // np*ks fp32 slabs of M x N: [K part][plane][M][N]
    float *parts = reinterpret_cast<float *>(static_cast<char *>(ws) + w_bytes + p_bytes);
    st = launch_checked("gemm", [&] {
        return q4::launch_gemm_tiled(Ab, Wd, nullptr, np * M, N, K, ks, parts, Q4_DTYPE_FP32, s);
    });
    if (st != Q4_OK) return st;
    return launch_checked("plane sum", [&] {
        return q4::launch_sum_planes(parts, np * ks, M, N, bias, C, c_dt, s);
    });
}

// The tile layout: N % 16 == 0 and K % 128 == 0 (whole 16-row tiles of
// whole 128-wide segments), offsets within the 32-bit range of the
// matrix-core kernels (no vector-ALU fallback reads tiles), blocksize >= 64.
q4_status check_tiles(int M, int N, int K, int blocksize) {
    if (N % 16 != 0 || K % 128 != 0)
        return fail(Q4_ERR_INVALID_ARGUMENT,
                    "the tile layout needs N %% 16 == 0 and K %% 128 == 0 (N=%d, K=%d)", N, K);
    if (blocksize < 64)
        return fail(Q4_ERR_UNSUPPORTED, "the tile layout needs blocksize >= 64 (got %d)",
                    blocksize);
    if (!q4::q4_fused_mfma_fits(M, N, K))
        return fail(Q4_ERR_UNSUPPORTED, "tile-layout matrix too large (N=%d, K=%d)", N, K);
    return Q4_OK;
}

q4_status gemm_impl(const void *A, int a_dtype, const uint8_t *Wpacked, int wl,
                    const float *absmax, const float *codebook, const void *bias, int M, int N,
                    int K, int blocksize, void *C, int c_dtype, void *stream, int path) {
    if (path != Q4_PATH_AUTO && path != Q4_PATH_FUSED && path != Q4_PATH_SPLIT)
        return fail(Q4_ERR_INVALID_ARGUMENT, "unknown path %d", path);
    if (!known_dtype(a_dtype) || !known_dtype(c_dtype))
        return fail(Q4_ERR_INVALID_ARGUMENT, "unknown dtype (a_dtype=%d, c_dtype=%d)", a_dtype,
                    c_dtype);
    if (M < 0) return fail(Q4_ERR_INVALID_ARGUMENT, "negative size (M=%d)", M);
    int bs_log2 = 0;
    q4_status st = check_q4_shape(N, K, blocksize, &bs_log2);
    if (st != Q4_OK) return st;
    if ((int64_t)M * K > (int64_t(1) << 40))
        return fail(Q4_ERR_UNSUPPORTED, "M*K too large");
    if (wl && (st = check_tiles(M, N, K, blocksize)) != Q4_OK) return st;
    bool fused;
    if (path == Q4_PATH_FUSED) fused = true;
    else if (path == Q4_PATH_SPLIT) fused = false;
    else fused = M <= crossover_for(N, K);
    if (!fused && a_dtype == Q4_DTYPE_FP32)
        return fail(Q4_ERR_UNSUPPORTED, "fp32 activations take the fused path only (M=%d)", M);
    if (M == 0 || N == 0) return ok();
    if (!A || !Wpacked || !absmax || !codebook || !C)
        return fail(Q4_ERR_INVALID_ARGUMENT, "NULL pointer argument");
    const size_t cs = dtype_size(c_dtype);
    if (!aligned(A, 16) || !aligned(Wpacked, 16) || !aligned(absmax, 16) || !aligned(codebook, 4) ||
        !aligned(C, cs) || (bias && !aligned(bias, cs)))
        return fail(Q4_ERR_INVALID_ARGUMENT,
                    "A, Wpacked and absmax must be 16-byte aligned, C and bias aligned to "
                    "their element size");
    drain_prior_error();
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = fused ? run_fused(A, a_dtype, Wpacked, absmax, codebook, bias, M, N, K, bs_log2, wl, C,
                           c_dtype, s)
               : run_split(A, a_dtype, Wpacked, absmax, codebook, bias, M, N, K, bs_log2, wl, C,
                           c_dtype, s);
    return st == Q4_OK ? ok() : st;
}

q4_status dequant_impl(const uint8_t *Wpacked, int wl, const float *absmax,
                       const float *codebook, int N, int K, int blocksize, void *out,
                       int out_dtype, void *stream) {
    if (!known_dtype(out_dtype))
        return fail(Q4_ERR_INVALID_ARGUMENT, "unknown out_dtype %d", out_dtype);
    int bs_log2 = 0;
    q4_status st = check_q4_shape(N, K, blocksize, &bs_log2);
    if (st != Q4_OK) return st;
    if (wl && (st = check_tiles(0, N, K, blocksize)) != Q4_OK) return st;
    if (N == 0) return ok();
    if (!Wpacked || !absmax || !codebook || !out)
        return fail(Q4_ERR_INVALID_ARGUMENT, "NULL pointer argument");
    if (!aligned(Wpacked, 16) || !aligned(absmax, 16) || !aligned(codebook, 4) || !aligned(out, 16))
        return fail(Q4_ERR_INVALID_ARGUMENT, "Wpacked, absmax and out must be 16-byte aligned");
    drain_prior_error();
    st = launch_checked("dequant", [&] {
        return q4::launch_dequant(Wpacked, absmax, codebook, N, K, bs_log2, wl, out, out_dtype,
                                  static_cast<hipStream_t>(stream));
    });
    return st == Q4_OK ? ok() : st;
}

// bf16_gemm_skinny over row-major (wl = 0) or tile-layout (wl = 1) weights.
q4_status bf16_impl(const void *A, const void *W, int wl, const void *bias, int M, int N, int K,
                    void *C, void *stream) {
    if (M < 0 || N < 0 || K < 0)
        return fail(Q4_ERR_INVALID_ARGUMENT, "negative size (M=%d, N=%d, K=%d)", M, N, K);
    if (K == 0) return fail(Q4_ERR_INVALID_ARGUMENT, "K must be positive");
    if (K % 8) return fail(Q4_ERR_INVALID_ARGUMENT, "K=%d must be a multiple of 8", K);
    if (wl && (N % 16 != 0 || K % 32 != 0))
        return fail(Q4_ERR_INVALID_ARGUMENT,
                    "the bf16 tile layout needs N %% 16 == 0 and K %% 32 == 0 (N=%d, K=%d)", N, K);
    if (M > 5) return fail(Q4_ERR_UNSUPPORTED, "bf16 skinny GEMM supports M <= 5 (M=%d)", M);
    if ((int64_t)N * (int64_t)K > (int64_t(1) << 40))
        return fail(Q4_ERR_UNSUPPORTED, "N*K too large");
    if (wl && !q4::bf16_tiles_fit(N, K))
        return fail(Q4_ERR_UNSUPPORTED, "bf16 tile-layout matrix too large (N=%d, K=%d)", N, K);
    if (M == 0 || N == 0) return ok();
    if (!A || !W || !C) return fail(Q4_ERR_INVALID_ARGUMENT, "NULL pointer argument");
    if (!aligned(A, 16) || !aligned(W, 16) || !aligned(C, 2) || (bias && !aligned(bias, 2)))
        return fail(Q4_ERR_INVALID_ARGUMENT,
                    "A and W must be 16-byte aligned, C and bias 2-byte aligned");
    drain_prior_error();
    q4_status st = launch_checked("gemm", [&] {
        return q4::launch_bf16_gemm(A, Q4_DTYPE_BF16, static_cast<const uint16_t *>(W), bias, M,
                                    N, K, C, Q4_DTYPE_BF16, static_cast<hipStream_t>(stream), wl);
    });
    return st == Q4_OK ? ok() : st;
}

}  // namespace

namespace q4 {

q4_status report(q4_status st, const char *what, hipError_t e) {
    (void)hipGetLastError();
    return fail(st, "%s: %s", what, hipGetErrorString(e));
}

q4_status gemm_ex_fixed_scratch(const void *A, int a_dtype, const uint8_t *Wpacked,
                                const float *absmax, const float *codebook, const void *bias,
                                int M, int N, int K, int blocksize, void *C, int c_dtype,
                                void *stream, int path, void *scratch, size_t scratch_bytes) {
    tl_fixed_scratch = scratch;
    tl_fixed_bytes = scratch_bytes;
    const q4_status st = gemm_impl(A, a_dtype, Wpacked, 0, absmax, codebook, bias, M, N, K,
                                   blocksize, C, c_dtype, stream, path);
    tl_fixed_scratch = nullptr;
    tl_fixed_bytes = 0;
    return st;
}

DeviceInfo device_info() {
    static std::atomic<int> cus[256];  // 0 = not yet queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) {
        (void)hipGetLastError();
        return DeviceInfo{0, 256};
    }
    int n = cus[dev].load();
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cus[dev].store(n);
    }
    return DeviceInfo{dev, n};
}

}  // namespace q4

extern "C" {

q4_status q4_gemm_skinny_ex(const void *A, int a_dtype, const uint8_t *Wpacked,
                            const float *absmax, const float *codebook, const void *bias, int M,
                            int N, int K, int blocksize, void *C, int c_dtype, void *stream,
                            int path) {
    return gemm_impl(A, a_dtype, Wpacked, 0, absmax, codebook, bias, M, N, K, blocksize, C,
                     c_dtype, stream, path);
}

q4_status q4_gemm_skinny_tiles(const void *A, int a_dtype, const uint8_t *Wtiles,
                               const float *absmax, const float *codebook, const void *bias,
                               int M, int N, int K, int blocksize, void *C, int c_dtype,
                               void *stream, int path) {
    return gemm_impl(A, a_dtype, Wtiles, 1, absmax, codebook, bias, M, N, K, blocksize, C,
                     c_dtype, stream, path);
}

q4_status q4_gemm_skinny_path(const void *A, const uint8_t *Wpacked, const float *absmax,
                              const float *codebook, int M, int N, int K, int blocksize,
                              void *C, void *stream, int path) {
    return q4_gemm_skinny_ex(A, Q4_DTYPE_BF16, Wpacked, absmax, codebook, nullptr, M, N, K,
                             blocksize, C, Q4_DTYPE_BF16, stream, path);
}

q4_status q4_gemm_skinny(const void *A, const uint8_t *Wpacked, const float *absmax,
                         const float *codebook, int M, int N, int K, int blocksize, void *C,
                         void *stream) {
    return q4_gemm_skinny_path(A, Wpacked, absmax, codebook, M, N, K, blocksize, C, stream,
                               Q4_PATH_AUTO);
}

q4_status bf16_gemm_skinny(const void *A, const void *W, const void *bias, int M, int N, int K,
                           void *C, void *stream) {
    return bf16_impl(A, W, 0, bias, M, N, K, C, stream);
}

q4_status bf16_gemm_skinny_tiles(const void *A, const void *Wtiles, const void *bias, int M,
                                 int N, int K, void *C, void *stream) {
    return bf16_impl(A, Wtiles, 1, bias, M, N, K, C, stream);
}

q4_status bf16_repack_tiles(const void *W, void *Wtiles, int N, int K, void *stream) {
    if (N < 0 || K < 0) return fail(Q4_ERR_INVALID_ARGUMENT, "negative size (N=%d, K=%d)", N, K);
    if (K == 0) return fail(Q4_ERR_INVALID_ARGUMENT, "K must be positive");
    if (N % 16 != 0 || K % 32 != 0)
        return fail(Q4_ERR_INVALID_ARGUMENT,
                    "the bf16 tile layout needs N %% 16 == 0 and K %% 32 == 0 (N=%d, K=%d)", N, K);
    if (!q4::bf16_tiles_fit(N, K))
        return fail(Q4_ERR_UNSUPPORTED, "bf16 tile-layout matrix too large (N=%d, K=%d)", N, K);
    if (N == 0) return ok();
    if (!W || !Wtiles) return fail(Q4_ERR_INVALID_ARGUMENT, "NULL pointer argument");
    if (!aligned(W, 16) || !aligned(Wtiles, 16))
        return fail(Q4_ERR_INVALID_ARGUMENT, "W and Wtiles must be 16-byte aligned");
    const size_t bytes = (size_t)N * (size_t)K * 2;
    const uintptr_t a = reinterpret_cast<uintptr_t>(W), b = reinterpret_cast<uintptr_t>(Wtiles);
    if (a < b + bytes && b < a + bytes)
        return fail(Q4_ERR_INVALID_ARGUMENT, "Wtiles must not overlap W");
    drain_prior_error();
    q4_status st = launch_checked("repack", [&] {
        return q4::launch_bf16_repack_tiles(static_cast<const uint16_t *>(W),
                                            static_cast<uint16_t *>(Wtiles), N, K,
                                            static_cast<hipStream_t>(stream));
    });
    return st == Q4_OK ? ok() : st;
}

q4_status q4_dequant(const uint8_t *Wpacked, const float *absmax, const float *codebook, int N,
                     int K, int blocksize, void *out, int out_dtype, void *stream) {
    return dequant_impl(Wpacked, 0, absmax, codebook, N, K, blocksize, out, out_dtype, stream);
}

q4_status q4_dequant_tiles(const uint8_t *Wtiles, const float *absmax, const float *codebook,
                           int N, int K, int blocksize, void *out, int out_dtype, void *stream) {
    return dequant_impl(Wtiles, 1, absmax, codebook, N, K, blocksize, out, out_dtype, stream);
}

q4_status q4_repack_tiles(const uint8_t *Wpacked, uint8_t *Wtiles, int N, int K, void *stream) {
    if (N < 0 || K < 0) return fail(Q4_ERR_INVALID_ARGUMENT, "negative size (N=%d, K=%d)", N, K);
    if (K == 0) return fail(Q4_ERR_INVALID_ARGUMENT, "K must be positive");
    if (N % 16 != 0 || K % 128 != 0)
        return fail(Q4_ERR_INVALID_ARGUMENT,
                    "the tile layout needs N %% 16 == 0 and K %% 128 == 0 (N=%d, K=%d)", N, K);
    if ((uint64_t)N * (uint64_t)K / 2 >= (1ull << 32))
        return fail(Q4_ERR_UNSUPPORTED, "tile-layout matrix too large (N=%d, K=%d)", N, K);
    if (N == 0) return ok();
    if (!Wpacked || !Wtiles) return fail(Q4_ERR_INVALID_ARGUMENT, "NULL pointer argument");
    if (!aligned(Wpacked, 16) || !aligned(Wtiles, 16))
        return fail(Q4_ERR_INVALID_ARGUMENT, "Wpacked and Wtiles must be 16-byte aligned");
    const size_t bytes = (size_t)N * (size_t)K / 2;
    const uintptr_t a = reinterpret_cast<uintptr_t>(Wpacked), b = reinterpret_cast<uintptr_t>(Wtiles);
    if (a < b + bytes && b < a + bytes)
        return fail(Q4_ERR_INVALID_ARGUMENT, "Wtiles must not overlap Wpacked");
    drain_prior_error();
    q4_status st = launch_checked("repack", [&] {
        return q4::launch_repack_tiles(Wpacked, Wtiles, N, K, static_cast<hipStream_t>(stream));
    });
    return st == Q4_OK ? ok() : st;
}

q4_status q4_quantize(const void *W, int w_dtype, const float *codebook, int N, int K,
                      int blocksize, uint8_t *Wpacked, float *absmax, void *stream) {
    if (!known_dtype(w_dtype)) return fail(Q4_ERR_INVALID_ARGUMENT, "unknown w_dtype %d", w_dtype);
    int bs_log2 = 0;
    q4_status st = check_q4_shape(N, K, blocksize, &bs_log2);
    if (st != Q4_OK) return st;
    if (blocksize < 32)
        return fail(Q4_ERR_UNSUPPORTED, "blocksize %d: the quantizer needs >= 32", blocksize);
    if (!codebook) return fail(Q4_ERR_INVALID_ARGUMENT, "NULL codebook");
    q4::QuantizeTable tab{};
    for (int i = 0; i < 16; ++i)
        if (!std::isfinite(codebook[i]))
            return fail(Q4_ERR_INVALID_ARGUMENT, "codebook entry %d is not finite", i);
    for (int i = 0; i < 15; ++i) {
        if (!(codebook[i] < codebook[i + 1]))
            return fail(Q4_ERR_INVALID_ARGUMENT,
                        "the quantizer needs a strictly increasing codebook (entries %d, %d)", i,
                        i + 1);
        tab.mid[i] = ((double)codebook[i] + (double)codebook[i + 1]) / 2.0;  // exact
    }
    // the entry nearest to 0, ties to the lower one: midpoints below 0
    tab.zero_code = 0;
    for (int i = 0; i < 15; ++i) tab.zero_code += tab.mid[i] < 0.0 ? 1u : 0u;
    if (N == 0) return ok();
    if (!W || !Wpacked || !absmax) return fail(Q4_ERR_INVALID_ARGUMENT, "NULL pointer argument");
    if (!aligned(W, 16) || !aligned(Wpacked, 16) || !aligned(absmax, 4))
        return fail(Q4_ERR_INVALID_ARGUMENT,
                    "W and Wpacked must be 16-byte aligned, absmax 4-byte aligned");
    drain_prior_error();
    st = launch_checked("quantize", [&] {
        return q4::launch_quantize(W, w_dtype, N, K, bs_log2, tab, Wpacked, absmax,
                                   static_cast<hipStream_t>(stream));
    });
    return st == Q4_OK ? ok() : st;
}

namespace {
// Standard normal quantile by bisection on 0.5 * erfc(-x / sqrt 2): the
// function is increasing, so 200 halvings of [-40, 40] pin the root to the
// last bit of a double.
double normal_quantile(double p) {
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 200; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid;
        else hi = mid;
    }
    return 0.5 * (lo + hi);
}
}  // namespace

q4_status q4_codebook_preset(int which, float *codebook) {
    if (!codebook) return fail(Q4_ERR_INVALID_ARGUMENT, "NULL codebook");
    if (which == Q4_CODEBOOK_INT4) {
        for (int i = 0; i < 16; ++i) codebook[i] = (float)(i - 8) / 8.0f;
        return ok();
    }
    if (which != Q4_CODEBOOK_NF4_STYLE)
        return fail(Q4_ERR_INVALID_ARGUMENT, "unknown codebook preset %d", which);
    const double p_max = 0.97;
    double pos[8], neg[7];
    for (int i = 1; i <= 8; ++i) pos[i - 1] = normal_quantile(0.5 + (i / 8.0) * (p_max - 0.5));
    for (int i = 1; i <= 7; ++i) neg[i - 1] = normal_quantile(0.5 - (i / 7.0) * (p_max - 0.5));
    double v[16];
    int n = 0;
    for (int i = 0; i < 7; ++i) v[n++] = neg[i] / -neg[6];
    v[n++] = 0.0;
    for (int i = 0; i < 8; ++i) v[n++] = pos[i] / pos[7];
    std::sort(v, v + 16);
    for (int i = 0; i < 16; ++i) codebook[i] = (float)v[i];
    return ok();
}

int q4_get_crossover_m(void) { return crossover(); }

q4_status q4_set_crossover_m(int m) {
    if (m < 0 || m > Q4_CROSSOVER_MAX)
        return fail(Q4_ERR_INVALID_ARGUMENT, "crossover %d not in 0..%d", m, Q4_CROSSOVER_MAX);
    g_crossover.store(m);
    return ok();
}

q4_status q4_set_crossover_shape(int N, int K, int m) {
    if (N <= 0 || K <= 0)
        return fail(Q4_ERR_INVALID_ARGUMENT, "shape N=%d K=%d must be positive", N, K);
    if (m > Q4_CROSSOVER_MAX)
        return fail(Q4_ERR_INVALID_ARGUMENT, "crossover %d above %d", m, Q4_CROSSOVER_MAX);
    std::lock_guard<std::mutex> lock(g_shape_mutex);
    load_shape_table_locked();
    if (m < 0) g_shape_crossover.erase({N, K});
    else g_shape_crossover[{N, K}] = m;
    return ok();
}

int q4_get_crossover_shape(int N, int K) { return crossover_for(N, K); }

int q4_skinny_kparts(int M, int N, int K) {
    if (M < 1 || M > 32 || N < 1 || K < 1) return 1;
    return q4::q4_fused_kparts(M, N, K);
}

q4_status q4_clear_crossover_shapes(void) {
    std::lock_guard<std::mutex> lock(g_shape_mutex);
    g_shape_loaded = true;  // the environment's table is not read again
    g_shape_crossover.clear();
    return ok();
}

q4_status q4_release_workspace(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    q4_status st = Q4_OK;
    int prev = 0;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    // Each device that owns a buffer is synchronised once (the streams the
    // buffers were used on may no longer exist), then its buffers are freed.
    std::map<int, bool> synced;
    for (auto &kv : g_ws) {
        if (!kv.second.ptr) continue;
        const int device = kv.first.first;
        hipError_t e = hipSetDevice(device);
        if (e == hipSuccess && !synced[device]) {
            e = hipDeviceSynchronize();
            synced[device] = true;
        }
        const hipError_t fe = hipFree(kv.second.ptr);
        if (e == hipSuccess) e = fe;
        if (e != hipSuccess && st == Q4_OK) {
            (void)hipGetLastError();
            st = fail(Q4_ERR_HIP, "workspace release: %s", hipGetErrorString(e));
        }
    }
    g_ws.clear();
    if (have_prev) (void)hipSetDevice(prev);
    return st == Q4_OK ? ok() : st;
}

const char *q4_last_error(void) { return tl_error.c_str(); }

q4_status q4_copy_probe(const void *src, void *dst, size_t bytes, void *stream) {
    if (bytes == 0) return ok();
    if (!src || !dst) return fail(Q4_ERR_INVALID_ARGUMENT, "NULL pointer argument");
    if (bytes % 16 || !aligned(src, 16) || !aligned(dst, 16))
        return fail(Q4_ERR_INVALID_ARGUMENT, "bytes and pointers must be multiples of 16");
    drain_prior_error();
    q4_status st = launch_checked("copy", [&] {
        return q4::launch_copy_probe(src, dst, bytes, static_cast<hipStream_t>(stream));
    });
    return st == Q4_OK ? ok() : st;
}

q4_status q4_read_probe(const void *src, size_t bytes, uint32_t *sink, int threads, int unroll,
                        int wgs_per_cu, int flags, void *stream) {
    if (threads == 0) threads = Q4_READ_PROBE_THREADS;
    if (unroll == 0) unroll = Q4_READ_PROBE_UNROLL;
    if (wgs_per_cu == 0) wgs_per_cu = Q4_READ_PROBE_WGS_PER_CU;
    if (!q4::read_probe_shape_ok(threads, unroll) || wgs_per_cu < 1 || wgs_per_cu > 32 ||
        (flags & ~(Q4_PROBE_NONTEMPORAL | Q4_PROBE_INTERLEAVE)) != 0)
        return fail(Q4_ERR_INVALID_ARGUMENT,
                    "read probe shape: threads %d (256, 512, 1024), unroll %d (2, 4, 8), "
                    "workgroups per CU %d (1..32), flags 0x%x",
                    threads, unroll, wgs_per_cu, flags);
    if (bytes >= (size_t(1) << 32))
        return fail(Q4_ERR_UNSUPPORTED, "read probe over %zu bytes (below 4 GiB)", bytes);
    if (bytes == 0) return ok();
    if (!src || !sink) return fail(Q4_ERR_INVALID_ARGUMENT, "NULL pointer argument");
    if (bytes % 16 || !aligned(src, 16) || !aligned(sink, 4))
        return fail(Q4_ERR_INVALID_ARGUMENT,
                    "bytes and src must be multiples of 16, sink 4-byte aligned");
    drain_prior_error();
    q4_status st = launch_checked("read", [&] {
        return q4::launch_read_probe(src, bytes, sink, threads, unroll, wgs_per_cu,
                                     (flags & Q4_PROBE_NONTEMPORAL) != 0,
                                     (flags & Q4_PROBE_INTERLEAVE) != 0,
                                     static_cast<hipStream_t>(stream));
    });
    return st == Q4_OK ? ok() : st;
}

const char *q4_version(void) { return "q4skinny 0.2.0 (gfx950)"; }

}  // extern "C"
