// C ABI of libmq: argument validation, device check and kernel dispatch.
//
// Every check runs on the host before the first HIP call, so each failure
// can be exercised without a GPU. Failures return a status and leave a
// message naming the argument and its value (minfer Compute Graph Design,
// §7.4 Error contract: errors name the actual values and never fall back).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/mq.h"
#include "mq_launch.h"

namespace mq {
KernelEvents &kernel_events()
{
    thread_local KernelEvents ev;
    return ev;
}
} // namespace mq

namespace {

thread_local char g_err[512];

// Entry points whose kernels the timing hook does not cover drop a pending
// timing request, so it can only ever attach to the matmul or quantizer call
// that follows it (the workspace queries launch nothing and leave it).
void drop_timing() { mq::kernel_events() = mq::KernelEvents{}; }

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxDim = 0x7fffffff;
// M and N: the launchers round them up to whole tiles in 32-bit arithmetic
constexpr int64_t kMaxRows = 0x7fff0000;

// Per-device result of the architecture query: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device()
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(MQ_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MQ_ERR_DEVICE, "device ordinal %d out of range", dev);
    int state = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(MQ_ERR_DEVICE, "hipGetDeviceProperties(%d) failed: %s", dev,
                        hipGetErrorString(e));
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_ok[dev].store(state, std::memory_order_relaxed);
        if (state == 2)
            return fail(MQ_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950",
                        dev, prop.gcnArchName);
    }
    if (state == 2)
        return fail(MQ_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return MQ_OK;
}

int launched(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(MQ_ERR_LAUNCH, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return MQ_OK;
}

int check_K(int64_t K, const char *fn)
{
    if (K < 256 || K % 256 != 0)
        return fail(MQ_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 256", fn, (long long)K);
    if (K > kMaxDim)
        return fail(MQ_ERR_SHAPE, "%s: K=%lld exceeds %lld", fn, (long long)K, (long long)kMaxDim);
    return MQ_OK;
}

enum class Fmt { Q4K = MQ_FMT_Q4K, Q5K = MQ_FMT_Q5K, Q6K = MQ_FMT_Q6K };

const char *fmt_fn(Fmt fmt)
{
    return fmt == Fmt::Q6K ? "mq_matmul_q6k" : fmt == Fmt::Q5K ? "mq_matmul_q5k" : "mq_matmul_q4k";
}

// Shape and path checks shared by a matmul and its workspace query.
int check_matmul_shape(const char *fn, int64_t M, int64_t N, int64_t K, int path)
{
    if (M <= 0) return fail(MQ_ERR_INVALID_ARG, "%s: M=%lld must be positive", fn, (long long)M);
    if (N <= 0) return fail(MQ_ERR_INVALID_ARG, "%s: N=%lld must be positive", fn, (long long)N);
    if (int rc = check_K(K, fn)) return rc;
    if (M > kMaxRows || N > kMaxRows)
        return fail(MQ_ERR_SHAPE, "%s: M=%lld, N=%lld: each must be at most %lld", fn,
                    (long long)M, (long long)N, (long long)kMaxRows);
    if (path != MQ_PATH_AUTO && path != MQ_PATH_GEMV && path != MQ_PATH_GEMM)
        return fail(MQ_ERR_INVALID_ARG, "%s: path=%d is not MQ_PATH_AUTO/GEMV/GEMM", fn, path);
    if (path == MQ_PATH_GEMV && M > mq::GEMV_MAX_M)
        return fail(MQ_ERR_INVALID_ARG, "%s: path=MQ_PATH_GEMV needs M <= %d, got M=%lld", fn,
                    mq::GEMV_MAX_M, (long long)M);
    // grid sizes must fit the launch limits
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles > kMaxDim)
        return fail(MQ_ERR_SHAPE, "%s: M=%lld x N=%lld needs too many tiles", fn, (long long)M, (long long)N);
    return MQ_OK;
}

// The kernel a matmul runs: the GEMV, or the GEMM in its small-M or its
// main configuration.
enum class Kern { GEMV, GEMM_SMALL, GEMM };

Kern matmul_kernel(Fmt fmt, int64_t M, int64_t N, int64_t K, int path)
{
    const bool q6 = fmt == Fmt::Q6K;
    const bool gemv = path == MQ_PATH_GEMV ||
                      (path == MQ_PATH_AUTO && (fmt == Fmt::Q5K ? mq::gemv_auto_q5k(M, N, K)
                                                                : mq::gemv_auto(q6, M, N, K)));
    if (gemv)
        return Kern::GEMV;
    const int small = q6 ? mq::GEMM_SMALL_M_Q6K : fmt == Fmt::Q5K ? mq::GEMM_SMALL_M_Q5K : mq::GEMM_SMALL_M_Q4K;
    return M <= small ? Kern::GEMM_SMALL : Kern::GEMM;
}

// Workspace bytes of the split-K partial sums of a GEMM configuration (0 =
// it does not split).
size_t split_ws_bytes(Fmt fmt, Kern kern, int64_t M, int64_t N, int64_t K)
{
    const int m = (int)M, n = (int)N, k = (int)K;
    int s = 1;
    if (kern == Kern::GEMM_SMALL)
        s = fmt == Fmt::Q6K ? mq::splits_gemm_q6k_small(m, n, k)
          : fmt == Fmt::Q5K ? mq::splits_gemm_q5k_small(m, n, k) : mq::splits_gemm_q4k_small(m, n, k);
    else if (kern == Kern::GEMM)
        s = fmt == Fmt::Q6K ? mq::splits_gemm_q6k(m, n, k)
          : fmt == Fmt::Q5K ? mq::splits_gemm_q5k(m, n, k) : mq::splits_gemm_q4k(m, n, k);
    return mq::split_bytes(s, M, N);
}

// The Q6_K expansion plan: a GEMM of at least MQ_Q6K_EXPAND_MIN_M tokens,
// given the full workspace, expands W there into the limb planes lo, hi
// [N][K] and d [N][K/256] (then the split-K sums) and runs the
// expansion-plane GEMM: each block decoded once per call instead of once
// per token tile, the same result bit for bit. Measured on MI355X at
// 3584 x 18944 (the expansion 42 us): M = 512 206 against 227 us on the
// raw blocks, M = 1024 328 against 393 us; at M = 384 the expansion about
// cancels the gain (163 against 163 us). Matrices of more than
// MQ_Q6K_EXPAND_MAX_WEIGHTS weights keep the raw blocks (their planes
// would pass 512 MB).
bool q6k_expands(Fmt fmt, Kern kern, int64_t M, int64_t N, int64_t K)
{
    return fmt == Fmt::Q6K && kern == Kern::GEMM && M >= MQ_Q6K_EXPAND_MIN_M &&
           N * K <= MQ_Q6K_EXPAND_MAX_WEIGHTS;
}
constexpr size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t q6k_planes_bytes(int64_t N, int64_t K)
{
    return 2 * round256((size_t)N * (size_t)K) + round256((size_t)N * (size_t)(K / 256) * sizeof(float));
}

// Workspace bytes of the full plan of a GEMM configuration (0 = none).
size_t gemm_ws_bytes(Fmt fmt, Kern kern, int64_t M, int64_t N, int64_t K)
{
    const size_t split = split_ws_bytes(fmt, kern, M, N, K);
    return q6k_expands(fmt, kern, M, N, K) ? q6k_planes_bytes(N, K) + split : split;
}

// The caller's workspace argument: NULL (with ws_bytes 0) selects the
// workspace-free plan; otherwise it must be 16-byte aligned and hold
// `need` bytes.
int check_ws(const char *fn, const void *ws, int64_t ws_bytes, size_t need)
{
    if (ws_bytes < 0)
        return fail(MQ_ERR_INVALID_ARG, "%s: ws_bytes=%lld is negative", fn, (long long)ws_bytes);
    if (!ws) {
        if (ws_bytes != 0)
            return fail(MQ_ERR_INVALID_ARG, "%s: ws is NULL but ws_bytes=%lld", fn, (long long)ws_bytes);
        return MQ_OK;
    }
    if (!aligned(ws, 16)) return fail(MQ_ERR_ALIGN, "%s: ws=%p is not 16-byte aligned", fn, ws);
    if ((uint64_t)ws_bytes < (uint64_t)need)
        return fail(MQ_ERR_WORKSPACE, "%s: the workspace holds %lld bytes, this call needs %llu", fn,
                    (long long)ws_bytes, (unsigned long long)need);
    return MQ_OK;
}

// expand: the call may take the Q6_K expansion plan (the static-array entry
// point keeps the split-K plan of the raw-block GEMM).
int matmul(Fmt fmt, const void *W, const int8_t *q, const float *d, const float *s,
           int64_t M, int64_t N, int64_t K, float *out, void *ws, int64_t ws_bytes, void *stream, int path,
           bool expand = true)
{
    const bool q6 = fmt == Fmt::Q6K;
    const char *fn = fmt_fn(fmt);
    if (!W) return fail(MQ_ERR_INVALID_ARG, "%s: W is NULL", fn);
    if (!q) return fail(MQ_ERR_INVALID_ARG, "%s: q is NULL", fn);
    if (!d) return fail(MQ_ERR_INVALID_ARG, "%s: d is NULL", fn);
    if (!q6 && !s) return fail(MQ_ERR_INVALID_ARG, "%s: s is NULL (the min term needs it)", fn);
    if (!out) return fail(MQ_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (int rc = check_matmul_shape(fn, M, N, K, path)) return rc;
    // Q4_K / Q5_K blocks are read as 16-byte pieces (their rows are whole
    // multiples of 16 bytes); Q6_K blocks are 2-byte aligned within a row
    // and read through aligned dwords, so W needs 4 bytes.
    if (!aligned(W, q6 ? 4 : 16))
        return fail(MQ_ERR_ALIGN, "%s: W=%p is not %d-byte aligned", fn, W, q6 ? 4 : 16);
    if (!aligned(q, 16)) return fail(MQ_ERR_ALIGN, "%s: q=%p is not 16-byte aligned", fn, (const void *)q);
    if (!aligned(d, 16)) return fail(MQ_ERR_ALIGN, "%s: d=%p is not 16-byte aligned", fn, (const void *)d);
    if (s && !aligned(s, 16)) return fail(MQ_ERR_ALIGN, "%s: s=%p is not 16-byte aligned", fn, (const void *)s);
    if (!aligned(out, 4)) return fail(MQ_ERR_ALIGN, "%s: out=%p is not 4-byte aligned", fn, (const void *)out);
    const Kern kern = matmul_kernel(fmt, M, N, K, path);
    // the split-K part is required; the full plan's bytes also enable the
    // Q6_K expansion
    if (int rc = check_ws(fn, ws, ws_bytes, ws ? split_ws_bytes(fmt, kern, M, N, K) : 0)) return rc;
    const bool x = expand && ws && q6k_expands(fmt, kern, M, N, K) &&
                   (uint64_t)ws_bytes >= (uint64_t)gemm_ws_bytes(fmt, kern, M, N, K);
    if (int rc = check_device()) return rc;

    const auto *Wb = static_cast<const uint8_t *>(W);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const mq::Ws w{ws, (size_t)ws_bytes};
    const int m = (int)M, n = (int)N, k = (int)K;
    hipError_t e;
    if (x) {
        // expand W into the workspace, then the expansion-plane GEMM with its
        // split-K sums after the planes (the expansion launches without the
        // timing hook, which stays for the GEMM)
        auto *lo = static_cast<int8_t *>(ws);
        int8_t *hi = lo + round256((size_t)N * (size_t)K);
        auto *dw = reinterpret_cast<float *>(hi + round256((size_t)N * (size_t)K));
        const size_t pb = q6k_planes_bytes(N, K);
        e = mq::launch_expand_q6k(Wb, N, K, lo, hi, dw, st);
        if (e == hipSuccess)
            e = mq::launch_gemm_q6k_x(lo, hi, dw, q, d, m, n, k, out,
                                      mq::Ws{static_cast<uint8_t *>(ws) + pb, (size_t)ws_bytes - pb}, st);
    } else if (q6 && kern == Kern::GEMV)
        e = mq::launch_gemv_q6k(Wb, q, d, m, n, k, out, st);
    else if (q6 && kern == Kern::GEMM_SMALL)
        e = mq::launch_gemm_q6k_small(Wb, q, d, m, n, k, out, w, st);
    else if (q6)
        e = mq::launch_gemm_q6k(Wb, q, d, m, n, k, out, w, st);
    else if (fmt == Fmt::Q5K && kern == Kern::GEMV)
        e = mq::launch_gemv_q5k(Wb, q, d, s, m, n, k, out, st);
    else if (fmt == Fmt::Q5K && kern == Kern::GEMM_SMALL)
        e = mq::launch_gemm_q5k_small(Wb, q, d, s, m, n, k, out, w, st);
    else if (fmt == Fmt::Q5K)
        e = mq::launch_gemm_q5k(Wb, q, d, s, m, n, k, out, w, st);
    else if (kern == Kern::GEMV)
        e = mq::launch_gemv_q4k(Wb, q, d, s, m, n, k, out, st);
    else if (kern == Kern::GEMM_SMALL)
        e = mq::launch_gemm_q4k_small(Wb, q, d, s, m, n, k, out, w, st);
    else
        e = mq::launch_gemm_q4k(Wb, q, d, s, m, n, k, out, w, st);
    return launched(e, fn);
}

// Shared checks of a GEMM-only matmul over registration-time planes.
int check_gemm_shape(const char *fn, const int8_t *q, const float *d, float *out, int64_t M, int64_t N,
                     int64_t K)
{
    if (!q) return fail(MQ_ERR_INVALID_ARG, "%s: q is NULL", fn);
    if (!d) return fail(MQ_ERR_INVALID_ARG, "%s: d is NULL", fn);
    if (!out) return fail(MQ_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (M <= 0) return fail(MQ_ERR_INVALID_ARG, "%s: M=%lld must be positive", fn, (long long)M);
    if (N <= 0) return fail(MQ_ERR_INVALID_ARG, "%s: N=%lld must be positive", fn, (long long)N);
    if (int rc = check_K(K, fn)) return rc;
    if (M > kMaxRows || N > kMaxRows)
        return fail(MQ_ERR_SHAPE, "%s: M=%lld, N=%lld: each must be at most %lld", fn,
                    (long long)M, (long long)N, (long long)kMaxRows);
    if (((M + 127) / 128) * ((N + 127) / 128) > kMaxDim)
        return fail(MQ_ERR_SHAPE, "%s: M=%lld x N=%lld needs too many tiles", fn, (long long)M, (long long)N);
    if (!aligned(q, 16)) return fail(MQ_ERR_ALIGN, "%s: q=%p is not 16-byte aligned", fn, (const void *)q);
    if (!aligned(d, 16)) return fail(MQ_ERR_ALIGN, "%s: d=%p is not 16-byte aligned", fn, (const void *)d);
    if (!aligned(out, 4)) return fail(MQ_ERR_ALIGN, "%s: out=%p is not 4-byte aligned", fn, (const void *)out);
    return MQ_OK;
}

// Shared checks of a plane builder reading N rows of K.
int check_planes(const char *fn, const void *W, int64_t N, int64_t K, int align)
{
    if (!W) return fail(MQ_ERR_INVALID_ARG, "%s: W is NULL", fn);
    if (N <= 0) return fail(MQ_ERR_INVALID_ARG, "%s: N=%lld must be positive", fn, (long long)N);
    if (int rc = check_K(K, fn)) return rc;
    if (N > kMaxRows) return fail(MQ_ERR_SHAPE, "%s: N=%lld exceeds %lld", fn, (long long)N, (long long)kMaxRows);
    if (N * (K / 256) > kMaxDim * 4)
        return fail(MQ_ERR_SHAPE, "%s: N=%lld x K=%lld has too many blocks", fn, (long long)N, (long long)K);
    if (!aligned(W, align)) return fail(MQ_ERR_ALIGN, "%s: W=%p is not %d-byte aligned", fn, W, align);
    return MQ_OK;
}

// Shape and path checks shared by the fused FFN and its workspace query.
int check_ffn_shape(const char *fn, int64_t M, int64_t N, int64_t K, int path)
{
    if (M <= 0) return fail(MQ_ERR_INVALID_ARG, "%s: M=%lld must be positive", fn, (long long)M);
    if (N <= 0 || N % 256 != 0)
        return fail(MQ_ERR_SHAPE, "%s: N=%lld must be a positive multiple of 256", fn, (long long)N);
    if (int rc = check_K(K, fn)) return rc;
    if (M > kMaxRows || N > kMaxRows)
        return fail(MQ_ERR_SHAPE, "%s: M=%lld, N=%lld: each must be at most %lld", fn, (long long)M,
                    (long long)N, (long long)kMaxRows);
    if (path != MQ_PATH_AUTO && path != MQ_PATH_GEMV && path != MQ_PATH_GEMM)
        return fail(MQ_ERR_INVALID_ARG, "%s: path=%d is not MQ_PATH_AUTO/GEMV/GEMM", fn, path);
    if (path == MQ_PATH_GEMV && M > mq::FFN_GEMV_MAX_M)
        return fail(MQ_ERR_INVALID_ARG, "%s: path=MQ_PATH_GEMV needs M <= %d, got M=%lld", fn,
                    mq::FFN_GEMV_MAX_M, (long long)M);
    const int64_t tiles = ((M + 127) / 128) * (N / 64);
    if (tiles > kMaxDim)
        return fail(MQ_ERR_SHAPE, "%s: M=%lld x N=%lld needs too many tiles", fn, (long long)M, (long long)N);
    return MQ_OK;
}

// The fused FFN's plan. With a workspace: the GEMV pass (path GEMV, or AUTO
// up to FFN_AUTO_M tokens) or the two GEMMs (up to FFN_TWO_PASS_MAX_M
// tokens) write g and u, then the SwiGLU quantizer; above that the
// one-launch GEMM. Without one: the one-launch GEMM at every M (path GEMV
// needs the workspace).
struct FfnPlan {
    bool two_pass, gemv;
    size_t bytes;   // workspace of the two-pass form
};
FfnPlan ffn_plan(int64_t M, int64_t N, int64_t K, int path)
{
    const bool gemv = path == MQ_PATH_GEMV || (path == MQ_PATH_AUTO && M <= mq::FFN_AUTO_M);
    const bool two_pass = gemv || M <= FFN_TWO_PASS_MAX_M;
    return {two_pass, gemv, two_pass ? mq::ffn_two_pass_bytes((int)M, (int)N, (int)K, gemv) : 0};
}

int ffn(const void *Wg, const void *Wu, const int8_t *q, const float *d, const float *s, int64_t M,
        int64_t N, int64_t K, int8_t *qo, float *do_, float *so, float *y, void *ws, int64_t ws_bytes,
        void *stream, int path)
{
    const char *fn = "mq_ffn_q4k";
    if (!Wg) return fail(MQ_ERR_INVALID_ARG, "%s: Wg is NULL", fn);
    if (!Wu) return fail(MQ_ERR_INVALID_ARG, "%s: Wu is NULL", fn);
    if (!q) return fail(MQ_ERR_INVALID_ARG, "%s: q is NULL", fn);
    if (!d) return fail(MQ_ERR_INVALID_ARG, "%s: d is NULL", fn);
    if (!s) return fail(MQ_ERR_INVALID_ARG, "%s: s is NULL (the Q4_K min term needs it)", fn);
    if (!qo) return fail(MQ_ERR_INVALID_ARG, "%s: qo is NULL", fn);
    if (!do_) return fail(MQ_ERR_INVALID_ARG, "%s: do_ is NULL", fn);
    if (!so) return fail(MQ_ERR_INVALID_ARG, "%s: so is NULL", fn);
    if (int rc = check_ffn_shape(fn, M, N, K, path)) return rc;
    if (!aligned(Wg, 16)) return fail(MQ_ERR_ALIGN, "%s: Wg=%p is not 16-byte aligned", fn, Wg);
    if (!aligned(Wu, 16)) return fail(MQ_ERR_ALIGN, "%s: Wu=%p is not 16-byte aligned", fn, Wu);
    if (!aligned(q, 16)) return fail(MQ_ERR_ALIGN, "%s: q=%p is not 16-byte aligned", fn, (const void *)q);
    if (!aligned(d, 16)) return fail(MQ_ERR_ALIGN, "%s: d=%p is not 16-byte aligned", fn, (const void *)d);
    if (!aligned(s, 16)) return fail(MQ_ERR_ALIGN, "%s: s=%p is not 16-byte aligned", fn, (const void *)s);
    if (!aligned(qo, 16)) return fail(MQ_ERR_ALIGN, "%s: qo=%p is not 16-byte aligned", fn, (const void *)qo);
    if (!aligned(do_, 16)) return fail(MQ_ERR_ALIGN, "%s: do_=%p is not 16-byte aligned", fn, (const void *)do_);
    if (!aligned(so, 16)) return fail(MQ_ERR_ALIGN, "%s: so=%p is not 16-byte aligned", fn, (const void *)so);
    if (y && !aligned(y, 16)) return fail(MQ_ERR_ALIGN, "%s: y=%p is not 16-byte aligned", fn, (const void *)y);
    const FfnPlan plan = ffn_plan(M, N, K, path);
    if (!ws && path == MQ_PATH_GEMV)
        return fail(MQ_ERR_WORKSPACE, "%s: path=MQ_PATH_GEMV needs a workspace of %llu bytes (ws is NULL)", fn,
                    (unsigned long long)plan.bytes);
    if (int rc = check_ws(fn, ws, ws_bytes, ws ? plan.bytes : 0)) return rc;
    if (int rc = check_device()) return rc;
    const auto *Wgb = static_cast<const uint8_t *>(Wg);
    const auto *Wub = static_cast<const uint8_t *>(Wu);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e =
        ws && plan.two_pass
            ? mq::launch_ffn_q4k_two_pass(Wgb, Wub, q, d, s, (int)M, (int)N, (int)K, qo, do_, so, y, plan.gemv,
                                          mq::Ws{ws, (size_t)ws_bytes}, st)
            : mq::launch_gemm_q4k_ffn(Wgb, Wub, q, d, s, (int)M, (int)N, (int)K, qo, do_, so, y, st);
    return launched(e, fn);
}

// The split-K workspace of mq_matmul_q6k_static: a file-scope device array,
// one copy per GPU the library runs on, held until the process ends. In host
// code `scratch` names a host-side stand-in, not the device memory: kernels
// get the address hipGetSymbolAddress returns for the current device, taken
// once per device (scratch_ptr) and used everywhere instead of the name.
constexpr size_t kScratchBytes = MQ_STATIC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (nullptr and a message on failure).
int scratch_ptr(const char *fn, void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(MQ_ERR_DEVICE, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MQ_ERR_DEVICE, "%s: device ordinal %d out of range", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MQ_ERR_DEVICE, "%s: hipGetSymbolAddress(scratch) on device %d failed: %s", fn, dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MQ_OK;
}

} // namespace

extern "C" {

int mq_quantize_act(const float *x, int64_t M, int64_t K, int64_t ldx, int8_t *q,
                    float *d, float *s, void *stream)
{
    g_err[0] = '\0';
    const char *fn = "mq_quantize_act";
    if (!x) return fail(MQ_ERR_INVALID_ARG, "%s: x is NULL", fn);
    if (!q) return fail(MQ_ERR_INVALID_ARG, "%s: q is NULL", fn);
    if (!d) return fail(MQ_ERR_INVALID_ARG, "%s: d is NULL", fn);
    if (!s) return fail(MQ_ERR_INVALID_ARG, "%s: s is NULL", fn);
    if (M <= 0) return fail(MQ_ERR_INVALID_ARG, "%s: M=%lld must be positive", fn, (long long)M);
    if (int rc = check_K(K, fn)) return rc;
    if (ldx < K) return fail(MQ_ERR_SHAPE, "%s: ldx=%lld is smaller than K=%lld", fn, (long long)ldx, (long long)K);
    if (M > kMaxRows) return fail(MQ_ERR_SHAPE, "%s: M=%lld exceeds %lld", fn, (long long)M, (long long)kMaxRows);
    // the scalar path uses 32 threads per block: the grid must fit in 2^31-1 workgroups
    if (M > (kMaxDim * 256 / 32) / (K / 32))
        return fail(MQ_ERR_SHAPE, "%s: M=%lld x K=%lld is too large for one launch", fn, (long long)M, (long long)K);
    if (!aligned(x, 4)) return fail(MQ_ERR_ALIGN, "%s: x=%p is not 4-byte aligned", fn, (const void *)x);
    if (!aligned(q, 16)) return fail(MQ_ERR_ALIGN, "%s: q=%p is not 16-byte aligned", fn, (const void *)q);
    if (!aligned(d, 16)) return fail(MQ_ERR_ALIGN, "%s: d=%p is not 16-byte aligned", fn, (const void *)d);
    if (!aligned(s, 16)) return fail(MQ_ERR_ALIGN, "%s: s=%p is not 16-byte aligned", fn, (const void *)s);
    if (int rc = check_device()) return rc;
    return launched(mq::launch_quantize(x, M, K, ldx, q, d, s, static_cast<hipStream_t>(stream)), fn);
}

int mq_rmsnorm_quantize(const float *x, const float *w, int64_t M, int64_t K, int64_t ldx, float eps,
                        int8_t *q, float *d, float *s, float *y, void *stream)
{
    g_err[0] = '\0';
    drop_timing();
    const char *fn = "mq_rmsnorm_quantize";
    if (!x) return fail(MQ_ERR_INVALID_ARG, "%s: x is NULL", fn);
    if (!w) return fail(MQ_ERR_INVALID_ARG, "%s: w is NULL", fn);
    if (!q) return fail(MQ_ERR_INVALID_ARG, "%s: q is NULL", fn);
    if (!d) return fail(MQ_ERR_INVALID_ARG, "%s: d is NULL", fn);
    if (!s) return fail(MQ_ERR_INVALID_ARG, "%s: s is NULL", fn);
    if (M <= 0) return fail(MQ_ERR_INVALID_ARG, "%s: M=%lld must be positive", fn, (long long)M);
    if (!(eps >= 0.0f) || eps > 3.4e38f)
        return fail(MQ_ERR_INVALID_ARG, "%s: eps=%g must be finite and >= 0", fn, (double)eps);
    if (int rc = check_K(K, fn)) return rc;
    if (ldx < K) return fail(MQ_ERR_SHAPE, "%s: ldx=%lld is smaller than K=%lld", fn, (long long)ldx, (long long)K);
    if (ldx % 4 != 0) return fail(MQ_ERR_ALIGN, "%s: ldx=%lld is not a multiple of 4", fn, (long long)ldx);
    if (M > kMaxRows) return fail(MQ_ERR_SHAPE, "%s: M=%lld exceeds %lld", fn, (long long)M, (long long)kMaxRows);
    if (!aligned(x, 16)) return fail(MQ_ERR_ALIGN, "%s: x=%p is not 16-byte aligned", fn, (const void *)x);
    if (!aligned(w, 16)) return fail(MQ_ERR_ALIGN, "%s: w=%p is not 16-byte aligned", fn, (const void *)w);
    if (!aligned(q, 16)) return fail(MQ_ERR_ALIGN, "%s: q=%p is not 16-byte aligned", fn, (const void *)q);
    if (!aligned(d, 16)) return fail(MQ_ERR_ALIGN, "%s: d=%p is not 16-byte aligned", fn, (const void *)d);
    if (!aligned(s, 16)) return fail(MQ_ERR_ALIGN, "%s: s=%p is not 16-byte aligned", fn, (const void *)s);
    if (y && !aligned(y, 16)) return fail(MQ_ERR_ALIGN, "%s: y=%p is not 16-byte aligned", fn, (const void *)y);
    if (int rc = check_device()) return rc;
    return launched(mq::launch_rmsnorm_quantize(x, w, M, K, ldx, eps, q, d, s, y,
                                                static_cast<hipStream_t>(stream)), fn);
}

int mq_swiglu_quantize(const float *g, const float *u, int64_t M, int64_t K, int64_t ldg, int64_t ldu,
                       int8_t *q, float *d, float *s, float *y, void *stream)
{
    g_err[0] = '\0';
    drop_timing();
    const char *fn = "mq_swiglu_quantize";
    if (!g) return fail(MQ_ERR_INVALID_ARG, "%s: g is NULL", fn);
    if (!u) return fail(MQ_ERR_INVALID_ARG, "%s: u is NULL", fn);
    if (!q) return fail(MQ_ERR_INVALID_ARG, "%s: q is NULL", fn);
    if (!d) return fail(MQ_ERR_INVALID_ARG, "%s: d is NULL", fn);
    if (!s) return fail(MQ_ERR_INVALID_ARG, "%s: s is NULL", fn);
    if (M <= 0) return fail(MQ_ERR_INVALID_ARG, "%s: M=%lld must be positive", fn, (long long)M);
    if (int rc = check_K(K, fn)) return rc;
    if (ldg < K) return fail(MQ_ERR_SHAPE, "%s: ldg=%lld is smaller than K=%lld", fn, (long long)ldg, (long long)K);
    if (ldu < K) return fail(MQ_ERR_SHAPE, "%s: ldu=%lld is smaller than K=%lld", fn, (long long)ldu, (long long)K);
    if (ldg % 4 != 0) return fail(MQ_ERR_ALIGN, "%s: ldg=%lld is not a multiple of 4", fn, (long long)ldg);
    if (ldu % 4 != 0) return fail(MQ_ERR_ALIGN, "%s: ldu=%lld is not a multiple of 4", fn, (long long)ldu);
    if (M > kMaxRows) return fail(MQ_ERR_SHAPE, "%s: M=%lld exceeds %lld", fn, (long long)M, (long long)kMaxRows);
    // 8 threads per 32-value block: the grid must fit in 2^31-1 workgroups
    if (M > (kMaxDim * 256 / 8) / (K / 32))
        return fail(MQ_ERR_SHAPE, "%s: M=%lld x K=%lld is too large for one launch", fn, (long long)M, (long long)K);
    if (!aligned(g, 16)) return fail(MQ_ERR_ALIGN, "%s: g=%p is not 16-byte aligned", fn, (const void *)g);
    if (!aligned(u, 16)) return fail(MQ_ERR_ALIGN, "%s: u=%p is not 16-byte aligned", fn, (const void *)u);
    if (!aligned(q, 16)) return fail(MQ_ERR_ALIGN, "%s: q=%p is not 16-byte aligned", fn, (const void *)q);
    if (!aligned(d, 16)) return fail(MQ_ERR_ALIGN, "%s: d=%p is not 16-byte aligned", fn, (const void *)d);
    if (!aligned(s, 16)) return fail(MQ_ERR_ALIGN, "%s: s=%p is not 16-byte aligned", fn, (const void *)s);
    if (y && !aligned(y, 16)) return fail(MQ_ERR_ALIGN, "%s: y=%p is not 16-byte aligned", fn, (const void *)y);
    if (int rc = check_device()) return rc;
    return launched(mq::launch_swiglu_quantize(g, u, M, K, ldg, ldu, q, d, s, y,
                                               static_cast<hipStream_t>(stream)), fn);
}

int mq_matmul_workspace(int fmt, int64_t M, int64_t N, int64_t K, int path, int64_t *bytes)
{
    g_err[0] = '\0';
    if (!bytes) return fail(MQ_ERR_INVALID_ARG, "mq_matmul_workspace: bytes is NULL");
    *bytes = 0;
    if (fmt != MQ_FMT_Q4K && fmt != MQ_FMT_Q5K && fmt != MQ_FMT_Q6K)
        return fail(MQ_ERR_INVALID_ARG, "mq_matmul_workspace: fmt=%d is not MQ_FMT_Q4K/Q5K/Q6K", fmt);
    const Fmt f = static_cast<Fmt>(fmt);
    if (int rc = check_matmul_shape(fmt_fn(f), M, N, K, path)) return rc;
    *bytes = (int64_t)gemm_ws_bytes(f, matmul_kernel(f, M, N, K, path), M, N, K);
    return MQ_OK;
}

int mq_ffn_q4k_workspace(int64_t M, int64_t N, int64_t K, int path, int64_t *bytes)
{
    g_err[0] = '\0';
    if (!bytes) return fail(MQ_ERR_INVALID_ARG, "mq_ffn_q4k_workspace: bytes is NULL");
    *bytes = 0;
    if (int rc = check_ffn_shape("mq_ffn_q4k", M, N, K, path)) return rc;
    *bytes = (int64_t)ffn_plan(M, N, K, path).bytes;
    return MQ_OK;
}

int mq_matmul_q4k(const void *W, const int8_t *q, const float *d, const float *s, int64_t M,
                  int64_t N, int64_t K, float *out, void *stream)
{
    g_err[0] = '\0';
    return matmul(Fmt::Q4K, W, q, d, s, M, N, K, out, nullptr, 0, stream, MQ_PATH_AUTO);
}

int mq_matmul_q5k(const void *W, const int8_t *q, const float *d, const float *s, int64_t M,
                  int64_t N, int64_t K, float *out, void *stream)
{
    g_err[0] = '\0';
    return matmul(Fmt::Q5K, W, q, d, s, M, N, K, out, nullptr, 0, stream, MQ_PATH_AUTO);
}

int mq_matmul_q6k(const void *W, const int8_t *q, const float *d, const float *s, int64_t M,
                  int64_t N, int64_t K, float *out, void *stream)
{
    g_err[0] = '\0';
    return matmul(Fmt::Q6K, W, q, d, s, M, N, K, out, nullptr, 0, stream, MQ_PATH_AUTO);
}

int mq_matmul_q4k_ex(const void *W, const int8_t *q, const float *d, const float *s, int64_t M,
                     int64_t N, int64_t K, float *out, void *stream, int path)
{
    g_err[0] = '\0';
    return matmul(Fmt::Q4K, W, q, d, s, M, N, K, out, nullptr, 0, stream, path);
}

int mq_matmul_q5k_ex(const void *W, const int8_t *q, const float *d, const float *s, int64_t M,
                     int64_t N, int64_t K, float *out, void *stream, int path)
{
    g_err[0] = '\0';
    return matmul(Fmt::Q5K, W, q, d, s, M, N, K, out, nullptr, 0, stream, path);
}

int mq_matmul_q6k_ex(const void *W, const int8_t *q, const float *d, const float *s, int64_t M,
                     int64_t N, int64_t K, float *out, void *stream, int path)
{
    g_err[0] = '\0';
    return matmul(Fmt::Q6K, W, q, d, s, M, N, K, out, nullptr, 0, stream, path);
}

int mq_matmul_q4k_ws(const void *W, const int8_t *q, const float *d, const float *s, int64_t M,
                     int64_t N, int64_t K, float *out, void *ws, int64_t ws_bytes, void *stream, int path)
{
    g_err[0] = '\0';
    return matmul(Fmt::Q4K, W, q, d, s, M, N, K, out, ws, ws_bytes, stream, path);
}

int mq_matmul_q5k_ws(const void *W, const int8_t *q, const float *d, const float *s, int64_t M,
                     int64_t N, int64_t K, float *out, void *ws, int64_t ws_bytes, void *stream, int path)
{
    g_err[0] = '\0';
    return matmul(Fmt::Q5K, W, q, d, s, M, N, K, out, ws, ws_bytes, stream, path);
}

int mq_matmul_q6k_ws(const void *W, const int8_t *q, const float *d, const float *s, int64_t M,
                     int64_t N, int64_t K, float *out, void *ws, int64_t ws_bytes, void *stream, int path)
{
    g_err[0] = '\0';
    return matmul(Fmt::Q6K, W, q, d, s, M, N, K, out, ws, ws_bytes, stream, path);
}

int mq_ffn_q4k(const void *Wg, const void *Wu, const int8_t *q, const float *d, const float *s, int64_t M,
               int64_t N, int64_t K, int8_t *qo, float *do_, float *so, float *y, void *stream)
{
    g_err[0] = '\0';
    return ffn(Wg, Wu, q, d, s, M, N, K, qo, do_, so, y, nullptr, 0, stream, MQ_PATH_AUTO);
}

int mq_ffn_q4k_ex(const void *Wg, const void *Wu, const int8_t *q, const float *d, const float *s, int64_t M,
                  int64_t N, int64_t K, int8_t *qo, float *do_, float *so, float *y, void *stream, int path)
{
    g_err[0] = '\0';
    return ffn(Wg, Wu, q, d, s, M, N, K, qo, do_, so, y, nullptr, 0, stream, path);
}

int mq_ffn_q4k_ws(const void *Wg, const void *Wu, const int8_t *q, const float *d, const float *s, int64_t M,
                  int64_t N, int64_t K, int8_t *qo, float *do_, float *so, float *y, void *ws, int64_t ws_bytes,
                  void *stream, int path)
{
    g_err[0] = '\0';
    return ffn(Wg, Wu, q, d, s, M, N, K, qo, do_, so, y, ws, ws_bytes, stream, path);
}

int mq_expand_q6k(const void *W, int64_t N, int64_t K, int8_t *lo, int8_t *hi, float *dw, void *stream)
{
    g_err[0] = '\0';
    drop_timing();
    const char *fn = "mq_expand_q6k";
    if (int rc = check_planes(fn, W, N, K, 4)) return rc;
    if (!lo) return fail(MQ_ERR_INVALID_ARG, "%s: lo is NULL", fn);
    if (!hi) return fail(MQ_ERR_INVALID_ARG, "%s: hi is NULL", fn);
    if (!dw) return fail(MQ_ERR_INVALID_ARG, "%s: dw is NULL", fn);
    if (!aligned(lo, 16)) return fail(MQ_ERR_ALIGN, "%s: lo=%p is not 16-byte aligned", fn, (void *)lo);
    if (!aligned(hi, 16)) return fail(MQ_ERR_ALIGN, "%s: hi=%p is not 16-byte aligned", fn, (void *)hi);
    if (!aligned(dw, 16)) return fail(MQ_ERR_ALIGN, "%s: dw=%p is not 16-byte aligned", fn, (void *)dw);
    if (int rc = check_device()) return rc;
    return launched(mq::launch_expand_q6k(static_cast<const uint8_t *>(W), N, K, lo, hi, dw,
                                          static_cast<hipStream_t>(stream)), fn);
}

int mq_matmul_q6k_x(const int8_t *lo, const int8_t *hi, const float *dw, const int8_t *q, const float *d,
                    int64_t M, int64_t N, int64_t K, float *out, void *ws, int64_t ws_bytes, void *stream)
{
    g_err[0] = '\0';
    const char *fn = "mq_matmul_q6k_x";
    if (!lo) return fail(MQ_ERR_INVALID_ARG, "%s: lo is NULL", fn);
    if (!hi) return fail(MQ_ERR_INVALID_ARG, "%s: hi is NULL", fn);
    if (!dw) return fail(MQ_ERR_INVALID_ARG, "%s: dw is NULL", fn);
    if (int rc = check_gemm_shape(fn, q, d, out, M, N, K)) return rc;
    if (!aligned(lo, 16)) return fail(MQ_ERR_ALIGN, "%s: lo=%p is not 16-byte aligned", fn, (const void *)lo);
    if (!aligned(hi, 16)) return fail(MQ_ERR_ALIGN, "%s: hi=%p is not 16-byte aligned", fn, (const void *)hi);
    if (!aligned(dw, 4)) return fail(MQ_ERR_ALIGN, "%s: dw=%p is not 4-byte aligned", fn, (const void *)dw);
    const Kern kern = M <= mq::GEMM_SMALL_M_Q6K ? Kern::GEMM_SMALL : Kern::GEMM;
    if (int rc = check_ws(fn, ws, ws_bytes, ws ? split_ws_bytes(Fmt::Q6K, kern, M, N, K) : 0)) return rc;
    if (int rc = check_device()) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const mq::Ws w{ws, (size_t)ws_bytes};
    const int m = (int)M, n = (int)N, k = (int)K;
    const hipError_t e = kern == Kern::GEMM_SMALL ? mq::launch_gemm_q6k_x_small(lo, hi, dw, q, d, m, n, k, out, w, st)
                                                  : mq::launch_gemm_q6k_x(lo, hi, dw, q, d, m, n, k, out, w, st);
    return launched(e, fn);
}

int mq_dsc_q4k(const void *W, int64_t N, int64_t K, float *fw, float *fm, void *stream)
{
    g_err[0] = '\0';
    drop_timing();
    const char *fn = "mq_dsc_q4k";
    if (int rc = check_planes(fn, W, N, K, 16)) return rc;
    if (!fw) return fail(MQ_ERR_INVALID_ARG, "%s: fw is NULL", fn);
    if (!fm) return fail(MQ_ERR_INVALID_ARG, "%s: fm is NULL", fn);
    if (!aligned(fw, 16)) return fail(MQ_ERR_ALIGN, "%s: fw=%p is not 16-byte aligned", fn, (void *)fw);
    if (!aligned(fm, 16)) return fail(MQ_ERR_ALIGN, "%s: fm=%p is not 16-byte aligned", fn, (void *)fm);
    if (int rc = check_device()) return rc;
    return launched(mq::launch_dsc_q4k(static_cast<const uint8_t *>(W), N, K, fw, fm,
                                       static_cast<hipStream_t>(stream)), fn);
}

int mq_matmul_q4k_dsc(const void *W, const float *fw, const float *fm, const int8_t *q, const float *d,
                      const float *s, int64_t M, int64_t N, int64_t K, float *out, void *ws, int64_t ws_bytes,
                      void *stream)
{
    g_err[0] = '\0';
    const char *fn = "mq_matmul_q4k_dsc";
    if (!W) return fail(MQ_ERR_INVALID_ARG, "%s: W is NULL", fn);
    if (!fw) return fail(MQ_ERR_INVALID_ARG, "%s: fw is NULL", fn);
    if (!fm) return fail(MQ_ERR_INVALID_ARG, "%s: fm is NULL", fn);
    if (!s) return fail(MQ_ERR_INVALID_ARG, "%s: s is NULL (the min term needs it)", fn);
    if (int rc = check_gemm_shape(fn, q, d, out, M, N, K)) return rc;
    if (!aligned(W, 16)) return fail(MQ_ERR_ALIGN, "%s: W=%p is not 16-byte aligned", fn, W);
    if (!aligned(fw, 16)) return fail(MQ_ERR_ALIGN, "%s: fw=%p is not 16-byte aligned", fn, (const void *)fw);
    if (!aligned(fm, 16)) return fail(MQ_ERR_ALIGN, "%s: fm=%p is not 16-byte aligned", fn, (const void *)fm);
    if (!aligned(s, 16)) return fail(MQ_ERR_ALIGN, "%s: s=%p is not 16-byte aligned", fn, (const void *)s);
    const Kern kern = M <= mq::GEMM_SMALL_M_Q4K ? Kern::GEMM_SMALL : Kern::GEMM;
    if (int rc = check_ws(fn, ws, ws_bytes, ws ? split_ws_bytes(Fmt::Q4K, kern, M, N, K) : 0)) return rc;
    if (int rc = check_device()) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const mq::Ws w{ws, (size_t)ws_bytes};
    const auto *Wb = static_cast<const uint8_t *>(W);
    const int m = (int)M, n = (int)N, k = (int)K;
    const hipError_t e = kern == Kern::GEMM_SMALL
                             ? mq::launch_gemm_q4k_dsc_small(Wb, fw, fm, q, d, s, m, n, k, out, w, st)
                             : mq::launch_gemm_q4k_dsc(Wb, fw, fm, q, d, s, m, n, k, out, w, st);
    return launched(e, fn);
}

int mq_matmul_q6k_static(const void *W, const int8_t *q, const float *d, const float *s, int64_t M,
                         int64_t N, int64_t K, float *out, void *stream)
{
    g_err[0] = '\0';
    const char *fn = "mq_matmul_q6k_static";
    // the checks of the call, then the size of the plan against the array
    if (int rc = check_matmul_shape(fn, M, N, K, MQ_PATH_AUTO)) return rc;
    const size_t need = split_ws_bytes(Fmt::Q6K, matmul_kernel(Fmt::Q6K, M, N, K, MQ_PATH_AUTO), M, N, K);
    if (need > kScratchBytes)
        return fail(MQ_ERR_WORKSPACE, "%s: M=%lld N=%lld K=%lld needs %llu bytes of scratch; the static array "
                    "holds %llu (use mq_matmul_q6k_ws)", fn, (long long)M, (long long)N, (long long)K,
                    (unsigned long long)need, (unsigned long long)kScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        if (int rc = check_device()) return rc;
        if (int rc = scratch_ptr(fn, &ws)) return rc;
    }
    return matmul(Fmt::Q6K, W, q, d, s, M, N, K, out, ws, ws ? (int64_t)kScratchBytes : 0, stream, MQ_PATH_AUTO,
                  false);
}

int mq_time_next_kernel(void *start_event, void *stop_event)
{
    g_err[0] = '\0';
    mq::kernel_events() = mq::KernelEvents{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
    return MQ_OK;
}

int64_t mq_gemv_max_m(void) { return mq::GEMV_MAX_M; }

const char *mq_last_error(void) { return g_err; }

int mq_abi_version(void) { return MQ_ABI_VERSION; }

} // extern "C"
