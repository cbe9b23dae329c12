// Kernel launchers of libmq (internal). Arguments are validated by the C-ABI
// layer before these are called; each launcher only enqueues work on `st`.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <cstddef>

namespace mq {

// Kernel-boundary timing (mq_time_next_kernel): when a pair of events is set
// for the calling thread, the next matmul or quantizer kernel launched
// through launch() records them at its own dispatch start and end
// (hipExtLaunchKernel) and the pair is cleared. Defined in mq_api.cpp.
struct KernelEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
KernelEvents &kernel_events();

// kernel<<<grid, block, lds, st>>>(args...), or with the thread's timing
// events when set. Like <<<>>>, it leaves a launch error for the caller's
// hipGetLastError().
template <class F, class... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st, Args... args)
{
    KernelEvents &e = kernel_events();
    if (e.start || e.stop) {
        const KernelEvents ev = e;
        e = KernelEvents{};
        hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev.start, ev.stop, 0u, args...);
    } else {
        kernel<<<grid, block, lds, st>>>(args...);
    }
}

// Largest token count the GEMV kernels serve (MQ_PATH_GEMV), and the fused
// FFN GEMV's.
constexpr int GEMV_MAX_M = 16;
constexpr int FFN_GEMV_MAX_M = 8;
// MQ_PATH_AUTO: GEMV or GEMM, at the crossovers measured on MI355X (GPU time
// per call, weights streamed from HBM). The GEMV's cost grows with M (its dot
// products are VALU work per token) while the 32-token GEMM stays near its
// floor (16-25 us for Q4_K at K = 3584..8192). Where the persistent stream
// takes the tokens (q4k_stream_fits / q5k_stream_fits) the GEMV keeps the lead
// while M*N*K stays below about 4.2e8 for Q4_K (at 18944 x 3584: M = 6 20.7
// against 24.7 us, M = 8 a tie; at 14336 x 4096, M = 8: 23.4 against 21.3)
// and through 8 tokens of the 7B shapes for Q5_K (18944 x 3584, M = 8: 23.3
// against 30.3 us). Otherwise the row-grid GEMV serves while M*N*K <= 2.6e8
// (Q4_K; 8192 x 8192, M = 4: 28.9 against 24.1 us) or 3.3e8 (Q5_K, whose
// GEMM is slower: M = 4 26.4 against 28.2 us). Q6_K runs the GEMV for
// M <= 4, and up to 8 tokens where its LDS ring kernel takes the plane while
// M*N*K <= 5.5e8 (18944 x 3584, M = 8: 33.5 against 42.5 us; the down
// projection's K = 18944 leaves the ring kernel at M = 3, and its register
// kernel loses from M = 6: 55.2 against 46.4 us).
bool q4k_stream_fits(int64_t M, int64_t K);
bool q5k_stream_fits(int64_t M, int64_t K);
bool q6k_stream_fits(int64_t M, int64_t K);
inline bool gemv_auto(bool q6, int64_t M, int64_t N, int64_t K)
{
    const double mnk = (double)M * (double)N * (double)K;
    if (q6)
        return M <= 4 || (M <= 8 && q6k_stream_fits(M, K) && mnk <= 5.5e8);
    return M <= 2 || (q4k_stream_fits(M, K) && mnk <= 4.2e8) || (M <= GEMV_MAX_M && mnk <= 2.6e8);
}
inline bool gemv_auto_q5k(int64_t M, int64_t N, int64_t K)
{
    const double mnk = (double)M * (double)N * (double)K;
    return M <= 2 || (q5k_stream_fits(M, K) && mnk <= 5.5e8) || (M <= GEMV_MAX_M && mnk <= 3.3e8);
}
constexpr int FFN_AUTO_M = 8;
// Above FFN_AUTO_M the FFN runs its two GEMMs and the SwiGLU quantizer as
// separate passes up to this token count, and the one-launch GEMM beyond.
// GPU time at 18944 x 3584: the one-launch GEMM's 128-token tiles cost about
// the same from 9 to 128 tokens (112-118 us); two passes took 51.5 us at
// M = 9, 80.1 at 64, 113.7 at 128; at 192 they were even (193 against 195)
// and at 256 and 3314 the one-launch GEMM was as fast or faster (197
// against 203, 1859 both) and keeps g and u out of memory.
#ifndef FFN_TWO_PASS_MAX_M
#define FFN_TWO_PASS_MAX_M 128
#endif
// The GEMMs run their small-M configuration (32-token tiles) up to these
// token counts: crossovers against the 128-token tiles by GPU time per call.
// Q4_K 18944 x 3584: M = 64 35.8 against 47.6 us, M = 80 56.2 against 49.0;
// Q5_K: M = 64 49.2 against 58.0, M = 80 63.0 against 59.3; Q6_K 3584 x
// 18944: M = 32 42.8 against 70.3, M = 48 72.6 against 71.2. (Rows of 3584
// favour the small tiles longer: Q4_K 3584 x 3584 at M = 128 23.4 against
// 25.0 us.)
constexpr int GEMM_SMALL_M_Q4K = 64;
constexpr int GEMM_SMALL_M_Q6K = 32;
constexpr int GEMM_SMALL_M_Q5K = 64;

hipError_t launch_quantize(const float *x, int64_t M, int64_t K, int64_t ldx,
                           int8_t *q, float *d, float *s, hipStream_t st);

hipError_t launch_gemv_q4k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           hipStream_t st);
hipError_t launch_gemv_q6k(const uint8_t *W, const int8_t *q, const float *d,
                           int M, int N, int K, float *out, hipStream_t st);
hipError_t launch_gemv_q5k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           hipStream_t st);

hipError_t launch_rmsnorm_quantize(const float *x, const float *w, int64_t M, int64_t K, int64_t ldx,
                                   float eps, int8_t *q, float *d, float *s, float *y, hipStream_t st);
hipError_t launch_swiglu_quantize(const float *g, const float *u, int64_t M, int64_t K, int64_t ldg,
                                  int64_t ldu, int8_t *q, float *d, float *s, float *y, hipStream_t st);

// The caller's device workspace for one call: split-K partial sums and the
// two-pass FFN's g and u. ptr == nullptr means none was given; the
// launchers then take their workspace-free plan (no split of K).
struct Ws {
    void *ptr = nullptr;
    size_t bytes = 0;
};

hipError_t launch_gemm_q4k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           const Ws &ws, hipStream_t st);
// Small-M configuration of the Q4_K GEMM (32 tokens x 256 rows per workgroup).
hipError_t launch_gemm_q4k_small(const uint8_t *W, const int8_t *q, const float *d,
                                 const float *s, int M, int N, int K, float *out,
                                 const Ws &ws, hipStream_t st);
// Small-M configuration of the Q6_K GEMM (32 tokens x 128 rows per workgroup).
hipError_t launch_gemm_q6k_small(const uint8_t *W, const int8_t *q, const float *d,
                                 int M, int N, int K, float *out, const Ws &ws, hipStream_t st);
hipError_t launch_gemm_q5k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           const Ws &ws, hipStream_t st);
// Small-M configuration of the Q5_K GEMM (32 tokens x 128 rows per workgroup).
hipError_t launch_gemm_q5k_small(const uint8_t *W, const int8_t *q, const float *d,
                                 const float *s, int M, int N, int K, float *out,
                                 const Ws &ws, hipStream_t st);
hipError_t launch_gemm_q4k_ffn(const uint8_t *Wg, const uint8_t *Wu, const int8_t *q, const float *d,
                               const float *s, int M, int N, int K, int8_t *qo, float *do_, float *so,
                               float *y, hipStream_t st);
// The gate and up matrices (N rows each) as one persistent stream of 2N rows
// over the shared plane: g = x Wg^T, u = x Wu^T (each M x N). Needs
// q4k_stream_fits(M, K) (else hipErrorInvalidValue).
// q4k_stream_fits(M, K): the persistent Q4_K stream takes M tokens at row
// length K.
hipError_t launch_gemv_q4k_pair(const uint8_t *Wg, const uint8_t *Wu, const int8_t *q, const float *d,
                                const float *s, int M, int N, int K, float *g, float *u, hipStream_t st);
// FFN up half in two passes: g and u into the caller's workspace (the GEMV
// when gemv is set, else the GEMM of the token count, whose split-K planes
// follow g and u in the workspace), then the SwiGLU quantizer.
// launch_gemm_q4k_ffn is the one-launch GEMM form. ffn_two_pass_bytes is
// the workspace it needs.
size_t ffn_two_pass_bytes(int M, int N, int K, bool gemv);
hipError_t launch_ffn_q4k_two_pass(const uint8_t *Wg, const uint8_t *Wu, const int8_t *q, const float *d,
                                   const float *s, int M, int N, int K, int8_t *qo, float *do_, float *so,
                                   float *y, bool gemv, const Ws &ws, hipStream_t st);
hipError_t launch_gemm_q6k(const uint8_t *W, const int8_t *q, const float *d,
                           int M, int N, int K, float *out, const Ws &ws, hipStream_t st);

// Registration-time planes (Q6_K expansion, Q4_K decoded scales) and the
// GEMMs that read them (the split choice of the raw-block GEMM of the same
// configuration).
hipError_t launch_expand_q6k(const uint8_t *W, int64_t N, int64_t K, int8_t *lo, int8_t *hi, float *dw,
                             hipStream_t st);
hipError_t launch_dsc_q4k(const uint8_t *W, int64_t N, int64_t K, float *fw, float *fm, hipStream_t st);
hipError_t launch_gemm_q6k_x(const int8_t *lo, const int8_t *hi, const float *dw, const int8_t *q,
                             const float *d, int M, int N, int K, float *out, const Ws &ws, hipStream_t st);
hipError_t launch_gemm_q6k_x_small(const int8_t *lo, const int8_t *hi, const float *dw, const int8_t *q,
                                   const float *d, int M, int N, int K, float *out, const Ws &ws,
                                   hipStream_t st);
hipError_t launch_gemm_q4k_dsc(const uint8_t *W, const float *fw, const float *fm, const int8_t *q,
                               const float *d, const float *s, int M, int N, int K, float *out,
                               const Ws &ws, hipStream_t st);
hipError_t launch_gemm_q4k_dsc_small(const uint8_t *W, const float *fw, const float *fm, const int8_t *q,
                                     const float *d, const float *s, int M, int N, int K, float *out,
                                     const Ws &ws, hipStream_t st);

// Compute units of the current device (cached per device).
int device_cu_count();

// Number of K ranges (1 = no split) for a GEMM of `tiles` output tiles of
// tile_elems outputs each over `pairs` = K/256 super-blocks; slot_ops is the
// int8 rate of one resident workgroup.
int gemm_splits(int tiles, int tile_elems, int pairs, int64_t M, int64_t N, int K, double slot_ops);

// out[i] = sum over s = 0..nsplit-1, in that order, of part[s * n + i].
hipError_t splitk_reduce(const float *part, int nsplit, int64_t n, float *out, hipStream_t st);

// Number of K ranges each GEMM configuration cuts a launch of M x N x K
// into when it is given a workspace (1 = no split); the launchers below use
// the same choice, so a caller can size the workspace before the call.
int splits_gemm_q4k(int M, int N, int K);
int splits_gemm_q4k_small(int M, int N, int K);
int splits_gemm_q5k(int M, int N, int K);
int splits_gemm_q5k_small(int M, int N, int K);
int splits_gemm_q6k(int M, int N, int K);
int splits_gemm_q6k_small(int M, int N, int K);

// Runs launch(dst) once: with dst = out when nsplit == 1, else with dst the
// caller's workspace holding nsplit [M][N] f32 planes (n = M*N elements
// each), followed by the reduction into out. A workspace too small for the
// planes is hipErrorInvalidValue (the C ABI checks the size before it gets
// here).
template <class Launch>
hipError_t run_split_k(int nsplit, int64_t n, float *out, const Ws &ws, hipStream_t st, Launch &&launch)
{
    if (nsplit <= 1)
        return launch(out);
    if (!ws.ptr || ws.bytes < (size_t)nsplit * (size_t)n * sizeof(float))
        return hipErrorInvalidValue;
    float *part = static_cast<float *>(ws.ptr);
    hipError_t e = launch(part);
    if (e == hipSuccess)
        e = splitk_reduce(part, nsplit, n, out, st);
    return e;
}

// Workspace bytes of a split-K GEMM (0 when it does not split).
inline size_t split_bytes(int nsplit, int64_t M, int64_t N)
{
    return nsplit > 1 ? (size_t)nsplit * (size_t)M * (size_t)N * sizeof(float) : 0;
}

} // namespace mq
