// Kernel launchers of libmq (internal). Arguments are validated by the C-ABI
// layer before these are called; each launcher only enqueues work on `st`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

// Largest token count the GEMV kernels serve.
constexpr int GEMV_MAX_M = 8;

hipError_t launch_quantize(const float *x, int64_t M, int64_t K, int64_t ldx,
                           int8_t *q, float *d, float *s, hipStream_t st);

hipError_t launch_gemv_q4k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           hipStream_t st);
hipError_t launch_gemv_q6k(const uint8_t *W, const int8_t *q, const float *d,
                           int M, int N, int K, float *out, hipStream_t st);

hipError_t launch_rmsnorm_quantize(const float *x, const float *w, int64_t M, int64_t K, int64_t ldx,
                                   float eps, int8_t *q, float *d, float *s, float *y, hipStream_t st);
hipError_t launch_swiglu_quantize(const float *g, const float *u, int64_t M, int64_t K, int64_t ldg,
                                  int64_t ldu, int8_t *q, float *d, float *s, float *y, hipStream_t st);

hipError_t launch_gemm_q4k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           hipStream_t st);
hipError_t launch_gemm_q4k_ffn(const uint8_t *Wg, const uint8_t *Wu, const int8_t *q, const float *d,
                               const float *s, int M, int N, int K, int8_t *qo, float *do_, float *so,
                               float *y, hipStream_t st);
hipError_t launch_gemv_q4k_ffn(const uint8_t *Wg, const uint8_t *Wu, const int8_t *q, const float *d,
                               const float *s, int M, int N, int K, int8_t *qo, float *do_, float *so,
                               float *y, hipStream_t st);
hipError_t launch_gemm_q6k(const uint8_t *W, const int8_t *q, const float *d,
                           int M, int N, int K, float *out, hipStream_t st);

// Compute units of the current device (cached per device).
int device_cu_count();

// Number of K ranges (1 = no split) for a GEMM of `tiles` 128x128 output
// tiles over `pairs` = K/256 super-blocks; slot_ops is the int8 rate of one
// resident workgroup.
int gemm_splits(int tiles, int pairs, int64_t M, int64_t N, int K, double slot_ops);

// out[i] = sum over s = 0..nsplit-1, in that order, of part[s * n + i].
hipError_t splitk_reduce(const float *part, int nsplit, int64_t n, float *out, hipStream_t st);

// Runs launch(dst) once: with dst = out when nsplit == 1, else with dst a
// workspace of nsplit [M][N] f32 planes (n = M*N elements each), allocated and
// freed in stream order on st, followed by the reduction into out.
template <class Launch>
hipError_t run_split_k(int nsplit, int64_t n, float *out, hipStream_t st, Launch &&launch)
{
    if (nsplit <= 1)
        return launch(out);
    float *part = nullptr;
    hipError_t e = hipMallocAsync(reinterpret_cast<void **>(&part), (size_t)nsplit * (size_t)n * sizeof(float), st);
    if (e != hipSuccess)
        return e;
    e = launch(part);
    if (e == hipSuccess)
        e = splitk_reduce(part, nsplit, n, out, st);
    const hipError_t f = hipFreeAsync(part, st);
    return e != hipSuccess ? e : f;
}

} // namespace mq
