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

hipError_t launch_gemm_q4k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           hipStream_t st);
hipError_t launch_gemm_q6k(const uint8_t *W, const int8_t *q, const float *d,
                           int M, int N, int K, float *out, hipStream_t st);

} // namespace mq
