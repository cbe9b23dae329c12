// Per-32 int8 activation quantizer (gfx950).
//
// x[M][ldx] f32 -> q[M][K] int8, d[M][K/32] f32, s[M][K/32] f32 with
//   d = amax / 127, q = clamp(roundf(x / d), -127, 127) (0 when d == 0, i.e.
//   amax == 0 or amax so small that amax / 127 underflows),
//   s = d * (float)sum(q).
// The pages call for activations quantized on the fly, once per activation,
// with per-block sums (minfer Support Matrix, "Supported Quantization
// Formats"; minfer Compute Graph Design, §9.3 Execution dispatch); the
// rounding rule is the reading stated in mq.h. Every step is one IEEE f32
// operation (correctly rounded division, no contraction, no denormal flush),
// so the plane is bit-exact against a host evaluation of the same rule.
//
// HBM-bound: 4 B read and 1 + 8/32 B written per element. One lane owns 4
// consecutive values (one 16-byte load, one 4-byte store); 8 lanes own a
// 32-value block and combine amax and sum(q) with cross-lane swizzles.
#include "mq_device.h"
#include "mq_launch.h"

#pragma clang fp contract(off)

namespace mq {
namespace {

__device__ __forceinline__ int quant1(float v, float db, bool zero)
{
    if (zero)
        return 0;
    float r = __builtin_roundf(v / db);
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    return (int)r;
}

// Vector path: x 16-byte aligned and ldx % 4 == 0.
__global__ __launch_bounds__(256) void quantize_act_v4(
    const float *__restrict__ x, int64_t nblk, int64_t nbk, int64_t K,
    int64_t ldx, int8_t *__restrict__ q, float *__restrict__ d,
    float *__restrict__ s)
{
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = g >> 3;            // flat (token, block) index
    if (blk >= nblk)
        return;                            // whole 8-lane groups exit together
    const int li = (int)(g & 7);
    const int64_t t = blk / nbk;
    const int64_t b = blk - t * nbk;
    const float4 v = *reinterpret_cast<const float4 *>(x + t * ldx + 32 * b + 4 * li);

    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 8));

    const float db = amax / 127.0f;
    const bool zero = db == 0.0f;
    const int q0 = quant1(v.x, db, zero), q1 = quant1(v.y, db, zero);
    const int q2 = quant1(v.z, db, zero), q3 = quant1(v.w, db, zero);
    const uint32_t packed = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
                            ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
    *reinterpret_cast<uint32_t *>(q + t * K + 32 * b + 4 * li) = packed;

    int sum = q0 + q1 + q2 + q3;
    sum += __shfl_xor(sum, 1, 8);
    sum += __shfl_xor(sum, 2, 8);
    sum += __shfl_xor(sum, 4, 8);
    if (li == 0) {
        d[blk] = db;
        s[blk] = db * (float)sum;
    }
}

// Scalar path: any 4-byte aligned x and any ldx >= K.
__global__ __launch_bounds__(256) void quantize_act_v1(
    const float *__restrict__ x, int64_t nblk, int64_t nbk, int64_t K,
    int64_t ldx, int8_t *__restrict__ q, float *__restrict__ d,
    float *__restrict__ s)
{
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = g >> 5;
    if (blk >= nblk)
        return;                            // whole 32-lane groups exit together
    const int li = (int)(g & 31);
    const int64_t t = blk / nbk;
    const int64_t b = blk - t * nbk;
    const float v = x[t * ldx + 32 * b + li];

    float amax = fabsf(v);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1)
        amax = fmaxf(amax, __shfl_xor(amax, o, 32));
    const float db = amax / 127.0f;
    const int qi = quant1(v, db, db == 0.0f);
    q[t * K + 32 * b + li] = (int8_t)qi;
    int sum = qi;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1)
        sum += __shfl_xor(sum, o, 32);
    if (li == 0) {
        d[blk] = db;
        s[blk] = db * (float)sum;
    }
}

} // namespace

hipError_t launch_quantize(const float *x, int64_t M, int64_t K, int64_t ldx,
                           int8_t *q, float *d, float *s, hipStream_t st)
{
    const int64_t nbk = K / 32;
    const int64_t nblk = M * nbk;
    const bool vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ldx % 4 == 0);
    const int64_t threads = nblk * (vec ? 8 : 32);
    const int64_t grid = (threads + 255) / 256;
    if (vec)
        quantize_act_v4<<<dim3((unsigned)grid), dim3(256), 0, st>>>(x, nblk, nbk, K, ldx, q, d, s);
    else
        quantize_act_v1<<<dim3((unsigned)grid), dim3(256), 0, st>>>(x, nblk, nbk, K, ldx, q, d, s);
    return hipGetLastError();
}

} // namespace mq
