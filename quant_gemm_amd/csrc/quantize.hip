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
// HBM-bound: 4 B read and 1 + 8/32 B written per element. A lane owns 4
// consecutive values of each of QA_ITEMS blocks (16-byte loads, 4-byte
// stores); 8 lanes own a 32-value block and combine amax and sum(q) with
// cross-lane swizzles (quant_core.h).
#include "mq_device.h"
#include "mq_launch.h"
#include "quant_core.h"

#pragma clang fp contract(off)

namespace mq {
namespace {

// Scalar form of the rule for the unaligned path (the quotient as in
// quant_chunks).
__device__ __forceinline__ int quant1(float v, float db, float rdb, bool zero)
{
    if (zero)
        return 0;
    const float t = v * rdb;
    return (int)q_clamp_round(db < 0x1p-100f || q_near_half(t) ? v / db : t);
}

// Vector path: x 16-byte aligned and ldx % 4 == 0. A workgroup covers
// QA_ITEMS * 1024 consecutive values of one token row: QA_ITEMS float4 per
// thread, 8 threads per 32-value block, all loads issued first.
constexpr int QA_ITEMS = 4;

__global__ __launch_bounds__(256) void quantize_act_v4(
    const float *__restrict__ x, int K, int chunks, int64_t ldx, int8_t *__restrict__ q,
    float *__restrict__ d, float *__restrict__ s)
{
    const int t = blockIdx.x / chunks;
    const int c = blockIdx.x - t * chunks;
    const int li = threadIdx.x & 7;
    const float *xr = x + (int64_t)t * ldx;
    const int nbk = K >> 5;
    float4 v[QA_ITEMS];
#pragma unroll
    for (int i = 0; i < QA_ITEMS; ++i) {
        const int k = (c * QA_ITEMS + i) * 1024 + 4 * threadIdx.x;
        v[i] = *reinterpret_cast<const float4 *>(xr + (k < K ? k : K - 4));   // in range; not stored past K
    }
    uint32_t qp[QA_ITEMS];
    float db[QA_ITEMS], sb[QA_ITEMS];
    quant_chunks<QA_ITEMS>(v, qp, db, sb);
#pragma unroll
    for (int i = 0; i < QA_ITEMS; ++i) {
        const int k = (c * QA_ITEMS + i) * 1024 + 4 * threadIdx.x;
        if (k < K) {                          // whole 8-lane groups (K is a multiple of 32)
            *reinterpret_cast<uint32_t *>(q + (int64_t)t * K + k) = qp[i];
            if (li == 0) {
                const int64_t b = (int64_t)t * nbk + (k >> 5);
                d[b] = db[i];
                s[b] = sb[i];
            }
        }
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
    const int qi = quant1(v, db, db == 0.0f ? 0.0f : 1.0f / db, db == 0.0f);
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
    const bool vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (ldx % 4 == 0);
    if (vec) {
        const int chunks = (int)((K + QA_ITEMS * 1024 - 1) / (QA_ITEMS * 1024));
        quantize_act_v4<<<dim3((unsigned)(M * chunks)), dim3(256), 0, st>>>(x, (int)K, chunks, ldx, q, d, s);
    } else {
        const int64_t nbk = K / 32;
        const int64_t nblk = M * nbk;
        const int64_t grid = (nblk * 32 + 255) / 256;
        quantize_act_v1<<<dim3((unsigned)grid), dim3(256), 0, st>>>(x, nblk, nbk, K, ldx, q, d, s);
    }
    return hipGetLastError();
}

} // namespace mq
