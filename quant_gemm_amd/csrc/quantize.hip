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

// Contiguous rows (ldx == K, x 16-byte aligned): the plane is one flat
// sequence of nblk = M*K/32 blocks, and so are q (32 bytes per block), d and
// s. A persistent grid walks units of 32*NC blocks (unit u: blocks
// 32*NC*u .. 32*NC*u + 32*NC - 1; 8-lane group g of the workgroup takes
// block 32*NC*u + 32*c + g of its chunk c), with the next unit's loads in
// flight while a unit is quantized and stored. Against one workgroup per
// row chunk (quantize_act_v4), measured by GPU time on MI355X: 3314 x 3584
// 19.6 -> 15.2 us, 512 x 18944 15.6 -> 12.8 us, one token 3.2 -> 2.7 us;
// but 3314 x 18944 (251 MB) 60.9 -> 66.0 us, so planes of more than 128 MB
// of input keep the row-chunk grid (many waves of workgroups already
// overlap there). 1, 2 and 4 blocks per group and unit and 1024, 2048 and
// 4096 workgroups were measured; 2 and 1024 were best up to 128 MB.
#ifndef QA_STREAM_NC
#define QA_STREAM_NC 2
#endif
#ifndef QA_STREAM_WGS
#define QA_STREAM_WGS 1024
#endif
constexpr int64_t QA_STREAM_MAX_BYTES = int64_t(128) << 20;

template <int NC>
__global__ __launch_bounds__(256) void quantize_act_stream(
    const float *__restrict__ x, int64_t nblk, int8_t *__restrict__ q, float *__restrict__ d,
    float *__restrict__ s)
{
    const int g = threadIdx.x >> 3;
    const int li = threadIdx.x & 7;
    const int64_t per = 32 * NC;
    const int64_t nunits = (nblk + per - 1) / per;
    auto load = [&](float4 (&v)[NC], int64_t u) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int64_t B = u * per + 32 * c + g;
            const int64_t Bc = B < nblk ? B : nblk - 1;   // in range; not stored past nblk
            const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(x + 32 * Bc + 4 * li));
            v[c] = make_float4(t[0], t[1], t[2], t[3]);
        }
    };
    float4 cur[NC], nxt[NC];
    int64_t u = blockIdx.x;
    if (u < nunits)
        load(cur, u);
    for (; u < nunits; u += gridDim.x) {
        const int64_t un = u + gridDim.x;
        if (un < nunits)                          // workgroup-uniform
            load(nxt, un);
        uint32_t qp[NC];
        float db[NC], sb[NC];
        quant_chunks<NC>(cur, qp, db, sb);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int64_t B = u * per + 32 * c + g;
            if (B < nblk) {                       // whole 8-lane groups
                *reinterpret_cast<uint32_t *>(q + 32 * B + 4 * li) = qp[c];
                if (li == 0) {
                    d[B] = db[c];
                    s[B] = sb[c];
                }
            }
        }
#pragma unroll
        for (int c = 0; c < NC; ++c)
            cur[c] = nxt[c];
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
    if (vec && ldx == K && M * K * 4 <= QA_STREAM_MAX_BYTES) {
        const int64_t nblk = M * (K / 32);
        const int64_t nunits = (nblk + 32 * QA_STREAM_NC - 1) / (32 * QA_STREAM_NC);
        const int64_t grid = nunits < QA_STREAM_WGS ? nunits : QA_STREAM_WGS;
        quantize_act_stream<QA_STREAM_NC><<<dim3((unsigned)grid), dim3(256), 0, st>>>(x, nblk, q, d, s);
    } else if (vec) {
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
