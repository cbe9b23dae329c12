// Per-32 int8 activation quantizer (gfx950).
//
// x[M][ldx] f32 -> q[M][K] int8, d[M][K/32] f32, s[M][K/32] f32 with
//   d = amax / 127, q = clamp(roundf(x / d), -127, 127) (0 when d == 0, i.e.
//   amax == 0 or amax so small that amax / 127 underflows),
//   s = d * (float)sum(q).
// The pages call for activations quantized on the fly, once per activation,
// with per-block sums (minfer Support Matrix, "Supported Quantization
// Formats"; minfer Compute Graph Design, §9.3 Execution dispatch); the
// rounding rule is the reading stated in mq.h. The plane equals, bit for
// bit, a host evaluation of the rule in IEEE f32 (correctly rounded
// division, no contraction, no denormal flush); quant_core.h gives the
// argument for the cheaper forms the kernels evaluate.
//
// HBM-bound: 4 B read and 1 + 8/32 B written per element. A lane owns 4
// consecutive values of each of a few blocks (16-byte loads, 4-byte stores);
// 8 lanes own a 32-value block and combine amax and sum(q) with DPP moves
// (quant_core.h).
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
    return (int)q_clamp_round(db < 0x1p-100f || q_near_half(t, __builtin_rintf(t)) ? v / db : t);
}

// Strided rows (x 16-byte aligned, ldx % 4 == 0, ldx > K): a workgroup
// covers QA_ITEMS * 1024 consecutive values of one token row: QA_ITEMS
// float4 per thread, 8 threads per 32-value block, all loads issued first.
constexpr int QA_ITEMS = 2;

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
        v[i] = ld_stream_f4(xr + (k < K ? k : K - 4));   // in range; not stored past K
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
// s. Workgroup b takes blocks 32*QA_FLAT_NC*b .. + 32*QA_FLAT_NC - 1
// (8-lane group g of it block 32*QA_FLAT_NC*b + 32*c + g of its chunk c), so
// no workgroup idles on a row's tail. Measured on MI355X, kernel time with
// the input cold in HBM: 3314 x 3584 12.5 us, 512 x 18944 10.6 us,
// 3314 x 18944 69 us; a kernel that moves the same bytes in the same pattern
// with no arithmetic takes 12.2, 10.1 and 72 us. Persistent grids (1024 to
// 4096 workgroups, the next unit's loads in flight), 1, 2 and 4 blocks per
// group and 2 or 4 units per workgroup were measured too and were no
// faster.
constexpr int QA_FLAT_NC = 2;

__global__ __launch_bounds__(256) void quantize_act_flat(
    const float *__restrict__ x, int64_t nblk, int8_t *__restrict__ q, float *__restrict__ d,
    float *__restrict__ s)
{
    const int g = threadIdx.x >> 3;
    const int li = threadIdx.x & 7;
    const int64_t base = (int64_t)blockIdx.x * (32 * QA_FLAT_NC) + g;
    float4 v[QA_FLAT_NC];
#pragma unroll
    for (int c = 0; c < QA_FLAT_NC; ++c) {
        const int64_t B = base + 32 * c;
        const int64_t Bc = B < nblk ? B : nblk - 1;   // in range; not stored past nblk
        v[c] = ld_stream_f4(x + 32 * Bc + 4 * li);
    }
    uint32_t qp[QA_FLAT_NC];
    float db[QA_FLAT_NC], sb[QA_FLAT_NC];
    quant_chunks<QA_FLAT_NC>(v, qp, db, sb);
#pragma unroll
    for (int c = 0; c < QA_FLAT_NC; ++c) {
        const int64_t B = base + 32 * c;
        if (B < nblk) {                           // whole 8-lane groups
            *reinterpret_cast<uint32_t *>(q + 32 * B + 4 * li) = qp[c];
            if (li == 0) {
                d[B] = db[c];
                s[B] = sb[c];
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
    if (vec && ldx == K) {
        const int64_t nblk = M * (K / 32);
        const int64_t grid = (nblk + 32 * QA_FLAT_NC - 1) / (32 * QA_FLAT_NC);
        launch(quantize_act_flat, dim3((unsigned)grid), dim3(256), 0, st, x, nblk, q, d, s);
    } else if (vec) {
        const int chunks = (int)((K + QA_ITEMS * 1024 - 1) / (QA_ITEMS * 1024));
        launch(quantize_act_v4, dim3((unsigned)(M * chunks)), dim3(256), 0, st, x, (int)K, chunks, ldx, q, d, s);
    } else {
        const int64_t nbk = K / 32;
        const int64_t nblk = M * nbk;
        const int64_t grid = (nblk * 32 + 255) / 256;
        launch(quantize_act_v1, dim3((unsigned)grid), dim3(256), 0, st, x, nblk, nbk, K, ldx, q, d, s);
    }
    return hipGetLastError();
}

} // namespace mq
