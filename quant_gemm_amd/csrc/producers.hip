// Producer-fused activation quantizers (gfx950): RMSNorm -> int8 plane and
// SwiGLU -> int8 plane, without an f32 activation tensor in between.
//
// The pages' GPU path has the RMS normalisation and the SwiGLU epilogue emit
// the int8 activation plane directly (minfer Features, "GPU — CUDA"); the
// ops are RmsNorm{eps} and SwiGLU = Silu(gate) * up (minfer Compute Graph
// Design, "The Op vocabulary"). Arithmetic, as declared in mq.h:
//   RMSNorm: ss = sum_k x_k^2 rounded once to f64 from the exact sum,
//            r = f32(1 / sqrt(ss / K + eps)) in f64, y_k = (x_k * r) * w_k (f32);
//   SwiGLU:  y_k = f32(g_k / (1 + exp(-g_k)) in f64) * u_k (f32);
// then the per-32 quantizer of mq_quantize_act on y. The sum of squares is
// accumulated as an unevaluated pair of doubles (error-free additions): its
// error is about 2^-100 of the sum, so rounding it to f64 gives the exactly
// rounded sum whatever the order of the terms. Optionally y itself is
// written too.
//
// HBM-bound: RMSNorm reads x once (kept in registers between the two passes
// over a row for K <= 8192) and writes 1 + 8/32 bytes per element; SwiGLU
// reads 8 bytes and writes the same, with about 20 f64 operations per value
// for the SiLU.
#include "mq_device.h"
#include "mq_launch.h"
#include "quant_core.h"

#include <type_traits>

#pragma clang fp contract(off)

namespace mq {
namespace {

// ---------------------------------------------------------------- double-double sums
struct DD {
    double hi, lo;
};

// hi + lo += v, error-free (Knuth's two-sum on hi, the error kept in lo)
__device__ __forceinline__ void dd_add(DD &a, double v)
{
    const double s = a.hi + v;
    const double bb = s - a.hi;
    const double err = (a.hi - (s - bb)) + (v - bb);
    a.hi = s;
    a.lo += err;
}

__device__ __forceinline__ DD dd_merge(DD a, DD b)
{
    const double s = a.hi + b.hi;
    const double bb = s - a.hi;
    const double err = (a.hi - (s - bb)) + (b.hi - bb) + a.lo + b.lo;
    const double hi = s + err;                 // renormalise (fast two-sum: |s| >= |err|)
    return DD{hi, err - (hi - s)};
}

__device__ __forceinline__ DD dd_shfl_xor(DD a, int m)
{
    return DD{__shfl_xor(a.hi, m), __shfl_xor(a.lo, m)};
}

// ---------------------------------------------------------------- RMSNorm
// One workgroup of 256 threads per row: thread i owns the float4 at
// 1024 j + 4 i of each 1024-value chunk j, so 8 consecutive threads own one
// 32-value block. The first NC chunks stay in registers between the two
// passes; any further ones are read again (an L2 hit).
constexpr int RMS_THREADS = 256;

template <int NC, bool Y>
__global__ __launch_bounds__(RMS_THREADS) void rmsnorm_quantize_kernel(
    const float *__restrict__ x, const float *__restrict__ w, int K, int64_t ldx, float eps,
    int8_t *__restrict__ q, float *__restrict__ d, float *__restrict__ s, float *__restrict__ y)
{
    __shared__ DD red[RMS_THREADS / 64];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const float *xr = x + t * ldx;
    const int nch = (K + 1023) >> 10;
    float4 v[NC];
    DD a0{0.0, 0.0}, a1{0.0, 0.0}, a2{0.0, 0.0}, a3{0.0, 0.0};   // four independent chains
    auto add4 = [&](const float4 e) {
        dd_add(a0, (double)e.x * (double)e.x);
        dd_add(a1, (double)e.y * (double)e.y);
        dd_add(a2, (double)e.z * (double)e.z);
        dd_add(a3, (double)e.w * (double)e.w);
    };
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int k = 1024 * j + 4 * tid;
        v[j] = k < K ? *reinterpret_cast<const float4 *>(xr + k) : float4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < NC; ++j)
        add4(v[j]);                          // zeros past the row add nothing
    for (int j = NC; j < nch; ++j) {
        const int k = 1024 * j + 4 * tid;
        if (k < K)
            add4(*reinterpret_cast<const float4 *>(xr + k));
    }
    DD acc = dd_merge(dd_merge(a0, a1), dd_merge(a2, a3));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        acc = dd_merge(acc, dd_shfl_xor(acc, m));
    if ((tid & 63) == 0)
        red[tid >> 6] = acc;
    __syncthreads();
    DD tot = red[0];
#pragma unroll
    for (int i = 1; i < RMS_THREADS / 64; ++i)
        tot = dd_merge(tot, red[i]);
    const double ss = tot.hi + tot.lo;
    const float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));

    const int li = tid & 7;
    const int nbk = K >> 5;
    auto scale = [&](float4 e, int k) {
        const float4 wv = *reinterpret_cast<const float4 *>(w + (k < K ? k : 0));
        e.x = (e.x * r) * wv.x;
        e.y = (e.y * r) * wv.y;
        e.z = (e.z * r) * wv.z;
        e.w = (e.w * r) * wv.w;
        return e;
    };
    auto store = [&](const float4 e, uint32_t qp, float db, float sb, int k) {
        if (Y)
            *reinterpret_cast<float4 *>(y + t * K + k) = e;
        *reinterpret_cast<uint32_t *>(q + t * K + k) = qp;
        if (li == 0) {
            d[t * nbk + (k >> 5)] = db;
            s[t * nbk + (k >> 5)] = sb;
        }
    };
    {
        uint32_t qp[NC];
        float db[NC], sb[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j)
            v[j] = scale(v[j], 1024 * j + 4 * tid);
        quant_chunks<NC>(v, qp, db, sb);     // blocks past the row are all zero and not stored
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int k = 1024 * j + 4 * tid;
            if (k < K)
                store(v[j], qp[j], db[j], sb[j], k);
        }
    }
    for (int j = NC; j < nch; ++j) {
        const int k = 1024 * j + 4 * tid;
        if (k < K) {                          // whole 8-lane groups (K is a multiple of 32)
            float4 e[1] = {scale(*reinterpret_cast<const float4 *>(xr + k), k)};
            uint32_t qp[1];
            float db[1], sb[1];
            quant_chunks<1>(e, qp, db, sb);
            store(e[0], qp[0], db[0], sb[0], k);
        }
    }
}

// ---------------------------------------------------------------- SwiGLU
// A workgroup covers SW_ITEMS * 1024 consecutive values of one token row
// (SW_ITEMS float4 per thread, 8 threads per 32-value block), all loads
// issued first. A few tokens take one float4 per thread, which spreads a
// decode row over 4x the workgroups (the f64 SiLU is the long pole there).
template <int SW_ITEMS, bool Y>
__global__ __launch_bounds__(256) void swiglu_quantize_kernel(
    const float *__restrict__ g, const float *__restrict__ u, int K, int chunks, int64_t ldg,
    int64_t ldu, int8_t *__restrict__ q, float *__restrict__ d, float *__restrict__ s,
    float *__restrict__ y)
{
    const int t = blockIdx.x / chunks;
    const int c = blockIdx.x - t * chunks;
    const int li = threadIdx.x & 7;
    const float *gr = g + (int64_t)t * ldg;
    const float *ur = u + (int64_t)t * ldu;
    const int nbk = K >> 5;
    float4 gv[SW_ITEMS], uv[SW_ITEMS];
#pragma unroll
    for (int i = 0; i < SW_ITEMS; ++i) {
        const int k = (c * SW_ITEMS + i) * 1024 + 4 * threadIdx.x;
        const int kk = k < K ? k : K - 4;    // in range; the result is not stored
        gv[i] = *reinterpret_cast<const float4 *>(gr + kk);
        uv[i] = *reinterpret_cast<const float4 *>(ur + kk);
    }
    auto silu = [](float a) {
        const double a64 = (double)a;
        return (float)(a64 / (1.0 + exp(-a64)));
    };
    float4 yv[SW_ITEMS];
#pragma unroll
    for (int i = 0; i < SW_ITEMS; ++i) {
        yv[i].x = silu(gv[i].x) * uv[i].x;
        yv[i].y = silu(gv[i].y) * uv[i].y;
        yv[i].z = silu(gv[i].z) * uv[i].z;
        yv[i].w = silu(gv[i].w) * uv[i].w;
    }
    uint32_t qp[SW_ITEMS];
    float db[SW_ITEMS], sb[SW_ITEMS];
    quant_chunks<SW_ITEMS>(yv, qp, db, sb);
#pragma unroll
    for (int i = 0; i < SW_ITEMS; ++i) {
        const int k = (c * SW_ITEMS + i) * 1024 + 4 * threadIdx.x;
        if (k < K) {
            if (Y)
                *reinterpret_cast<float4 *>(y + (int64_t)t * K + k) = yv[i];
            *reinterpret_cast<uint32_t *>(q + (int64_t)t * K + k) = qp[i];
            if (li == 0) {
                const int64_t b = (int64_t)t * nbk + (k >> 5);
                d[b] = db[i];
                s[b] = sb[i];
            }
        }
    }
}

} // namespace

hipError_t launch_rmsnorm_quantize(const float *x, const float *w, int64_t M, int64_t K, int64_t ldx,
                                   float eps, int8_t *q, float *d, float *s, float *y, hipStream_t st)
{
    const dim3 grid((unsigned)M), block(RMS_THREADS);
    const int k = (int)K;
    auto go = [&](auto nc) {
        constexpr int N = decltype(nc)::value;
        if (y)
            rmsnorm_quantize_kernel<N, true><<<grid, block, 0, st>>>(x, w, k, ldx, eps, q, d, s, y);
        else
            rmsnorm_quantize_kernel<N, false><<<grid, block, 0, st>>>(x, w, k, ldx, eps, q, d, s, y);
    };
    if (K <= 1024)
        go(std::integral_constant<int, 1>{});
    else if (K <= 2048)
        go(std::integral_constant<int, 2>{});
    else if (K <= 4096)
        go(std::integral_constant<int, 4>{});
    else
        go(std::integral_constant<int, 8>{});
    return hipGetLastError();
}

hipError_t launch_swiglu_quantize(const float *g, const float *u, int64_t M, int64_t K, int64_t ldg,
                                  int64_t ldu, int8_t *q, float *d, float *s, float *y, hipStream_t st)
{
    auto go = [&](auto it) {
        constexpr int IT = decltype(it)::value;
        const int chunks = (int)((K + IT * 1024 - 1) / (IT * 1024));
        const dim3 grid((unsigned)(M * chunks)), block(256);
        if (y)
            swiglu_quantize_kernel<IT, true><<<grid, block, 0, st>>>(g, u, (int)K, chunks, ldg, ldu, q, d, s, y);
        else
            swiglu_quantize_kernel<IT, false><<<grid, block, 0, st>>>(g, u, (int)K, chunks, ldg, ldu, q, d, s, y);
    };
    if (M * ((K + 4095) / 4096) < 256)
        go(std::integral_constant<int, 1>{});
    else
        go(std::integral_constant<int, 4>{});
    return hipGetLastError();
}

} // namespace mq
