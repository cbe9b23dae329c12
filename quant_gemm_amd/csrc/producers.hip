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
// a plain f64 sum whose effect on r is certified, with an exact
// (double-double) sum for the rare rows where the certificate fails (see
// the RMSNorm section). Optionally y itself is written too.
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


// ---------------------------------------------------------------- RMSNorm
// The sum of squares. Each square x^2 is exact in f64 and none is negative,
// so a plain f64 sum whose every term passes through at most h roundings is
// within h 2^-53 (1 + 2^-40) relative of the exact sum, and so within
// (h + 1) 2^-53 of the exact sum rounded to f64. r is computed once from
// that sum; the rule's r (from the exact sum rounded to f64) differs from
// it, before the final rounding to f32, by at most (h / 2 + 9) 2^-53
// relative (half the input error through the square root, plus four
// roundings on each side). Where the f64 r is farther than
// rel = (h + 20) 2^-53 from every f32 rounding boundary, both round to the
// same f32 (an all-zero row gives an exact sum of 0). Otherwise, about one
// row in 10^5, the row is summed again as an unevaluated pair of doubles
// with error-free additions (error about 2^-100 of the sum), whose rounding
// to f64 is the exactly rounded sum whatever the order of the terms.

// A double moved between lanes by a DPP pattern (both halves; lanes the
// pattern leaves without a source, or in masked rows, receive 0).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double x)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xf, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xf, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane63_f64(double x)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sums over the 64 lanes of a wavefront, every lane receiving the total:
// pairs, quads, half-rows and rows of 16 with DPP, then rows 0+1 and 2+3 and
// all four through the row broadcasts into lane 63 (lanes a broadcast leaves
// out combine with zero, which changes nothing), read back from lane 63.
// Six levels of additions.
__device__ __forceinline__ double wave_sum_f64(double a)
{
    a += dpp_f64<0xb1>(a);                 // quad_perm [1,0,3,2]
    a += dpp_f64<0x4e>(a);                 // quad_perm [2,3,0,1]
    a += dpp_f64<0x141>(a);                // row_half_mirror
    a += dpp_f64<0x140>(a);                // row_mirror
    a += dpp_f64<0x142, 0xa>(a);           // row_bcast:15 into rows 1 and 3
    a += dpp_f64<0x143, 0xc>(a);           // row_bcast:31 into rows 2 and 3
    return readlane63_f64(a);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ DD dd_dpp(DD a)
{
    return DD{dpp_f64<CTRL, ROW_MASK>(a.hi), dpp_f64<CTRL, ROW_MASK>(a.lo)};
}

__device__ __forceinline__ DD dd_wave_sum(DD a)
{
    a = dd_merge(a, dd_dpp<0xb1>(a));
    a = dd_merge(a, dd_dpp<0x4e>(a));
    a = dd_merge(a, dd_dpp<0x141>(a));
    a = dd_merge(a, dd_dpp<0x140>(a));
    a = dd_merge(a, dd_dpp<0x142, 0xa>(a));
    a = dd_merge(a, dd_dpp<0x143, 0xc>(a));
    return DD{readlane63_f64(a.hi), readlane63_f64(a.lo)};
}

// 1 / sqrt(ss / K + eps), every step a correctly rounded f64 operation.
__device__ __forceinline__ double rms_r64(double ss, int K, float eps)
{
    return 1.0 / sqrt(ss / (double)K + (double)eps);
}

// True when every value within rel (relative) of r64 rounds to f32(r64).
__device__ __forceinline__ bool f32_rounding_certain(double r64, double rel)
{
    const float r32 = (float)r64;
    const uint32_t b = __builtin_bit_cast(uint32_t, r32);
    if (b == 0u || b >= 0x7f800000u)
        return false;                          // not a positive finite f32: take the exact sum
    const double lo = 0.5 * ((double)r32 + (double)__builtin_bit_cast(float, b - 1u));
    const double hi = 0.5 * ((double)r32 + (double)__builtin_bit_cast(float, b + 1u));
    return r64 - r64 * rel > lo && r64 + r64 * rel < hi;
}

// Row per workgroup of 256 threads: thread i owns the float4 at
// 1024 j + 4 i of each 1024-value chunk j, so 8 consecutive threads own one
// 32-value block. The first NC chunks stay in registers between the two
// passes; any further ones are read again (an L2 hit). The row is read with
// streaming loads (a cold sweep with plain loads took twice as long).
// Measured on MI355X at 3314 x 3584 against one wavefront per row (the row
// in registers, the next row prefetched): 17.1 against 19.5 us per call; a
// kernel of this shape with f32 arithmetic and no weight takes 13.4 us.
constexpr int RMS_THREADS = 256;

template <int NC, bool Y>
__global__ __launch_bounds__(RMS_THREADS) void rmsnorm_quantize_kernel(
    const float *__restrict__ x, const float *__restrict__ w, int K, int64_t ldx, float eps,
    int8_t *__restrict__ q, float *__restrict__ d, float *__restrict__ s, float *__restrict__ y)
{
    __shared__ double red[RMS_THREADS / 64];
    __shared__ DD dred[RMS_THREADS / 64];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const float *xr = x + t * ldx;
    const int nch = (K + 1023) >> 10;
    float4 v[NC], wv[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int k = 1024 * j + 4 * tid;
        v[j] = k < K ? ld_stream_f4(xr + k) : float4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {           // w is read by every row: cached loads, issued early
        const int k = 1024 * j + 4 * tid;
        wv[j] = *reinterpret_cast<const float4 *>(w + (k < K ? k : 0));
    }
    double c0 = 0.0, c1 = 0.0, c2 = 0.0, c3 = 0.0;   // four chains of nch terms
    auto fma4 = [&](const float4 e) {
        c0 = __builtin_fma((double)e.x, (double)e.x, c0);
        c1 = __builtin_fma((double)e.y, (double)e.y, c1);
        c2 = __builtin_fma((double)e.z, (double)e.z, c2);
        c3 = __builtin_fma((double)e.w, (double)e.w, c3);
    };
#pragma unroll
    for (int j = 0; j < NC; ++j)
        fma4(v[j]);                          // zeros past the row add nothing
    for (int j = NC; j < nch; ++j) {
        const int k = 1024 * j + 4 * tid;
        if (k < K)
            fma4(*reinterpret_cast<const float4 *>(xr + k));
    }
    const double wsum = wave_sum_f64((c0 + c1) + (c2 + c3));
    if ((tid & 63) == 0)
        red[tid >> 6] = wsum;
    __syncthreads();
    const double ssa = ((red[0] + red[1]) + red[2]) + red[3];
    const int h = nch + 2 + 6 + 3;           // roundings on any term's way to ssa
    double r64 = rms_r64(ssa, K, eps);
    if (ssa != 0.0 && !f32_rounding_certain(r64, (double)(h + 20) * 0x1p-53)) {   // workgroup-uniform
        DD a0{0.0, 0.0}, a1{0.0, 0.0}, a2{0.0, 0.0}, a3{0.0, 0.0};
#pragma unroll 1
        for (int k = 4 * tid; k < K; k += 1024) {
            const float4 e = *reinterpret_cast<const float4 *>(xr + k);
            dd_add(a0, (double)e.x * (double)e.x);
            dd_add(a1, (double)e.y * (double)e.y);
            dd_add(a2, (double)e.z * (double)e.z);
            dd_add(a3, (double)e.w * (double)e.w);
        }
        const DD acc = dd_wave_sum(dd_merge(dd_merge(a0, a1), dd_merge(a2, a3)));
        if ((tid & 63) == 0)
            dred[tid >> 6] = acc;
        __syncthreads();
        const DD tot = dd_merge(dd_merge(dred[0], dred[1]), dd_merge(dred[2], dred[3]));
        r64 = rms_r64(tot.hi + tot.lo, K, eps);
    }
    const float r = (float)r64;

    const int li = tid & 7;
    const int nbk = K >> 5;
    auto scale = [&](float4 e, const float4 wk) {
        e.x = (e.x * r) * wk.x;
        e.y = (e.y * r) * wk.y;
        e.z = (e.z * r) * wk.z;
        e.w = (e.w * r) * wk.w;
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
            v[j] = scale(v[j], wv[j]);
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
            float4 e[1] = {scale(*reinterpret_cast<const float4 *>(xr + k), *reinterpret_cast<const float4 *>(w + k))};
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
        gv[i] = ld_stream_f4(gr + kk);
        uv[i] = ld_stream_f4(ur + kk);
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
