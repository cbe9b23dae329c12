// Ceiling probes for gfx950 (libmq_probes.so): not part of the matmul
// library, only measured by `bench.py --ceilings`, so that the hardware
// ceilings the kernels are judged against can be reproduced.
//
//   mqp_read(kind, depth, src, bytes, grid, sink, stream)
//       reads `bytes` (a multiple of 1024) from src once:
//       kind 0: grid-stride 16-byte register loads, `depth` (4, 8, 16) in
//               flight per lane;
//       kind 1: global->LDS DMA through a ring of `depth` (2, 4, 8) 1 KB
//               slots per wavefront.
//       The data are folded into a value that is stored to sink[0] only if
//       it equals a constant no input produces, so the loads are kept and
//       nothing is written.
//   mqp_mix(k, iters, grid, sink, stream)
//       a stream of v_mfma_i32_32x32x32_i8 (4 independent tiles per
//       iteration per wavefront) with k f32 VALU operations per int32
//       result: k = 0 chains the MFMAs only; k = 2 converts and adds
//       (cvt, fma); k = 3 also forms a scale product (cvt, mul, fma), as
//       the GEMM epilogue does; k = 4 one more multiply. k = 10, 11, 12:
//       the scaled fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, one
//       32-value sub-block's exact dot as an f32 from two base-16 digits
//       of the activation) chained, or followed by fma, or by scale
//       product and fma. sink holds grid * 256 floats.
// Both return the hipError_t of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int MAGIC = 0x5a5a1234;

template <int D>
__global__ __launch_bounds__(256) void read_regs(const v4i *__restrict__ src, int64_t n16, int *sink)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    int fold = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride * D) {
        v4i v[D];
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int64_t j = i + u * stride;
            v[u] = j < n16 ? __builtin_nontemporal_load(src + j) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < D; ++u)
            fold += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (fold == MAGIC)
        sink[0] = fold;
}

__device__ __forceinline__ void dma16(const void *src, const void *lds_dst)
{
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds_dst);
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %2\n\t"
                 "global_load_lds_dwordx4 %1, off\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(src), "s"(base)
                 : "memory");
}

// Wavefront w of NW streams 1 KB chunks w, w + NW, ... through a ring of D
// LDS slots, D - 1 chunks in flight beyond the one it reads.
template <int D>
__global__ __launch_bounds__(256) void read_lds(const v4i *__restrict__ src, int64_t n1k, int *sink)
{
    __shared__ v4i ring[4][D][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nw = (int64_t)gridDim.x * 4, w = (int64_t)blockIdx.x * 4 + wave;
    const int64_t cnt = w < n1k ? (n1k - 1 - w) / nw + 1 : 0;
    if (cnt == 0)
        return;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const int64_t c = w + (d < cnt ? d : cnt - 1) * nw;
        dma16(src + c * 64 + lane, &ring[wave][d][0]);
    }
    int fold = 0;
    for (int64_t i = 0; i < cnt; ++i) {
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(D - 1) : "memory");
        const v4i v = ring[wave][i % D][lane];
        fold += v.x ^ v.w;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int64_t nx = i + D < cnt ? i + D : cnt - 1;     // past the end: reload the last chunk
        dma16(src + (w + nx * nw) * 64 + lane, &ring[wave][i % D][0]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (fold == MAGIC)
        sink[0] = fold;
}

// K = 0, 2, 3, 4: int8 32x32x32 MFMAs, each int32 result followed by K f32
// VALU operations (0: the MFMAs alone, chained). K = 10, 11, 12: the scaled
// fp8 32x32x64 MFMA that gives one 32-value sub-block's dot as an f32 (two
// base-16 digits of the activation against the same quants), followed by 0
// (chained), 1 (fma) or 2 (scale product, fma) VALU operations per result.
template <int K>
__global__ __launch_bounds__(256) void mix(int iters, float *sink)
{
    if constexpr (K >= 10) {
        v8i a8 = {(int)threadIdx.x & 0x07070707, 1, 2, 3, 4, 5, 6, 7};
        v8i b8 = {3, 2, 1, (int)threadIdx.x & 0x07070707, 4, 5, 6, 7};
        float scale[16];
#pragma unroll
        for (int v = 0; v < 16; ++v)
            scale[v] = 1.0f + v * 1e-3f;
        float f = 1e-3f * threadIdx.x;
        v16f acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            acc[t] = v16f{};
        for (int i = 0; i < iters; ++i) {
            b8.x += i & 0x0101;
            if constexpr (K == 10) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    v8i bt = b8;
                    bt.y += t;
                    acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, bt, acc[t], 0, 0, 0, 140, 0, 136);
                }
            } else {
                v16f I[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    v8i bt = b8;
                    bt.y += t;
                    I[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, bt, v16f{}, 0, 0, 0, 140, 0, 136);
                }
                float rowf[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    rowf[t] = f * (1.0f + 1e-3f * t);
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        if constexpr (K == 11)
                            acc[t][v] = __builtin_fmaf(I[t][v], rowf[t], acc[t][v]);
                        else
                            acc[t][v] = __builtin_fmaf(I[t][v], rowf[t] * scale[v], acc[t][v]);
                    }
                f += 1e-7f;
            }
        }
        float s = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                s += acc[t][v];
        sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
        return;
    } else {
    v4i a = {(int)threadIdx.x, 1, 2, 3}, b = {3, 2, 1, (int)threadIdx.x};
    float scale[16];
#pragma unroll
    for (int v = 0; v < 16; ++v)
        scale[v] = 1.0f + v * 1e-3f;
    float f = 1e-3f * threadIdx.x;
    v16f acc[4];
    v16i chain[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        acc[t] = v16f{};
        chain[t] = v16i{};
    }
    for (int i = 0; i < iters; ++i) {
        b.x += i;
        if constexpr (K == 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                v4i bt = b;
                bt.y += t;
                chain[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bt, chain[t], 0, 0, 0);
            }
        } else {
            // distinct operands per tile, so that the four MFMAs stay four
            v16i I[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                v4i bt = b;
                bt.y += t;
                I[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bt, v16i{}, 0, 0, 0);
            }
            // a per-tile factor that changes every iteration times a
            // per-element one: one distinct scale product per result, as
            // d_x[token] * (d*sc)[row] in the GEMM epilogue
            float rowf[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                rowf[t] = f * (1.0f + 1e-3f * t);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const float y = (float)I[t][v];
                    if constexpr (K == 2)
                        acc[t][v] = __builtin_fmaf(y, rowf[t], acc[t][v]);
                    else if constexpr (K == 3)
                        acc[t][v] = __builtin_fmaf(y, rowf[t] * scale[v], acc[t][v]);
                    else
                        acc[t][v] = __builtin_fmaf(y * scale[v], rowf[t] * scale[15 - v], acc[t][v]);
                }
            f += 1e-7f;
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            s += acc[t][v] + (float)chain[t][v];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
    }
}

} // namespace

extern "C" int mqp_read(int kind, int depth, const void *src, int64_t bytes, int grid, int *sink,
                        void *stream)
{
    if (bytes <= 0 || bytes % 1024 != 0 || grid <= 0 || !src || !sink)
        return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const v4i *p = static_cast<const v4i *>(src);
    if (kind == 0) {
        const int64_t n16 = bytes / 16;
        if (depth == 4) read_regs<4><<<grid, 256, 0, st>>>(p, n16, sink);
        else if (depth == 8) read_regs<8><<<grid, 256, 0, st>>>(p, n16, sink);
        else if (depth == 16) read_regs<16><<<grid, 256, 0, st>>>(p, n16, sink);
        else return (int)hipErrorInvalidValue;
    } else if (kind == 1) {
        const int64_t n1k = bytes / 1024;
        if (depth == 2) read_lds<2><<<grid, 256, 0, st>>>(p, n1k, sink);
        else if (depth == 4) read_lds<4><<<grid, 256, 0, st>>>(p, n1k, sink);
        else if (depth == 8) read_lds<8><<<grid, 256, 0, st>>>(p, n1k, sink);
        else return (int)hipErrorInvalidValue;
    } else {
        return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

extern "C" int mqp_mix(int k, int iters, int grid, float *sink, void *stream)
{
    if (iters <= 0 || grid <= 0 || !sink)
        return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (k == 0) mix<0><<<grid, 256, 0, st>>>(iters, sink);
    else if (k == 2) mix<2><<<grid, 256, 0, st>>>(iters, sink);
    else if (k == 3) mix<3><<<grid, 256, 0, st>>>(iters, sink);
    else if (k == 4) mix<4><<<grid, 256, 0, st>>>(iters, sink);
    else if (k == 10) mix<10><<<grid, 256, 0, st>>>(iters, sink);
    else if (k == 11) mix<11><<<grid, 256, 0, st>>>(iters, sink);
    else if (k == 12) mix<12><<<grid, 256, 0, st>>>(iters, sink);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}
