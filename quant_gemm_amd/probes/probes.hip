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
//       product and fma. k = 20..23, 30: a sub-block step of the GEMM
//       inner loop with its operands read from LDS (4 tiles of 32 x 32 per
//       wavefront, one 32-value sub-block per iteration):
//         20: two chained v_mfma_f32_32x32x16_f16 per tile (the f16 route,
//             6-bit scale folded into the weights: sc * q is exact in f16);
//         21: 20 plus one fma per result (J times the activation scale);
//         22: 21 with the weights converted from raw nibbles in registers
//             (mask, then v_cvt_scalef32_pk_f16_fp8: the nibble is an e4m3
//             code q * 2^-9, scaled by sc * 2^9 to sc * q exactly);
//         23: 22 with the activations converted from int8 in registers;
//         30: the int8 route for comparison: nibble unpack, one
//             v_mfma_i32_32x32x32_i8 per tile, then cvt, mul, fma.
//       sink holds grid * 256 floats.
//   mqp_valu(k, iters, grid, sink, cycles, stream)
//       the VALU issue rate: per iteration 16 independent f32 results per
//       lane, updated by
//         k = 0: fma;  1: convert (from an int counter) and fma;
//         2: scale product and fma;  3: convert, scale product and fma (the
//         GEMM epilogue, plus the counter's integer add);
//         7, 8: 3 plus one or two independent v_mfma_i32_32x32x32_i8;
//         9: 3 plus one independent v_mfma_f32_32x32x16_bf16.
//       Workgroups of 256 threads; each wavefront writes the shader clocks
//       it ran (s_memtime) to cycles[wavefront], so clock and issue cycles
//       per instruction follow from the launch time. sink holds grid * 256
//       floats, cycles grid * 4 int64.
// All return the hipError_t of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

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

// Two e4m3 codes (bytes 2 hi, 2 hi + 1 of w) as an f16 pair, times s.
__device__ __forceinline__ uint32_t e4m3x2_to_f16(uint32_t w, float s, bool hi)
{
    const v2h r = hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, s, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, s, false);
    return __builtin_bit_cast(uint32_t, r);
}

// Four int8 as two exact f16 pairs: x + 128 under the exponent of 1024,
// then 1152 subtracted.
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, uint32_t &h01, uint32_t &h23)
{
    const uint32_t u = w ^ 0x80808080u;
    const v2h c = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    h01 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + c);
    h23 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + c);
}

// LDS-fed inner-loop mixes (k = 20..23, 30; see the header). The 64 KB of
// LDS hold arbitrary data; every index is masked into it.
template <int K>
__global__ __launch_bounds__(256, 2) void mix_lds(int iters, float *sink)
{
    __shared__ v4i lds[4096];
    const int tid = threadIdx.x, lane = tid & 63;
    for (int i = tid; i < 4096; i += 256)
        lds[i] = v4i{i * 0x01030507, i * 0x0b0d1113, i ^ 0x5a5a5a5a, i * 7};
    __syncthreads();
    const float *ldf = reinterpret_cast<const float *>(lds);
    v16f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        acc[t] = v16f{};
    v4i raw[4];
    float sc = 2.0f, f = 1e-3f;
    for (int i = 0; i < iters; ++i) {
        const int base = ((i & 15) * 64 + lane) & 1023;
        const v4i ai = lds[base];
        float dv[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int o = 4 * (2048 + ((((i & 7) * 64 + lane) * 4 + 256 * g) & 1023));
            const float4 d4 = *reinterpret_cast<const float4 *>(ldf + o);
            dv[4 * g] = d4.x;
            dv[4 * g + 1] = d4.y;
            dv[4 * g + 2] = d4.z;
            dv[4 * g + 3] = d4.w;
        }
        const bool hi = i & 1;
        if (!hi) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                raw[t] = lds[(base + 128 * (t + 1)) & 4095];
        }
        if constexpr (K == 30) {
            v16i I[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const v4i b = hi ? ((raw[t] >> 4) & 0x0f0f0f0f) : (raw[t] & 0x0f0f0f0f);
                I[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ai, b, v16i{}, 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float fw = f * (1.0f + 1e-3f * t);
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[t][v] = __builtin_fmaf((float)I[t][v], dv[v] * fw, acc[t][v]);
            }
            f += 1e-7f;
            continue;
        } else {
            v8h a0, a1;
            if constexpr (K >= 23) {
                uint32_t ah[8];
                i8x4_to_f16(ai.x, ah[0], ah[1]);
                i8x4_to_f16(ai.y, ah[2], ah[3]);
                i8x4_to_f16(ai.z, ah[4], ah[5]);
                i8x4_to_f16(ai.w, ah[6], ah[7]);
                a0 = __builtin_bit_cast(v8h, v4i{(int)ah[0], (int)ah[1], (int)ah[2], (int)ah[3]});
                a1 = __builtin_bit_cast(v8h, v4i{(int)ah[4], (int)ah[5], (int)ah[6], (int)ah[7]});
            } else {
                a0 = __builtin_bit_cast(v8h, ai);
                a1 = __builtin_bit_cast(v8h, lds[base + 1024]);
            }
            v16f J[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                v8h b0, b1;
                if constexpr (K >= 22) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = hi ? (((uint32_t)raw[t][e] >> 4) & 0x0f0f0f0fu) : ((uint32_t)raw[t][e] & 0x0f0f0f0fu);
                    const float s = sc + t;
                    b0 = __builtin_bit_cast(v8h, v4i{(int)e4m3x2_to_f16(w[0], s, false), (int)e4m3x2_to_f16(w[0], s, true),
                                                     (int)e4m3x2_to_f16(w[1], s, false), (int)e4m3x2_to_f16(w[1], s, true)});
                    b1 = __builtin_bit_cast(v8h, v4i{(int)e4m3x2_to_f16(w[2], s, false), (int)e4m3x2_to_f16(w[2], s, true),
                                                     (int)e4m3x2_to_f16(w[3], s, false), (int)e4m3x2_to_f16(w[3], s, true)});
                } else {
                    b0 = __builtin_bit_cast(v8h, lds[(base + 128 * (t + 5)) & 4095]);
                    b1 = __builtin_bit_cast(v8h, lds[(base + 128 * (t + 9)) & 4095]);
                }
                if constexpr (K == 20) {
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc[t], 0, 0, 0);
                } else {
                    J[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, v16f{}, 0, 0, 0);
                    J[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, J[t], 0, 0, 0);
                }
            }
            if constexpr (K >= 21) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc[t][v] = __builtin_fmaf(J[t][v], dv[v], acc[t][v]);
            }
            sc += 1.0f;
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            s += acc[t][v];
    sink[(int64_t)blockIdx.x * 256 + tid] = s;
}

// VALU issue-rate probe (see the header). The MFMAs of k = 7..9 take no
// VALU result, so they add matrix-core work without adding dependencies.
template <int K>
__global__ __launch_bounds__(256) void valu_rate(int iters, float s0, float *sink, long long *cycles)
{
    const long long c0 = clock64();
    const int tid = blockIdx.x * 256 + threadIdx.x;
    float acc[16], x[16];
    int xi[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        acc[v] = tid * 1e-7f + v;
        x[v] = 1.0f + v * 1e-3f;
        xi[v] = tid + v * 977;
    }
    v16i mi = {};
    v16f mf = {};
    const v4i ma = {tid, tid * 3, tid ^ 5, 7}, mb = {tid * 5, 11, tid, 13};
    float s = s0;   // a launch argument, so that no product folds away
    for (int i = 0; i < iters; ++i) {
        if constexpr (K == 7 || K == 8) {
#pragma unroll
            for (int m = 0; m < K - 6; ++m)
                mi = __builtin_amdgcn_mfma_i32_32x32x32_i8(ma, mb, mi, 0, 0, 0);
        }
        if constexpr (K == 9)
            mf = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ma), __builtin_bit_cast(v8bf, mb), mf,
                                                         0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            if constexpr (K == 0) {
                acc[v] = __builtin_fmaf(x[v], s, acc[v]);
            } else if constexpr (K == 1) {
                acc[v] = __builtin_fmaf((float)xi[v], s, acc[v]);
                xi[v] += 1;
            } else if constexpr (K == 2) {
                acc[v] = __builtin_fmaf(x[v], s * x[15 - v], acc[v]);
            } else {
                acc[v] = __builtin_fmaf((float)xi[v], s * x[15 - v], acc[v]);
                xi[v] += 1;
            }
        }
        s += 1e-9f;
    }
    float r = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v)
        r += acc[v] + (float)xi[v] + (float)mi[v] + mf[v];
    sink[tid] = r;
    const long long c1 = clock64();
    if ((threadIdx.x & 63) == 0)
        cycles[tid >> 6] = c1 - c0;
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
    else if (k == 20) mix_lds<20><<<grid, 256, 0, st>>>(iters, sink);
    else if (k == 21) mix_lds<21><<<grid, 256, 0, st>>>(iters, sink);
    else if (k == 22) mix_lds<22><<<grid, 256, 0, st>>>(iters, sink);
    else if (k == 23) mix_lds<23><<<grid, 256, 0, st>>>(iters, sink);
    else if (k == 30) mix_lds<30><<<grid, 256, 0, st>>>(iters, sink);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

extern "C" int mqp_valu(int k, int iters, int grid, float *sink, long long *cycles, void *stream)
{
    if (iters <= 0 || grid <= 0 || !sink || !cycles)
        return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (k == 0) valu_rate<0><<<grid, 256, 0, st>>>(iters, 1.0f, sink, cycles);
    else if (k == 1) valu_rate<1><<<grid, 256, 0, st>>>(iters, 1.0f, sink, cycles);
    else if (k == 2) valu_rate<2><<<grid, 256, 0, st>>>(iters, 1.0f, sink, cycles);
    else if (k == 3) valu_rate<3><<<grid, 256, 0, st>>>(iters, 1.0f, sink, cycles);
    else if (k == 7) valu_rate<7><<<grid, 256, 0, st>>>(iters, 1.0f, sink, cycles);
    else if (k == 8) valu_rate<8><<<grid, 256, 0, st>>>(iters, 1.0f, sink, cycles);
    else if (k == 9) valu_rate<9><<<grid, 256, 0, st>>>(iters, 1.0f, sink, cycles);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}
