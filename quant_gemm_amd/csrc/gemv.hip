// Decode GEMV for Q4_K / Q5_K / Q6_K weights x per-32 int8 activations (gfx950).
//
// The decode path of the pages streams the quantized weight bytes once per
// token with 4-way int8 dot products (minfer Features, "GPU — CUDA": decode
// uses the MMVQ weight-streaming path; minfer Support Matrix, "CUDA notes":
// dp4a MMVQ kernels for Q4_K/Q6_K at one token). Here the same idea is laid
// out for 64-wide wavefronts:
//   * a wavefront owns R consecutive weight rows; lane i owns the same
//     K-slices of every one of them, so its slice of the int8 activation
//     plane is loaded once and reused for all R rows and M (<= 8) tokens;
//   * weights stream with 16-byte loads (Q4_K) or aligned dword loads
//     realigned in registers (Q6_K, whose 210-byte blocks are only 2-byte
//     aligned);
//   * each 16- or 32-value scale group is an exact int32 dot (v_dot4),
//     scaled in f32; the 64 lane partials are summed across the wavefront.
//
// HBM-bound: the weight bytes dominate (4.5 bits/weight for Q4_K, 6.5625 for
// Q6_K); activations (K bytes + K/8 floats per token) stay in cache.
#include "mq_device.h"
#include "mq_launch.h"
#include "quant_core.h"

#include <type_traits>

namespace mq {
namespace {

constexpr int GEMV_WAVES = 4;          // wavefronts per workgroup
// The persistent Q4_K stream runs 8 wavefronts per workgroup (32 per CU in
// its 1024-workgroup grid): measured 5% faster than 4 at N = 18944, equal
// on the smaller matrices.
constexpr int STREAM_WAVES = 8;
#ifndef GEMV_STREAM_WGS
#define GEMV_STREAM_WGS 1024        // workgroups of the persistent stream kernel
#endif
#ifndef GEMV_STREAM_NP_MAX
#define GEMV_STREAM_NP_MAX 6        // passes per row the persistent Q4_K stream handles
#endif
#ifndef GEMV_STREAM_D
#define GEMV_STREAM_D 1             // rows in flight per wavefront (beside the one computed)
#endif

// ---------------------------------------------------------------- Q4_K
// The R rows of a wavefront are consecutive, so their blocks form one
// contiguous byte range of R * K/256 * 144 bytes. The wavefront streams it
// as 16-byte chunks, 7 blocks (63 lanes) per pass: lane 9s + p holds chunk p
// of block s of the pass. Chunk 0 is the block header (d, dmin, 6-bit
// codes); chunk p = 1..8 holds quant bytes 16(p-1)..16(p-1)+15, i.e.
// positions po..po+15 (po = 16*((p-1)&1)) of sub-blocks j0 = 2*((p-1)>>1)
// (low nibbles) and j0+1 (high nibbles). The header reaches the other eight
// lanes of its block through ds_bpermute. Every load of a lane is issued
// before any of its arithmetic, so a wavefront waits on memory once.
//
// With ACT_LDS the workgroup first copies the whole activation plane
// (M x K int8 plus the per-32 scales and sums, at most GEMV_ACT_LDS bytes)
// into LDS; the loads for it are issued before the weight loads, so the copy
// overlaps the weight stream, and the dot products then read activations
// from LDS instead of making one cache round trip per pass.
constexpr int GEMV_ACT_LDS = 32 * 1024;

// Copy the activation plane (q, then d, then s: M*K + 2*M*K/8 bytes, a
// multiple of 16) into LDS. Loads are issued here; the stores wait for them.
// WAVES: wavefronts of the workgroup that copies.
// BYTES: the largest plane the copy handles.
template <int WAVES = GEMV_WAVES, int BYTES = GEMV_ACT_LDS>
struct ActCopy {
    static constexpr int NT = 64 * WAVES;
    static constexpr int MAXC = BYTES / 16 / NT;         // chunks per thread
    static_assert(MAXC * 16 * NT == BYTES, "whole chunks per thread");
    v4i v[MAXC];
};

template <int WAVES, int BYTES>
__device__ __forceinline__ void act_load(ActCopy<WAVES, BYTES> &c, const int8_t *q, const float *d,
                                         const float *s, int M, int K)
{
    const int qchunks = M * K / 16, dchunks = M * K / 128;
#pragma unroll
    for (int i = 0; i < ActCopy<WAVES, BYTES>::MAXC; ++i) {
        const int ch = threadIdx.x + i * ActCopy<WAVES, BYTES>::NT;
        const v4i *src;
        if (ch < qchunks)
            src = reinterpret_cast<const v4i *>(q) + ch;
        else if (ch < qchunks + dchunks)
            src = reinterpret_cast<const v4i *>(d) + (ch - qchunks);
        else
            src = reinterpret_cast<const v4i *>(s) + min(ch - qchunks - dchunks, dchunks - 1);
        c.v[i] = ch < qchunks + 2 * dchunks ? *src : v4i{0, 0, 0, 0};
    }
}

template <int WAVES, int BYTES>
__device__ __forceinline__ void act_store(const ActCopy<WAVES, BYTES> &c, v4i *lds, int M, int K)
{
    const int nchunks = M * K / 16 + 2 * (M * K / 128);
#pragma unroll
    for (int i = 0; i < ActCopy<WAVES, BYTES>::MAXC; ++i) {
        const int ch = threadIdx.x + i * ActCopy<WAVES, BYTES>::NT;
        if (ch < nchunks)
            lds[ch] = c.v[i];
    }
}

// This lane's partial dot products for the R consecutive rows that start at
// `base` (each nb blocks; `rows` of them are real), accumulated into
// acc[r][m]. qa / da / sa are the activation plane (global memory or its
// LDS copy). after_first_loads() runs once, right after the first batch of
// weight loads is issued: the activation copy into LDS goes there, so that
// it overlaps the weight stream.
template <int MT, int R, int IT, bool PIPE = false, class F>
__device__ __forceinline__ void q4k_rows(const uint8_t *__restrict__ base, int rows, int nb, int K, int M,
                                         const int8_t *qa, const float *da, const float *sa, int lane,
                                         float (&acc)[R][MT], F &&after_first_loads)
{
    const int nb32 = K >> 5;
    const int total = rows * nb;                 // blocks of this wavefront
    const int slot = lane / 9;                   // block within a pass (7 = idle lane)
    const int part = lane - 9 * slot;            // chunk within the block
    const int hdr_lane = 9 * slot;
    // this lane's (row, block) position, advanced by 7 blocks per pass
    int rl = 0, blk = slot;
    while (blk >= nb) { blk -= nb; ++rl; }
    auto load = [&](v4i (&v)[IT], int it0) {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int fb = it0 + 7 * i + slot;
            v[i] = (slot < 7 && fb < total)
                       ? __builtin_nontemporal_load(reinterpret_cast<const v4i *>(base + (int64_t)fb * 144 + 16 * part))
                       : v4i{0, 0, 0, 0};
        }
    };
    auto compute = [&](const v4i (&v)[IT], int it0) {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int fb = it0 + 7 * i + slot;
            // block header from lane 9*slot
            const uint32_t h0 = __builtin_amdgcn_ds_bpermute(4 * hdr_lane, v[i].x);
            const uint32_t h1 = __builtin_amdgcn_ds_bpermute(4 * hdr_lane, v[i].y);
            const uint32_t h2 = __builtin_amdgcn_ds_bpermute(4 * hdr_lane, v[i].z);
            const uint32_t h3 = __builtin_amdgcn_ds_bpermute(4 * hdr_lane, v[i].w);
            if (slot < 7 && fb < total && part > 0) {
                const int c = part - 1;
                const int cc = c >> 1;
                const int po = (c & 1) << 4;
                const int k0 = (blk << 8) + (cc << 6) + po;   // sub-block j0, positions po..
                const int b0 = (blk << 3) + (cc << 1);        // its 32-block index
                const float dd = f16_bits_to_f32(h0);
                const float dm = f16_bits_to_f32(h0 >> 16);
                const uint32_t scw = cc < 2 ? (h1 & 0x3f3f3f3fu)
                                            : ((h3 & 0x0f0f0f0fu) | ((h1 >> 2) & 0x30303030u));
                const uint32_t mw = cc < 2 ? (h2 & 0x3f3f3f3fu)
                                           : (((h3 >> 4) & 0x0f0f0f0fu) | ((h2 >> 2) & 0x30303030u));
                const int sh = (cc & 1) << 4;
                const float f0 = dd * (float)((scw >> sh) & 0xffu);
                const float f1 = dd * (float)((scw >> (sh + 8)) & 0xffu);
                const float g0 = po == 0 ? dm * (float)((mw >> sh) & 0xffu) : 0.0f;
                const float g1 = po == 0 ? dm * (float)((mw >> (sh + 8)) & 0xffu) : 0.0f;
                const int lo0 = v[i].x & 0x0f0f0f0f, lo1 = v[i].y & 0x0f0f0f0f;
                const int lo2 = v[i].z & 0x0f0f0f0f, lo3 = v[i].w & 0x0f0f0f0f;
                const int hi0 = (v[i].x >> 4) & 0x0f0f0f0f, hi1 = (v[i].y >> 4) & 0x0f0f0f0f;
                const int hi2 = (v[i].z >> 4) & 0x0f0f0f0f, hi3 = (v[i].w >> 4) & 0x0f0f0f0f;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m < M) {
                        const v4i xa = *reinterpret_cast<const v4i *>(qa + (int64_t)m * K + k0);
                        const v4i xb = *reinterpret_cast<const v4i *>(qa + (int64_t)m * K + k0 + 32);
                        const float2 dpair = *reinterpret_cast<const float2 *>(da + (int64_t)m * nb32 + b0);
                        const float2 spair = *reinterpret_cast<const float2 *>(sa + (int64_t)m * nb32 + b0);
                        int i0 = dot4(lo0, xa.x, 0);
                        i0 = dot4(lo1, xa.y, i0);
                        i0 = dot4(lo2, xa.z, i0);
                        i0 = dot4(lo3, xa.w, i0);
                        int i1 = dot4(hi0, xb.x, 0);
                        i1 = dot4(hi1, xb.y, i1);
                        i1 = dot4(hi2, xb.z, i1);
                        i1 = dot4(hi3, xb.w, i1);
                        float contrib = (float)i0 * (dpair.x * f0);
                        contrib = fmaf((float)i1, dpair.y * f1, contrib);
                        contrib = fmaf(-g0, spair.x, contrib);
                        contrib = fmaf(-g1, spair.y, contrib);
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            acc[r][m] += rl == r ? contrib : 0.0f;
                    }
                }
            }
            blk += 7;
            while (blk >= nb) { blk -= nb; ++rl; }
        }
    };
    if constexpr (!PIPE) {
        for (int it0 = 0; it0 < max(total, 1); it0 += 7 * IT) {
            v4i v[IT];
            load(v, it0);
            if (it0 == 0)
                after_first_loads();
            compute(v, it0);
        }
    } else {
        // two batches: the loads of the next batch are in flight while this
        // one is reduced (long rows, several batches per wavefront)
        v4i va[IT], vb[IT];
        load(va, 0);
        after_first_loads();
        for (int it0 = 0; it0 < max(total, 1); it0 += 14 * IT) {
            const bool b_live = it0 + 7 * IT < total;
            if (b_live)
                load(vb, it0 + 7 * IT);
            compute(va, it0);
            if (!b_live)
                break;
            if (it0 + 14 * IT < total)
                load(va, it0 + 14 * IT);
            compute(vb, it0 + 7 * IT);
        }
    }
}

template <int MT, int R, int IT, bool ACT_LDS, bool PIPE = false>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_q4k_kernel(
    const uint8_t *__restrict__ W, const int8_t *__restrict__ q,
    const float *__restrict__ dx, const float *__restrict__ sx, int M, int N,
    int K, float *__restrict__ out)
{
    __shared__ v4i act[ACT_LDS ? GEMV_ACT_LDS / 16 : 1];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * GEMV_WAVES + wave) * R;
    ActCopy<> ac;
    if constexpr (ACT_LDS)
        act_load(ac, q, dx, sx, M, K);
    const int nb = K >> 8;
    const int rows = max(0, min(R, N - row0));  // 0 for a wavefront past the last row
    const uint8_t *base = W + (int64_t)row0 * nb * 144;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[r][m] = 0.0f;
    const int8_t *qa = q;                        // activation sources: global or LDS
    const float *da = dx, *sa = sx;
    if constexpr (ACT_LDS) {
        qa = reinterpret_cast<const int8_t *>(act);
        da = reinterpret_cast<const float *>(qa + M * K);
        sa = da + M * (K >> 5);
    }
    q4k_rows<MT, R, IT, PIPE>(base, rows, nb, K, M, qa, da, sa, lane, acc, [&] {
        if constexpr (ACT_LDS) {
            act_store(ac, act, M, K);
            __syncthreads();
        }
    });
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float v = wave_sum(acc[r][m]);
            if (lane == 0 && m < M && r < rows)
                out[(int64_t)m * N + row0 + r] = v;
        }
    }
}

// Persistent, software-pipelined form of the same stream for short rows
// (K <= NP * 7 * 256). A fixed grid of wavefronts walks the rows
// n = w, w + NW, w + 2 NW, ... (NW wavefronts in all, so neighbouring
// wavefronts read neighbouring rows). Each row is NP passes of 7 blocks; the
// loads of the next D rows stay in flight while a row is reduced across the
// wavefront and stored. Blocks past the end of a row are clamped to its last
// block and masked afterwards; past its last row a wavefront loads nothing
// (measured on MI355X: one row ahead, without clamped tail loads, is the
// fastest depth, most of all for short matrices).
//
// The N rows may come from two matrices of N1 rows each sharing the
// activation plane (the gate and up matrices of an FFN): rows n < N1 are
// row n of W into out, rows n >= N1 row n - N1 of W2 into out2 (both
// outputs M x N1). A single matrix passes N1 = N.
//
// REG (one token, rows of up to 3 passes): a lane's activation values,
// scales and sums are the same for every row it reads, so it loads them
// once into registers and the workgroup keeps no LDS copy (no copy, no
// barrier); such grids run 4 wavefronts per workgroup (WV). Measured on
// MI355X at 18944 x 3584: 9.1 us against 10.5-11.1 us for the LDS copy with
// 8 wavefronts per workgroup on the same boxes.
constexpr int stream_act_bytes(int MT) { return MT > 4 ? 40 * 1024 : GEMV_ACT_LDS; }

template <int MT, int NP, int D, int WV = STREAM_WAVES, bool REG = false>
__global__ __launch_bounds__(64 * WV) void gemv_q4k_stream_kernel(
    const uint8_t *__restrict__ W, const uint8_t *__restrict__ W2, int N1,
    const int8_t *__restrict__ q, const float *__restrict__ dx, const float *__restrict__ sx,
    int M, int N, int K, float *__restrict__ out, float *__restrict__ out2)
{
    static_assert(!REG || (MT == 1 && NP <= 3), "register activations: one token, short rows");
    constexpr int AB = REG ? 16 * 64 * WV : stream_act_bytes(MT);
    __shared__ v4i act[REG ? 1 : AB / 16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = gridDim.x * WV;
    const int w = blockIdx.x * WV + wave;
    ActCopy<WV, AB> ac;
    if constexpr (!REG)
        act_load(ac, q, dx, sx, M, K);

    const int nb = K >> 8;
    const int nb32 = K >> 5;
    const int64_t rowb = (int64_t)nb * 144;
    const int slot = lane / 9;
    const int part = lane - 9 * slot;
    const int hdr_lane = 9 * slot;
    const int nrows = w < N ? (N - 1 - w) / nw + 1 : 0;   // rows of this wavefront

    // per pass p this lane owns block 7p + slot of the row
    bool valid[NP];
    int boff[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int blk = 7 * p + slot;
        valid[p] = slot < 7 && blk < nb;
        boff[p] = min(blk, nb - 1) * 144 + 16 * part;
    }

    auto row = [&](int n) { return n < N1 ? W + (int64_t)n * rowb : W2 + (int64_t)(n - N1) * rowb; };
    v4i ring[D][NP];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        const uint8_t *r = row(min(w + d * nw, N - 1));
#pragma unroll
        for (int p = 0; p < NP; ++p)
            ring[d][p] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(r + boff[p]));
    }
    const int8_t *qa = q;
    const float *da = dx, *sa = sx;
    // REG: this lane's activation values (positions k0, k0 + 32 of pass p),
    // scales and sums, read once
    v4i rxa[REG ? NP : 1], rxb[REG ? NP : 1];
    float2 rdp[REG ? NP : 1], rsp[REG ? NP : 1];
    if constexpr (REG) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int blk = min(7 * p + slot, nb - 1);
            const int c = max(part - 1, 0);
            const int k0 = (blk << 8) + ((c >> 1) << 6) + ((c & 1) << 4);
            const int b0 = (blk << 3) + ((c >> 1) << 1);
            rxa[p] = *reinterpret_cast<const v4i *>(q + k0);
            rxb[p] = *reinterpret_cast<const v4i *>(q + k0 + 32);
            rdp[p] = *reinterpret_cast<const float2 *>(dx + b0);
            rsp[p] = *reinterpret_cast<const float2 *>(sx + b0);
        }
    } else {
        act_store(ac, act, M, K);
        __syncthreads();
        qa = reinterpret_cast<const int8_t *>(act);
        da = reinterpret_cast<const float *>(qa + M * K);
        sa = da + M * nb32;
    }

    for (int i0 = 0; i0 < nrows; i0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = i0 + d;
            if (i < nrows) {
                float acc[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    acc[m] = 0.0f;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const v4i v = ring[d][p];
                    const uint32_t h0 = __builtin_amdgcn_ds_bpermute(4 * hdr_lane, v.x);
                    const uint32_t h1 = __builtin_amdgcn_ds_bpermute(4 * hdr_lane, v.y);
                    const uint32_t h2 = __builtin_amdgcn_ds_bpermute(4 * hdr_lane, v.z);
                    const uint32_t h3 = __builtin_amdgcn_ds_bpermute(4 * hdr_lane, v.w);
                    if (valid[p] && part > 0) {
                        const int blk = 7 * p + slot;
                        const int c = part - 1;
                        const int cc = c >> 1;
                        const int po = (c & 1) << 4;
                        const int k0 = (blk << 8) + (cc << 6) + po;
                        const int b0 = (blk << 3) + (cc << 1);
                        const float dd = f16_bits_to_f32(h0);
                        const float dm = f16_bits_to_f32(h0 >> 16);
                        const uint32_t scw = cc < 2 ? (h1 & 0x3f3f3f3fu)
                                                    : ((h3 & 0x0f0f0f0fu) | ((h1 >> 2) & 0x30303030u));
                        const uint32_t mw = cc < 2 ? (h2 & 0x3f3f3f3fu)
                                                   : (((h3 >> 4) & 0x0f0f0f0fu) | ((h2 >> 2) & 0x30303030u));
                        const int sh = (cc & 1) << 4;
                        const float f0 = dd * (float)((scw >> sh) & 0xffu);
                        const float f1 = dd * (float)((scw >> (sh + 8)) & 0xffu);
                        const float g0 = po == 0 ? dm * (float)((mw >> sh) & 0xffu) : 0.0f;
                        const float g1 = po == 0 ? dm * (float)((mw >> (sh + 8)) & 0xffu) : 0.0f;
                        const int lo0 = v.x & 0x0f0f0f0f, lo1 = v.y & 0x0f0f0f0f;
                        const int lo2 = v.z & 0x0f0f0f0f, lo3 = v.w & 0x0f0f0f0f;
                        const int hi0 = (v.x >> 4) & 0x0f0f0f0f, hi1 = (v.y >> 4) & 0x0f0f0f0f;
                        const int hi2 = (v.z >> 4) & 0x0f0f0f0f, hi3 = (v.w >> 4) & 0x0f0f0f0f;
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            if (m < M) {
                                v4i xa, xb;
                                float2 dp, sp;
                                if constexpr (REG) {
                                    xa = rxa[p];
                                    xb = rxb[p];
                                    dp = rdp[p];
                                    sp = rsp[p];
                                } else {
                                    xa = *reinterpret_cast<const v4i *>(qa + m * K + k0);
                                    xb = *reinterpret_cast<const v4i *>(qa + m * K + k0 + 32);
                                    dp = *reinterpret_cast<const float2 *>(da + m * nb32 + b0);
                                    sp = *reinterpret_cast<const float2 *>(sa + m * nb32 + b0);
                                }
                                int i0v = dot4(lo0, xa.x, 0);
                                i0v = dot4(lo1, xa.y, i0v);
                                i0v = dot4(lo2, xa.z, i0v);
                                i0v = dot4(lo3, xa.w, i0v);
                                int i1v = dot4(hi0, xb.x, 0);
                                i1v = dot4(hi1, xb.y, i1v);
                                i1v = dot4(hi2, xb.z, i1v);
                                i1v = dot4(hi3, xb.w, i1v);
                                float a = fmaf((float)i0v, dp.x * f0, acc[m]);
                                a = fmaf((float)i1v, dp.y * f1, a);
                                a = fmaf(-g0, sp.x, a);
                                acc[m] = fmaf(-g1, sp.y, a);
                            }
                        }
                    }
                }
                // refill this ring slot with the row D ahead (a wave-uniform
                // branch: past its last row the wavefront loads nothing, so
                // the tail does not pile clamped loads onto one row)
                if (i + D < nrows) {
                    const uint8_t *r = row(w + (i + D) * nw);
#pragma unroll
                    for (int p = 0; p < NP; ++p)
                        ring[d][p] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(r + boff[p]));
                }
                const int n = w + i * nw;
                float *o = n < N1 ? out + n : out2 + (n - N1);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const float v = wave_sum(acc[m]);
                    if (lane == 0 && m < M)
                        o[(int64_t)m * N1] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- Q5_K
// 176-byte blocks (16-byte aligned): header (d, dmin, 6-bit codes) at 0, the
// high-bit plane qh[32] at 16, the low nibbles qs[128] at 48. Eight lanes
// share a block, 8 blocks per pass: lane 8s + c loads the 16 quant bytes
// 16c..16c+15 (positions po..po+15, po = 16 (c & 1), of sub-blocks
// j0 = 2 (c >> 1) in the low nibbles and j0 + 1 in the high ones), the
// matching half qh[po..po+15] of the high-bit plane (bit j of qh[i] is the
// fifth bit of position i of sub-block j) and the header itself: three
// 16-byte loads, no cross-lane exchange. The replicated header and qh loads
// hit the lines the block's own loads bring in, so HBM sees each byte once.
template <int MT, int R, int IT, bool PIPE = false, class F>
__device__ __forceinline__ void q5k_rows(const uint8_t *__restrict__ base, int rows, int nb, int K, int M,
                                         const int8_t *qa, const float *da, const float *sa, int lane,
                                         float (&acc)[R][MT], F &&after_first_loads)
{
    const int nb32 = K >> 5;
    const int total = rows * nb;
    const int slot = lane >> 3;                  // block within a pass
    const int c = lane & 7;                      // quant chunk within the block
    const int cc = c >> 1, po = (c & 1) << 4;
    const int j0 = 2 * cc;
    // rotating a qh dword right by j + 28 (mod 32) puts bit j of every byte
    // at bit 4 of the same byte
    const int rot0 = (j0 + 28) & 31, rot1 = (j0 + 29) & 31;
    int rl = 0, blk = slot;
    while (blk >= nb) { blk -= nb; ++rl; }
    struct Batch {
        v4i hv[IT], hq[IT], v[IT];
    };
    auto load = [&](Batch &bt, int it0) {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int fb = it0 + 8 * i + slot;
            const uint8_t *b = base + (int64_t)min(fb, max(total, 1) - 1) * 176;
            bt.hv[i] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(b));
            bt.hq[i] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(b + 16 + po));
            bt.v[i] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(b + 48 + 16 * c));
        }
    };
    auto compute = [&](const Batch &bt, int it0) {
        const auto &hv = bt.hv;
        const auto &hq = bt.hq;
        const auto &v = bt.v;
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int fb = it0 + 8 * i + slot;
            if (fb < total) {
                const uint32_t h0 = hv[i].x, h1 = hv[i].y, h2 = hv[i].z, h3 = hv[i].w;
                const int k0 = (blk << 8) + (cc << 6) + po;
                const int b0 = (blk << 3) + (cc << 1);
                const float dd = f16_bits_to_f32(h0);
                const float dm = f16_bits_to_f32(h0 >> 16);
                const uint32_t scw = cc < 2 ? (h1 & 0x3f3f3f3fu)
                                            : ((h3 & 0x0f0f0f0fu) | ((h1 >> 2) & 0x30303030u));
                const uint32_t mw = cc < 2 ? (h2 & 0x3f3f3f3fu)
                                           : (((h3 >> 4) & 0x0f0f0f0fu) | ((h2 >> 2) & 0x30303030u));
                const int sh = (cc & 1) << 4;
                const float f0 = dd * (float)((scw >> sh) & 0xffu);
                const float f1 = dd * (float)((scw >> (sh + 8)) & 0xffu);
                const float g0 = po == 0 ? dm * (float)((mw >> sh) & 0xffu) : 0.0f;
                const float g1 = po == 0 ? dm * (float)((mw >> (sh + 8)) & 0xffu) : 0.0f;
                // 5-bit quants: bit j0 (j0 + 1) of each qh byte rotated to bit 4
                const uint32_t hx = (uint32_t)hq[i].x, hy = (uint32_t)hq[i].y;
                const uint32_t hz = (uint32_t)hq[i].z, hw = (uint32_t)hq[i].w;
                const int lo0 = (v[i].x & 0x0f0f0f0f) | (int)(__builtin_rotateright32(hx, rot0) & 0x10101010u);
                const int lo1 = (v[i].y & 0x0f0f0f0f) | (int)(__builtin_rotateright32(hy, rot0) & 0x10101010u);
                const int lo2 = (v[i].z & 0x0f0f0f0f) | (int)(__builtin_rotateright32(hz, rot0) & 0x10101010u);
                const int lo3 = (v[i].w & 0x0f0f0f0f) | (int)(__builtin_rotateright32(hw, rot0) & 0x10101010u);
                const int hi0 = ((v[i].x >> 4) & 0x0f0f0f0f) | (int)(__builtin_rotateright32(hx, rot1) & 0x10101010u);
                const int hi1 = ((v[i].y >> 4) & 0x0f0f0f0f) | (int)(__builtin_rotateright32(hy, rot1) & 0x10101010u);
                const int hi2 = ((v[i].z >> 4) & 0x0f0f0f0f) | (int)(__builtin_rotateright32(hz, rot1) & 0x10101010u);
                const int hi3 = ((v[i].w >> 4) & 0x0f0f0f0f) | (int)(__builtin_rotateright32(hw, rot1) & 0x10101010u);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m < M) {
                        const v4i xa = *reinterpret_cast<const v4i *>(qa + (int64_t)m * K + k0);
                        const v4i xb = *reinterpret_cast<const v4i *>(qa + (int64_t)m * K + k0 + 32);
                        const float2 dpair = *reinterpret_cast<const float2 *>(da + (int64_t)m * nb32 + b0);
                        const float2 spair = *reinterpret_cast<const float2 *>(sa + (int64_t)m * nb32 + b0);
                        int i0 = dot4(lo0, xa.x, 0);
                        i0 = dot4(lo1, xa.y, i0);
                        i0 = dot4(lo2, xa.z, i0);
                        i0 = dot4(lo3, xa.w, i0);
                        int i1 = dot4(hi0, xb.x, 0);
                        i1 = dot4(hi1, xb.y, i1);
                        i1 = dot4(hi2, xb.z, i1);
                        i1 = dot4(hi3, xb.w, i1);
                        float contrib = (float)i0 * (dpair.x * f0);
                        contrib = fmaf((float)i1, dpair.y * f1, contrib);
                        contrib = fmaf(-g0, spair.x, contrib);
                        contrib = fmaf(-g1, spair.y, contrib);
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            acc[r][m] += rl == r ? contrib : 0.0f;
                    }
                }
            }
            blk += 8;
            while (blk >= nb) { blk -= nb; ++rl; }
        }
    };
    if constexpr (!PIPE) {
        for (int it0 = 0; it0 < max(total, 1); it0 += 8 * IT) {
            Batch bt;
            load(bt, it0);
            if (it0 == 0)
                after_first_loads();
            compute(bt, it0);
        }
    } else {
        // double-buffered batches for long rows, as q4k_rows
        Batch ba, bb;
        load(ba, 0);
        after_first_loads();
        for (int it0 = 0; it0 < max(total, 1); it0 += 16 * IT) {
            const bool b_live = it0 + 8 * IT < total;
            if (b_live)
                load(bb, it0 + 8 * IT);
            compute(ba, it0);
            if (!b_live)
                break;
            if (it0 + 16 * IT < total)
                load(ba, it0 + 16 * IT);
            compute(bb, it0 + 8 * IT);
        }
    }
}

template <int MT, int R, int IT, bool ACT_LDS, bool PIPE = false>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_q5k_kernel(
    const uint8_t *__restrict__ W, const int8_t *__restrict__ q,
    const float *__restrict__ dx, const float *__restrict__ sx, int M, int N,
    int K, float *__restrict__ out)
{
    __shared__ v4i act[ACT_LDS ? GEMV_ACT_LDS / 16 : 1];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * GEMV_WAVES + wave) * R;
    ActCopy<> ac;
    if constexpr (ACT_LDS)
        act_load(ac, q, dx, sx, M, K);
    const int nb = K >> 8;
    const int rows = max(0, min(R, N - row0));
    // a wavefront past the last row reads (and discards) the last block
    const uint8_t *base = W + (int64_t)(rows > 0 ? row0 : N - 1) * nb * 176;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[r][m] = 0.0f;
    const int8_t *qa = q;
    const float *da = dx, *sa = sx;
    if constexpr (ACT_LDS) {
        qa = reinterpret_cast<const int8_t *>(act);
        da = reinterpret_cast<const float *>(qa + M * K);
        sa = da + M * (K >> 5);
    }
    q5k_rows<MT, R, IT, PIPE>(base, max(rows, 1), nb, K, M, qa, da, sa, lane, acc, [&] {
        if constexpr (ACT_LDS) {
            act_store(ac, act, M, K);
            __syncthreads();
        }
    });
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float v = wave_sum(acc[r][m]);
            if (lane == 0 && m < M && r < rows)
                out[(int64_t)m * N + row0 + r] = v;
        }
    }
}

// Persistent form of the Q5_K stream for short rows (K <= NP * 8 * 256),
// organised as the Q4_K one: wavefront w of NW walks rows w, w + NW, ...,
// each row NP passes of 8 blocks, the loads of the next D rows in flight
// while a row is reduced and stored; blocks past a row's end are clamped and
// masked, and nothing is loaded past the wavefront's last row.
template <int MT, int NP, int D>
#ifndef Q5S_WAVES
#define Q5S_WAVES GEMV_WAVES
#endif
__global__ __launch_bounds__(64 * Q5S_WAVES) void gemv_q5k_stream_kernel(
    const uint8_t *__restrict__ W, const int8_t *__restrict__ q,
    const float *__restrict__ dx, const float *__restrict__ sx, int M, int N,
    int K, float *__restrict__ out)
{
    constexpr int AB = stream_act_bytes(MT);
    __shared__ v4i act[AB / 16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = gridDim.x * Q5S_WAVES;
    const int w = blockIdx.x * Q5S_WAVES + wave;
    ActCopy<Q5S_WAVES, AB> ac;
    act_load(ac, q, dx, sx, M, K);

    const int nb = K >> 8;
    const int nb32 = K >> 5;
    const int64_t rowb = (int64_t)nb * 176;
    const int slot = lane >> 3;
    const int c = lane & 7;
    const int cc = c >> 1, po = (c & 1) << 4;
    const int j0 = 2 * cc;
    const int rot0 = (j0 + 28) & 31, rot1 = (j0 + 29) & 31;
    const int nrows = w < N ? (N - 1 - w) / nw + 1 : 0;

    bool valid[NP];
    int boff[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int blk = 8 * p + slot;
        valid[p] = blk < nb;
        boff[p] = min(blk, nb - 1) * 176;
    }
    struct Blk {
        v4i h, qh, qs;
    };
    auto load = [&](Blk &b, int n, int p) {
        const uint8_t *a = W + (int64_t)n * rowb + boff[p];
        b.h = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(a));
        b.qh = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(a + 16 + po));
        b.qs = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(a + 48 + 16 * c));
    };

    Blk ring[D][NP];
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
        for (int p = 0; p < NP; ++p)
            load(ring[d][p], min(w + d * nw, N - 1), p);
    act_store(ac, act, M, K);
    __syncthreads();
    const int8_t *qa = reinterpret_cast<const int8_t *>(act);
    const float *da = reinterpret_cast<const float *>(qa + M * K);
    const float *sa = da + M * nb32;

    for (int i0 = 0; i0 < nrows; i0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = i0 + d;
            if (i < nrows) {
                float acc[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    acc[m] = 0.0f;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    if (valid[p]) {
                        const Blk &b = ring[d][p];
                        const int blk = 8 * p + slot;
                        const uint32_t h0 = b.h.x, h1 = b.h.y, h2 = b.h.z, h3 = b.h.w;
                        const int k0 = (blk << 8) + (cc << 6) + po;
                        const int b0 = (blk << 3) + (cc << 1);
                        const float dd = f16_bits_to_f32(h0);
                        const float dm = f16_bits_to_f32(h0 >> 16);
                        const uint32_t scw = cc < 2 ? (h1 & 0x3f3f3f3fu)
                                                    : ((h3 & 0x0f0f0f0fu) | ((h1 >> 2) & 0x30303030u));
                        const uint32_t mw = cc < 2 ? (h2 & 0x3f3f3f3fu)
                                                   : (((h3 >> 4) & 0x0f0f0f0fu) | ((h2 >> 2) & 0x30303030u));
                        const int sh = (cc & 1) << 4;
                        const float f0 = dd * (float)((scw >> sh) & 0xffu);
                        const float f1 = dd * (float)((scw >> (sh + 8)) & 0xffu);
                        const float g0 = po == 0 ? dm * (float)((mw >> sh) & 0xffu) : 0.0f;
                        const float g1 = po == 0 ? dm * (float)((mw >> (sh + 8)) & 0xffu) : 0.0f;
                        int lo[4], hi[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t hb = (uint32_t)b.qh[e];
                            lo[e] = (b.qs[e] & 0x0f0f0f0f) | (int)(__builtin_rotateright32(hb, rot0) & 0x10101010u);
                            hi[e] = ((b.qs[e] >> 4) & 0x0f0f0f0f) | (int)(__builtin_rotateright32(hb, rot1) & 0x10101010u);
                        }
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            if (m < M) {
                                const v4i xa = *reinterpret_cast<const v4i *>(qa + m * K + k0);
                                const v4i xb = *reinterpret_cast<const v4i *>(qa + m * K + k0 + 32);
                                const float2 dp = *reinterpret_cast<const float2 *>(da + m * nb32 + b0);
                                const float2 sp = *reinterpret_cast<const float2 *>(sa + m * nb32 + b0);
                                int i0v = dot4(lo[0], xa.x, 0);
                                i0v = dot4(lo[1], xa.y, i0v);
                                i0v = dot4(lo[2], xa.z, i0v);
                                i0v = dot4(lo[3], xa.w, i0v);
                                int i1v = dot4(hi[0], xb.x, 0);
                                i1v = dot4(hi[1], xb.y, i1v);
                                i1v = dot4(hi[2], xb.z, i1v);
                                i1v = dot4(hi[3], xb.w, i1v);
                                float a = fmaf((float)i0v, dp.x * f0, acc[m]);
                                a = fmaf((float)i1v, dp.y * f1, a);
                                a = fmaf(-g0, sp.x, a);
                                acc[m] = fmaf(-g1, sp.y, a);
                            }
                        }
                    }
                }
                if (i + D < nrows) {
#pragma unroll
                    for (int p = 0; p < NP; ++p)
                        load(ring[d][p], w + (i + D) * nw, p);
                }
                const int n = w + i * nw;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const float v = wave_sum(acc[m]);
                    if (lane == 0 && m < M)
                        out[(int64_t)m * N + n] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- Q6_K
// Row slice owned by one lane: unit u = (blk, g, hh) = 64 weights
// w = 128g + 32r + 16hh + i (r = 0..3, i = 0..15) of block blk. It reads
// ql[64g + 16hh .. +16] (r = 0 low / r = 2 high nibbles),
// ql[64g + 32 + 16hh .. +16] (r = 1 / r = 3), qh[32g + 16hh .. +16]
// (bits 2r..2r+1), and the int8 scales 8g + 2r + hh.
template <int MT, int R>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_q6k_kernel(
    const uint8_t *__restrict__ W, const int8_t *__restrict__ q,
    const float *__restrict__ dx, int M, int N, int K, float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * GEMV_WAVES + wave) * R;
    if (row0 >= N)
        return;
    const int nsb = K >> 8;
    const int nun = nsb * 4;
    const int nb32 = K >> 5;
    const int64_t rowb = (int64_t)nsb * 210;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[r][m] = 0.0f;

    for (int u = lane; u < nun; u += 64) {
        const int blk = u >> 2;
        const int g = (u >> 1) & 1;
        const int hh = u & 1;
        const int kb = (blk << 8) + (g << 7) + (hh << 4);   // + 32r
        const int b0 = (blk << 3) + (g << 2);               // + r
        v4i x[MT][4];
        int xs[MT][4];
        float dr[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (m < M) {
                    x[m][r] = *reinterpret_cast<const v4i *>(q + (int64_t)m * K + kb + 32 * r);
                    dr[m][r] = dx[(int64_t)m * nb32 + b0 + r];
                } else {
                    x[m][r] = v4i{0, 0, 0, 0};
                    dr[m][r] = 0.0f;
                }
                int t = dot4(x[m][r].x, 0x01010101, 0);
                t = dot4(x[m][r].y, 0x01010101, t);
                t = dot4(x[m][r].z, 0x01010101, t);
                xs[m][r] = dot4(x[m][r].w, 0x01010101, t);   // sum of the 16 activations
            }
        }
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const int n = row0 + rr;
            if (n < N) {
                const uint8_t *bp = W + (int64_t)n * rowb + (int64_t)blk * 210;
                uint32_t l0[4], l1[4], h[4], sc[2];
                load_dwords_a2<4>(bp + 64 * g + 16 * hh, l0);
                load_dwords_a2<4>(bp + 64 * g + 32 + 16 * hh, l1);
                load_dwords_a2<4>(bp + 128 + 32 * g + 16 * hh, h);
                load_dwords_a2<2>(bp + 192 + 8 * g, sc);
                const float dd = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(bp + 208));
                // int8 scales for r = 0..3: bytes hh, 2+hh, 4+hh, 6+hh of sc[]
                const int s0 = (int)(int8_t)(sc[0] >> (8 * hh));
                const int s1 = (int)(int8_t)(sc[0] >> (16 + 8 * hh));
                const int s2 = (int)(int8_t)(sc[1] >> (8 * hh));
                const int s3 = (int)(int8_t)(sc[1] >> (16 + 8 * hh));
                int qr[4][4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qr[0][i] = (int)((l0[i] & 0x0f0f0f0fu) | ((h[i] << 4) & 0x30303030u));
                    qr[1][i] = (int)((l1[i] & 0x0f0f0f0fu) | ((h[i] << 2) & 0x30303030u));
                    qr[2][i] = (int)(((l0[i] >> 4) & 0x0f0f0f0fu) | (h[i] & 0x30303030u));
                    qr[3][i] = (int)(((l1[i] >> 4) & 0x0f0f0f0fu) | ((h[i] >> 2) & 0x30303030u));
                }
                const float ds0 = dd * (float)s0, ds1 = dd * (float)s1;
                const float ds2 = dd * (float)s2, ds3 = dd * (float)s3;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    int J[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        int t = dot4(qr[r][0], x[m][r].x, 0);
                        t = dot4(qr[r][1], x[m][r].y, t);
                        t = dot4(qr[r][2], x[m][r].z, t);
                        t = dot4(qr[r][3], x[m][r].w, t);
                        J[r] = t - 32 * xs[m][r];              // sum (q - 32) * x
                    }
                    float a = acc[rr][m];
                    a = fmaf((float)J[0], dr[m][0] * ds0, a);
                    a = fmaf((float)J[1], dr[m][1] * ds1, a);
                    a = fmaf((float)J[2], dr[m][2] * ds2, a);
                    a = fmaf((float)J[3], dr[m][3] * ds3, a);
                    acc[rr][m] = a;
                }
            }
        }
    }
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float v = wave_sum(acc[rr][m]);
            const int n = row0 + rr;
            if (lane == 0 && m < M && n < N)
                out[(int64_t)m * N + n] = v;
        }
    }
}

// ---------------------------------------------------------------- Q6_K stream
// The 210-byte Q6_K blocks are only 2-byte aligned, so instead of loading
// each lane's fields straight from memory, a wavefront copies its weight
// bytes into LDS with 16-byte global->LDS DMA (aligned chunks covering the
// byte range, 64 lanes x 16 bytes per instruction: fully coalesced) and the
// lanes decode from there, realigning dwords in registers. A wavefront owns
// the rows n = w, w + NW, w + 2 NW, ... (NW wavefronts in all) and walks
// them in segments of 16 blocks, one 64-weight unit per lane per segment;
// segments stream through a ring of Q6S_D LDS slots, Q6S_D - 1 ahead of the
// one being decoded. The activation plane (int8 values, per-32 scales and
// the sums of each 16-value group) is staged in LDS once per workgroup, so
// the only vector-memory loads in the loop are the DMAs and the waits on
// them are exact.
#ifndef Q6S_WAVES_CFG
#define Q6S_WAVES_CFG 4
#endif
#ifndef Q6S_D_CFG
#define Q6S_D_CFG 2
#endif
constexpr int Q6S_WAVES = Q6S_WAVES_CFG;      // wavefronts per workgroup
constexpr int Q6S_D = Q6S_D_CFG;              // ring slots per wavefront
constexpr int Q6S_SEG = 16;                   // blocks per segment
constexpr int Q6S_SLOT = 4096;                // bytes per slot (16*210 + alignment, whole DMA rows)
constexpr int Q6S_DMA = Q6S_SLOT / 1024;      // DMA instructions per segment
constexpr int Q6S_ACT_MAX = 48 * 1024;        // LDS budget of the activation plane (two tokens at K = 18944)
constexpr size_t Q6S_LDS_PER_CU = 160 * 1024;  // gfx950 LDS per compute unit
static_assert(Q6S_SEG * 210 + 16 <= Q6S_SLOT, "segment fits a slot");

// LDS bytes of the staged activation plane of M tokens: int8 values, f32
// per-32 scales, int16 per-16 sums.
__host__ __device__ constexpr int64_t q6s_act_bytes(int64_t M, int64_t K)
{
    return M * K + M * (K / 32) * 4 + M * (K / 16) * 2;
}

// n dwords at byte offset p (even) of an LDS buffer, realigned in registers.
template <int n>
__device__ __forceinline__ void lds_dwords_a2(const uint8_t *buf, int p, uint32_t (&out)[n])
{
    const uint32_t *b = reinterpret_cast<const uint32_t *>(buf + (p & ~3));
    const uint32_t sh = (uint32_t)(p & 3);
    uint32_t wv[n + 1];
#pragma unroll
    for (int i = 0; i <= n; ++i)
        wv[i] = b[i];
#pragma unroll
    for (int i = 0; i < n; ++i)
        out[i] = __builtin_amdgcn_alignbyte(wv[i + 1], wv[i], sh);
}

template <int MT>
__global__ __launch_bounds__(64 * Q6S_WAVES) void gemv_q6k_stream_kernel(
    const uint8_t *__restrict__ W, const int8_t *__restrict__ q,
    const float *__restrict__ dx, int M, int N, int K, float *__restrict__ out)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nb = K >> 8, nb32 = K >> 5, ng = K >> 4;
    int8_t *xq = reinterpret_cast<int8_t *>(smem);
    float *xd = reinterpret_cast<float *>(smem + M * K);
    int16_t *xs = reinterpret_cast<int16_t *>(smem + M * K + M * nb32 * 4);
    uint8_t *ring = smem + q6s_act_bytes(M, K) + wave * (Q6S_D * Q6S_SLOT);

    const int nw = gridDim.x * Q6S_WAVES;
    const int w = blockIdx.x * Q6S_WAVES + wave;
    const int nrows = w < N ? (N - 1 - w) / nw + 1 : 0;
    const int nseg = (nb + Q6S_SEG - 1) / Q6S_SEG;
    const int nitems = nrows * nseg;
    const int64_t rowb = (int64_t)nb * 210;

    // DMA of item it (row w + (it / nseg) * NW, segment it % nseg) into slot
    // it % Q6S_D. Items past the end reload the last one (same number of
    // DMAs per item keeps the waits exact); lanes past the segment's last
    // chunk reload that chunk into the slot's unused tail.
    auto issue = [&](int it) {
        const int ic = min(it, nitems - 1);
        const int ri = ic / nseg, seg = ic - ri * nseg;
        const uintptr_t ab = reinterpret_cast<uintptr_t>(W) + (uintptr_t)((int64_t)(w + ri * nw) * rowb +
                                                                          (int64_t)seg * (Q6S_SEG * 210));
        const int nbytes = min(Q6S_SEG, nb - seg * Q6S_SEG) * 210;
        const uintptr_t c0 = ab >> 4, c1 = (ab + nbytes - 1) >> 4;
        uint8_t *slot = ring + (it % Q6S_D) * Q6S_SLOT;
#pragma unroll
        for (int i = 0; i < Q6S_DMA; ++i)
            dma16(reinterpret_cast<const uint8_t *>(16 * min(c0 + 64 * i + lane, c1)), slot + 1024 * i);
    };

    // Activation plane -> LDS: all loads first (one memory latency), with the
    // ring's first segments already in flight, then the stores. Then the sums
    // of the 16-value groups, stored in the order the lanes read them: group
    // (blk, g, hh, r) at ((4 blk + 2 g + hh) * 4 + r).
    constexpr int ACT_C = (Q6S_ACT_MAX / 16 + 64 * Q6S_WAVES - 1) / (64 * Q6S_WAVES);
    const int qch = M * K / 16, dch = M * nb32 / 4;
    v4i av[ACT_C];
#pragma unroll
    for (int i = 0; i < ACT_C; ++i) {
        const int c = threadIdx.x + i * 64 * Q6S_WAVES;
        av[i] = c < qch ? reinterpret_cast<const v4i *>(q)[c]
                        : reinterpret_cast<const v4i *>(dx)[min(c - qch, dch - 1)];
    }
    if (nitems > 0) {
#pragma unroll
        for (int d = 0; d < Q6S_D - 1; ++d)
            issue(d);
    }
#pragma unroll
    for (int i = 0; i < ACT_C; ++i) {
        const int c = threadIdx.x + i * 64 * Q6S_WAVES;
        if (c < qch + dch)
            reinterpret_cast<v4i *>(smem)[c] = av[i];      // q, then d right after it
    }
    __syncthreads();
    for (int i = threadIdx.x; i < M * ng; i += 64 * Q6S_WAVES) {
        const int m = i / ng, gi = i - m * ng;
        const int r = gi & 3, hh = (gi >> 2) & 1, g = (gi >> 3) & 1, blk = gi >> 4;
        const v4i x = *reinterpret_cast<const v4i *>(xq + m * K + blk * 256 + 128 * g + 32 * r + 16 * hh);
        int t = dot4(x.x, 0x01010101, 0);
        t = dot4(x.y, 0x01010101, t);
        t = dot4(x.z, 0x01010101, t);
        xs[i] = (int16_t)dot4(x.w, 0x01010101, t);
    }
    __syncthreads();
    if (nitems == 0)
        return;

    const int bl = lane >> 2, g = (lane >> 1) & 1, hh = lane & 1;
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        acc[m] = 0.0f;
    for (int it = 0; it < nitems; ++it) {
        issue(it + Q6S_D - 1);
        wait_vm<Q6S_DMA * (Q6S_D - 1)>();
        const int ri = it / nseg, seg = it - ri * nseg;
        const int n = w + ri * nw;
        const int blk = seg * Q6S_SEG + bl;
        if (blk < nb) {
            const uint8_t *sl = ring + (it % Q6S_D) * Q6S_SLOT;
            const uintptr_t ab = reinterpret_cast<uintptr_t>(W) + (uintptr_t)((int64_t)n * rowb +
                                                                              (int64_t)seg * (Q6S_SEG * 210));
            const int p = (int)(ab & 15) + 210 * bl;    // this block in the slot
            uint32_t l0[4], l1[4], h[4], sc[2], dw[1];
            lds_dwords_a2<4>(sl, p + 64 * g + 16 * hh, l0);
            lds_dwords_a2<4>(sl, p + 64 * g + 32 + 16 * hh, l1);
            lds_dwords_a2<4>(sl, p + 128 + 32 * g + 16 * hh, h);
            lds_dwords_a2<2>(sl, p + 192 + 8 * g, sc);
            lds_dwords_a2<1>(sl, p + 208, dw);
            const float dd = f16_bits_to_f32(dw[0]);
            // int8 scales 8g + 2r + hh: bytes hh, 2 + hh, 4 + hh, 6 + hh of sc
            const float ds0 = dd * (float)(int)(int8_t)(sc[0] >> (8 * hh));
            const float ds1 = dd * (float)(int)(int8_t)(sc[0] >> (16 + 8 * hh));
            const float ds2 = dd * (float)(int)(int8_t)(sc[1] >> (8 * hh));
            const float ds3 = dd * (float)(int)(int8_t)(sc[1] >> (16 + 8 * hh));
            int qr[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qr[0][i] = (int)((l0[i] & 0x0f0f0f0fu) | ((h[i] << 4) & 0x30303030u));
                qr[1][i] = (int)((l1[i] & 0x0f0f0f0fu) | ((h[i] << 2) & 0x30303030u));
                qr[2][i] = (int)(((l0[i] >> 4) & 0x0f0f0f0fu) | (h[i] & 0x30303030u));
                qr[3][i] = (int)(((l1[i] >> 4) & 0x0f0f0f0fu) | ((h[i] >> 2) & 0x30303030u));
            }
            const int kb = (blk << 8) + (g << 7) + (hh << 4);   // + 32 r
            const int b0 = (blk << 3) + (g << 2);               // + r
            const int gs = ((blk << 2) + (g << 1) + hh) << 2;   // + r
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < M) {
                    const v4f dr = *reinterpret_cast<const v4f *>(xd + m * nb32 + b0);
                    const v2i s2 = *reinterpret_cast<const v2i *>(xs + m * ng + gs);
                    const int xsum[4] = {(int)(int16_t)s2.x, s2.x >> 16, (int)(int16_t)s2.y, s2.y >> 16};
                    const float dsr[4] = {ds0, ds1, ds2, ds3};
                    float a = acc[m];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const v4i x = *reinterpret_cast<const v4i *>(xq + m * K + kb + 32 * r);
                        int t = dot4(qr[r][0], x.x, 0);
                        t = dot4(qr[r][1], x.y, t);
                        t = dot4(qr[r][2], x.z, t);
                        t = dot4(qr[r][3], x.w, t);
                        const int J = t - 32 * xsum[r];           // sum (q - 32) * x
                        a = fmaf((float)J, dr[r] * dsr[r], a);
                    }
                    acc[m] = a;
                }
            }
        }
        if (seg == nseg - 1) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float v = wave_sum(acc[m]);
                if (lane == 0 && m < M)
                    out[(int64_t)m * N + n] = v;
                acc[m] = 0.0f;
            }
        }
    }
    // the ring's last DMAs target this workgroup's LDS: let them land first
    wait_vm<0>();
}

#ifndef GEMV_LONG_IT
#define GEMV_LONG_IT 4
#define GEMV_LONG_PIPE true
#endif
template <int MT, int R>
hipError_t gemv_q4k_launch(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           hipStream_t st)
{
    // passes (of 7 blocks) in flight: 8 in one batch for short rows; long
    // rows (one per wavefront) stream in double-buffered batches
    constexpr bool PIPE = R == 1 && GEMV_LONG_PIPE;
    constexpr int IT = R == 1 ? GEMV_LONG_IT : 8;
    const int rows_per_wg = GEMV_WAVES * R;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    const bool act_lds = (int64_t)M * K * 5 / 4 <= GEMV_ACT_LDS;
    if (act_lds)
        launch(gemv_q4k_kernel<MT, R, IT, true, PIPE>, dim3(grid), dim3(64 * GEMV_WAVES), 0, st, W, q, d, s, M, N, K, out);
    else
        launch(gemv_q4k_kernel<MT, R, IT, false, PIPE>, dim3(grid), dim3(64 * GEMV_WAVES), 0, st, W, q, d, s, M, N, K, out);
    return hipGetLastError();
}

// Rows per wavefront: several for short rows; one for long rows (K >= 8192),
// where a few rows per wavefront would leave too few wavefronts for the
// chip (N = 3584, K = 18944: 896 instead of 3584).
template <int MT>
hipError_t gemv_q4k_mt(const uint8_t *W, const int8_t *q, const float *d,
                       const float *s, int M, int N, int K, float *out,
                       hipStream_t st)
{
    if (K >= 8192)
        return gemv_q4k_launch<MT, 1>(W, q, d, s, M, N, K, out, st);
    return gemv_q4k_launch<MT, MT <= 2 ? 4 : 2>(W, q, d, s, M, N, K, out, st);
}

#ifndef GEMV_Q5K_IT
#define GEMV_Q5K_IT 4
#endif
#ifndef GEMV_Q5K_LONG_IT
#define GEMV_Q5K_LONG_IT 2
#endif
template <int MT, int R>
hipError_t gemv_q5k_launch(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           hipStream_t st)
{
    // passes (of 8 blocks) in flight; long rows stream in double-buffered batches
    constexpr bool PIPE = R == 1 && GEMV_LONG_PIPE;
    constexpr int IT = R == 1 ? GEMV_Q5K_LONG_IT : GEMV_Q5K_IT;
    const int rows_per_wg = GEMV_WAVES * R;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    const bool act_lds = (int64_t)M * K * 5 / 4 <= GEMV_ACT_LDS;
    if (act_lds)
        launch(gemv_q5k_kernel<MT, R, IT, true, PIPE>, dim3(grid), dim3(64 * GEMV_WAVES), 0, st, W, q, d, s, M, N, K, out);
    else
        launch(gemv_q5k_kernel<MT, R, IT, false, PIPE>, dim3(grid), dim3(64 * GEMV_WAVES), 0, st, W, q, d, s, M, N, K, out);
    return hipGetLastError();
}

template <int MT>
hipError_t gemv_q5k_mt(const uint8_t *W, const int8_t *q, const float *d,
                       const float *s, int M, int N, int K, float *out,
                       hipStream_t st)
{
    if (K >= 8192)                               // as for Q4_K
        return gemv_q5k_launch<MT, 1>(W, q, d, s, M, N, K, out, st);
    return gemv_q5k_launch<MT, MT <= 2 ? 4 : 2>(W, q, d, s, M, N, K, out, st);
}

template <int MT, int R>
hipError_t gemv_q6k_launch(const uint8_t *W, const int8_t *q, const float *d,
                           int M, int N, int K, float *out, hipStream_t st)
{
    const int rows_per_wg = GEMV_WAVES * R;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    launch(gemv_q6k_kernel<MT, R>, dim3(grid), dim3(64 * GEMV_WAVES), 0, st, W, q, d, M, N, K, out);
    return hipGetLastError();
}

template <int MT>
hipError_t gemv_q6k_mt(const uint8_t *W, const int8_t *q, const float *d,
                       int M, int N, int K, float *out, hipStream_t st)
{
    // long rows: one row per wavefront keeps enough wavefronts in flight
    if (K >= 8192)
        return gemv_q6k_launch<MT, 1>(W, q, d, M, N, K, out, st);
    return gemv_q6k_launch<MT, MT <= 2 ? 4 : 2>(W, q, d, M, N, K, out, st);
}

// Persistent Q4_K stream over N rows (N1 of them from W, the rest from W2;
// see gemv_q4k_stream_kernel): up to 1024 workgroups of 8 wavefronts (32 per
// CU), never more than one wavefront per row; a row is 2, 3 or 6 passes of 7
// blocks. The caller has checked q4k_stream_fits().
hipError_t q4k_stream(const uint8_t *W, const uint8_t *W2, int N1, const int8_t *q, const float *d,
                      const float *s, int M, int N, int K, float *out, float *out2, hipStream_t st)
{
    if (M == 1 && K <= 3 * 7 * 256) {
        // one token, short rows: activations in registers, 4 wavefronts per workgroup
        constexpr int WV = 4;
        const int nwg = max(1, min((N + WV - 1) / WV, GEMV_STREAM_WGS));
        if (K <= 2 * 7 * 256)
            launch(gemv_q4k_stream_kernel<1, 2, GEMV_STREAM_D, WV, true>, dim3(nwg), dim3(64 * WV), 0, st, W, W2,
                   N1, q, d, s, M, N, K, out, out2);
        else
            launch(gemv_q4k_stream_kernel<1, 3, GEMV_STREAM_D, WV, true>, dim3(nwg), dim3(64 * WV), 0, st, W, W2,
                   N1, q, d, s, M, N, K, out, out2);
        return hipGetLastError();
    }
    const int nwg = max(1, min((N + STREAM_WAVES - 1) / STREAM_WAVES, GEMV_STREAM_WGS));
    const dim3 grid(nwg), block(64 * STREAM_WAVES);
    auto go = [&](auto mt, auto np) {
        constexpr int MT = decltype(mt)::value, NP = decltype(np)::value;
        launch(gemv_q4k_stream_kernel<MT, NP, GEMV_STREAM_D>, grid, block, 0, st, W, W2, N1, q, d, s, M, N, K,
               out, out2);
    };
    auto np = [&](auto mt) {
        if (K <= 2 * 7 * 256) go(mt, std::integral_constant<int, 2>{});
        else if (K <= 3 * 7 * 256) go(mt, std::integral_constant<int, 3>{});
        else go(mt, std::integral_constant<int, 6>{});
    };
    if (M <= 1) np(std::integral_constant<int, 1>{});
    else if (M <= 2) np(std::integral_constant<int, 2>{});
    else if (M <= 4) np(std::integral_constant<int, 4>{});
    else np(std::integral_constant<int, 8>{});
    return hipGetLastError();
}

} // namespace

// The persistent streams take up to 8 tokens whose activation plane fits
// their LDS copy, with rows of up to 6 passes of 7 blocks (Q4_K) or 3 of 8
// (Q5_K).
bool q4k_stream_fits(int64_t M, int64_t K)
{
    if (M < 1 || M > 8 || K > GEMV_STREAM_NP_MAX * 7 * 256)
        return false;
    return M * K * 5 / 4 <= stream_act_bytes(M <= 4 ? 4 : 8);
}

bool q6k_stream_fits(int64_t M, int64_t K)
{
    return M >= 1 && M <= 16 && K >= 256 && q6s_act_bytes(M, K) <= Q6S_ACT_MAX &&
           q6s_act_bytes(M, K) + (int64_t)Q6S_WAVES * Q6S_D * Q6S_SLOT <= (int64_t)Q6S_LDS_PER_CU;
}

bool q5k_stream_fits(int64_t M, int64_t K)
{
    if (M < 1 || M > 8 || K > 3 * 8 * 256)
        return false;
    return M * K * 5 / 4 <= stream_act_bytes(M <= 4 ? 4 : 8);
}

hipError_t launch_gemv_q4k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           hipStream_t st)
{
    // rows of up to 6 passes with the plane in LDS: the persistent stream
    // (measured against the row-grid kernel: 13.2 -> 8.3 us at 14336 x 4096,
    // 12.7 -> 11.3 us at 8192 x 8192; longer rows keep the row-grid kernel)
    if (q4k_stream_fits(M, K))
        return q4k_stream(W, W, N, q, d, s, M, N, K, out, out, st);
    if (M <= 1) return gemv_q4k_mt<1>(W, q, d, s, M, N, K, out, st);
    if (M <= 2) return gemv_q4k_mt<2>(W, q, d, s, M, N, K, out, st);
    if (M <= 4) return gemv_q4k_mt<4>(W, q, d, s, M, N, K, out, st);
    if (M <= 8) return gemv_q4k_mt<8>(W, q, d, s, M, N, K, out, st);
    return gemv_q4k_mt<16>(W, q, d, s, M, N, K, out, st);
}

hipError_t launch_gemv_q4k_pair(const uint8_t *Wg, const uint8_t *Wu, const int8_t *q, const float *d,
                                const float *s, int M, int N, int K, float *g, float *u, hipStream_t st)
{
    if (!q4k_stream_fits(M, K) || (int64_t)2 * N > 0x7fffffff)
        return hipErrorInvalidValue;
    return q4k_stream(Wg, Wu, N, q, d, s, M, 2 * N, K, g, u, st);
}

hipError_t launch_gemv_q5k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           hipStream_t st)
{
    // persistent stream up to 3 passes of 8 blocks (at 4 passes and more the
    // row-grid kernel measured faster for Q5_K) and 8 tokens whose plane fits
    // the LDS copy
    if (q5k_stream_fits(M, K)) {
        const int nwg = max(1, min((N + Q5S_WAVES - 1) / Q5S_WAVES, GEMV_STREAM_WGS));
        const dim3 grid(nwg), block(64 * Q5S_WAVES);
        auto go = [&](auto mt) {
            constexpr int MT = decltype(mt)::value;
            if (K <= 2 * 8 * 256)
                launch(gemv_q5k_stream_kernel<MT, 2, GEMV_STREAM_D>, grid, block, 0, st, W, q, d, s, M, N, K, out);
            else
                launch(gemv_q5k_stream_kernel<MT, 3, GEMV_STREAM_D>, grid, block, 0, st, W, q, d, s, M, N, K, out);
        };
        if (M <= 1) go(std::integral_constant<int, 1>{});
        else if (M <= 2) go(std::integral_constant<int, 2>{});
        else if (M <= 4) go(std::integral_constant<int, 4>{});
        else go(std::integral_constant<int, 8>{});
        return hipGetLastError();
    }
    if (M <= 1) return gemv_q5k_mt<1>(W, q, d, s, M, N, K, out, st);
    if (M <= 2) return gemv_q5k_mt<2>(W, q, d, s, M, N, K, out, st);
    if (M <= 4) return gemv_q5k_mt<4>(W, q, d, s, M, N, K, out, st);
    if (M <= 8) return gemv_q5k_mt<8>(W, q, d, s, M, N, K, out, st);
    return gemv_q5k_mt<16>(W, q, d, s, M, N, K, out, st);
}

// The GEMMs of the two-pass FFN: the configuration of the token count.
static int ffn_gemm_splits(int M, int N, int K)
{
    return M <= GEMM_SMALL_M_Q4K ? splits_gemm_q4k_small(M, N, K) : splits_gemm_q4k(M, N, K);
}

size_t ffn_two_pass_bytes(int M, int N, int K, bool gemv)
{
    const size_t gu = (size_t)2 * M * N * sizeof(float);
    return gemv ? gu : gu + split_bytes(ffn_gemm_splits(M, N, K), M, N);
}

hipError_t launch_ffn_q4k_two_pass(const uint8_t *Wg, const uint8_t *Wu, const int8_t *q, const float *d,
                                   const float *s, int M, int N, int K, int8_t *qo, float *do_, float *so,
                                   float *y, bool gemv, const Ws &ws, hipStream_t st)
{
    // Where the persistent stream takes the plane, both matrices run as one
    // stream of 2N rows. (A single GEMV kernel with the SwiGLU in its
    // epilogue, each workgroup owning one 32-value block of y, measured
    // slower than these launches at every M <= 8 on 18944 x 3584: its N / 32
    // equal work units leave a tail, and each wavefront streams its rows
    // without the persistent kernel's pipelining.)
    // Workspace: g [M][N], u [M][N], then the GEMMs' split-K planes (the two
    // GEMMs run one after the other on st and reuse them).
    if (!ws.ptr || ws.bytes < ffn_two_pass_bytes(M, N, K, gemv))
        return hipErrorInvalidValue;
    float *g = static_cast<float *>(ws.ptr), *u = g + (int64_t)M * N;
    const size_t gu = (size_t)2 * M * N * sizeof(float);
    const Ws split{static_cast<uint8_t *>(ws.ptr) + gu, ws.bytes - gu};
    hipError_t e;
    if (gemv && q4k_stream_fits(M, K)) {
        e = launch_gemv_q4k_pair(Wg, Wu, q, d, s, M, N, K, g, u, st);
    } else {
        auto mm = [&](const uint8_t *W, float *o) {
            if (gemv)
                return launch_gemv_q4k(W, q, d, s, M, N, K, o, st);
            if (M <= GEMM_SMALL_M_Q4K)
                return launch_gemm_q4k_small(W, q, d, s, M, N, K, o, split, st);
            return launch_gemm_q4k(W, q, d, s, M, N, K, o, split, st);
        };
        e = mm(Wg, g);
        if (e == hipSuccess)
            e = mm(Wu, u);
    }
    if (e == hipSuccess)
        e = launch_swiglu_quantize(g, u, M, N, N, N, qo, do_, so, y, st);
    return e;
}

hipError_t launch_gemv_q6k(const uint8_t *W, const int8_t *q, const float *d,
                           int M, int N, int K, float *out, hipStream_t st)
{
    if (q6k_stream_fits(M, K)) {
        // as many workgroups as fit on the chip at once (LDS-limited)
        const int n_cu = device_cu_count();
        const size_t lds = (size_t)q6s_act_bytes(M, K) + (size_t)Q6S_WAVES * Q6S_D * Q6S_SLOT;
        const int per_cu = max(1, (int)(Q6S_LDS_PER_CU / lds));
        const int nwg = max(1, min((N + Q6S_WAVES - 1) / Q6S_WAVES, per_cu * n_cu));
        dim3 grid(nwg), block(64 * Q6S_WAVES);
        if (M <= 1) launch(gemv_q6k_stream_kernel<1>, grid, block, lds, st, W, q, d, M, N, K, out);
        else if (M <= 2) launch(gemv_q6k_stream_kernel<2>, grid, block, lds, st, W, q, d, M, N, K, out);
        else if (M <= 4) launch(gemv_q6k_stream_kernel<4>, grid, block, lds, st, W, q, d, M, N, K, out);
        else if (M <= 8) launch(gemv_q6k_stream_kernel<8>, grid, block, lds, st, W, q, d, M, N, K, out);
        else launch(gemv_q6k_stream_kernel<16>, grid, block, lds, st, W, q, d, M, N, K, out);
        return hipGetLastError();
    }
    if (M <= 1) return gemv_q6k_mt<1>(W, q, d, M, N, K, out, st);
    if (M <= 2) return gemv_q6k_mt<2>(W, q, d, M, N, K, out, st);
    if (M <= 4) return gemv_q6k_mt<4>(W, q, d, M, N, K, out, st);
    if (M <= 8) return gemv_q6k_mt<8>(W, q, d, M, N, K, out, st);
    return gemv_q6k_mt<16>(W, q, d, M, N, K, out, st);
}

} // namespace mq
