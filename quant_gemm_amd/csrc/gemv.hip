// Decode GEMV for Q4_K / Q6_K weights x per-32 int8 activations (gfx950).
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

namespace mq {
namespace {

constexpr int GEMV_WAVES = 4;   // wavefronts per workgroup

// ---------------------------------------------------------------- Q4_K
// Row slice owned by one lane: one 16-byte chunk c (0..7) of a block's 128
// quant bytes. Chunk c covers positions po..po+15 (po = 16*(c&1)) of the
// sub-blocks j0 = 2*(c>>1) (low nibbles) and j0+1 (high nibbles).
template <int MT, int R>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_q4k_kernel(
    const uint8_t *__restrict__ W, const int8_t *__restrict__ q,
    const float *__restrict__ dx, const float *__restrict__ sx, int M, int N,
    int K, float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * GEMV_WAVES + wave) * R;
    if (row0 >= N)
        return;
    const int nsb = K >> 8;
    const int nch = nsb * 8;
    const int nb32 = K >> 5;
    const int64_t rowb = (int64_t)nsb * 144;

    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[r][m] = 0.0f;

    for (int ch = lane; ch < nch; ch += 64) {
        const int blk = ch >> 3;
        const int c = ch & 7;
        const int cc = c >> 1;
        const int po = (c & 1) << 4;
        const int k0 = (blk << 8) + (cc << 6) + po;     // sub-block j0, positions po..
        const int b0 = (blk << 3) + (cc << 1);          // its 32-block index
        // activation slices (shared by all R rows)
        v4i xa[MT], xb[MT];
        float da[MT], db[MT], sa[MT], sb[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {
                xa[m] = *reinterpret_cast<const v4i *>(q + (int64_t)m * K + k0);
                xb[m] = *reinterpret_cast<const v4i *>(q + (int64_t)m * K + k0 + 32);
                da[m] = dx[(int64_t)m * nb32 + b0];
                db[m] = dx[(int64_t)m * nb32 + b0 + 1];
                sa[m] = sx[(int64_t)m * nb32 + b0];
                sb[m] = sx[(int64_t)m * nb32 + b0 + 1];
            } else {
                xa[m] = xb[m] = v4i{0, 0, 0, 0};
                da[m] = db[m] = sa[m] = sb[m] = 0.0f;
            }
        }
        const float minw = po == 0 ? 1.0f : 0.0f;   // one of the two lanes adds the min term
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = row0 + r;
            if (n < N) {
                const uint8_t *bp = W + (int64_t)n * rowb + (int64_t)blk * 144;
                const uint4 hdr = *reinterpret_cast<const uint4 *>(bp);
                const uint4 qw = *reinterpret_cast<const uint4 *>(bp + 16 + 16 * c);
                const float dd = f16_bits_to_f32(hdr.x);
                const float dm = f16_bits_to_f32(hdr.x >> 16);
                // 6-bit codes: bytes 0..3 of sc_lo/m_lo are j = 0..3, of
                // sc_hi/m_hi j = 4..7.
                const uint32_t sc_lo = hdr.y & 0x3f3f3f3fu;
                const uint32_t m_lo = hdr.z & 0x3f3f3f3fu;
                const uint32_t sc_hi = (hdr.w & 0x0f0f0f0fu) | ((hdr.y >> 2) & 0x30303030u);
                const uint32_t m_hi = ((hdr.w >> 4) & 0x0f0f0f0fu) | ((hdr.z >> 2) & 0x30303030u);
                const uint32_t scw = cc < 2 ? sc_lo : sc_hi;
                const uint32_t mw = cc < 2 ? m_lo : m_hi;
                const int sh = (cc & 1) << 4;               // byte 2*(cc&1)
                const float f0 = dd * (float)((scw >> sh) & 0xffu);
                const float f1 = dd * (float)((scw >> (sh + 8)) & 0xffu);
                const float g0 = dm * (float)((mw >> sh) & 0xffu);
                const float g1 = dm * (float)((mw >> (sh + 8)) & 0xffu);
                const int lo0 = qw.x & 0x0f0f0f0f, lo1 = qw.y & 0x0f0f0f0f;
                const int lo2 = qw.z & 0x0f0f0f0f, lo3 = qw.w & 0x0f0f0f0f;
                const int hi0 = (qw.x >> 4) & 0x0f0f0f0f, hi1 = (qw.y >> 4) & 0x0f0f0f0f;
                const int hi2 = (qw.z >> 4) & 0x0f0f0f0f, hi3 = (qw.w >> 4) & 0x0f0f0f0f;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    int i0 = dot4(lo0, xa[m].x, 0);
                    i0 = dot4(lo1, xa[m].y, i0);
                    i0 = dot4(lo2, xa[m].z, i0);
                    i0 = dot4(lo3, xa[m].w, i0);
                    int i1 = dot4(hi0, xb[m].x, 0);
                    i1 = dot4(hi1, xb[m].y, i1);
                    i1 = dot4(hi2, xb[m].z, i1);
                    i1 = dot4(hi3, xb[m].w, i1);
                    float a = acc[r][m];
                    a = fmaf((float)i0, da[m] * f0, a);
                    a = fmaf((float)i1, db[m] * f1, a);
                    a = fmaf(-minw * g0, sa[m], a);
                    a = fmaf(-minw * g1, sb[m], a);
                    acc[r][m] = a;
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const float v = wave_sum(acc[r][m]);
            const int n = row0 + r;
            if (lane == 0 && m < M && n < N)
                out[(int64_t)m * N + n] = v;
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

template <int MT>
hipError_t gemv_q4k_mt(const uint8_t *W, const int8_t *q, const float *d,
                       const float *s, int M, int N, int K, float *out,
                       hipStream_t st)
{
    constexpr int R = MT <= 2 ? 4 : 2;
    const int rows_per_wg = GEMV_WAVES * R;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    gemv_q4k_kernel<MT, R><<<dim3(grid), dim3(64 * GEMV_WAVES), 0, st>>>(W, q, d, s, M, N, K, out);
    return hipGetLastError();
}

template <int MT>
hipError_t gemv_q6k_mt(const uint8_t *W, const int8_t *q, const float *d,
                       int M, int N, int K, float *out, hipStream_t st)
{
    constexpr int R = MT <= 2 ? 4 : 2;
    const int rows_per_wg = GEMV_WAVES * R;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    gemv_q6k_kernel<MT, R><<<dim3(grid), dim3(64 * GEMV_WAVES), 0, st>>>(W, q, d, M, N, K, out);
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemv_q4k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           hipStream_t st)
{
    if (M <= 1) return gemv_q4k_mt<1>(W, q, d, s, M, N, K, out, st);
    if (M <= 2) return gemv_q4k_mt<2>(W, q, d, s, M, N, K, out, st);
    if (M <= 4) return gemv_q4k_mt<4>(W, q, d, s, M, N, K, out, st);
    return gemv_q4k_mt<8>(W, q, d, s, M, N, K, out, st);
}

hipError_t launch_gemv_q6k(const uint8_t *W, const int8_t *q, const float *d,
                           int M, int N, int K, float *out, hipStream_t st)
{
    if (M <= 1) return gemv_q6k_mt<1>(W, q, d, M, N, K, out, st);
    if (M <= 2) return gemv_q6k_mt<2>(W, q, d, M, N, K, out, st);
    if (M <= 4) return gemv_q6k_mt<4>(W, q, d, M, N, K, out, st);
    return gemv_q6k_mt<8>(W, q, d, M, N, K, out, st);
}

} // namespace mq
