// Registration-time weight planes for the prefill GEMMs (gfx950).
//
// The pages add two kinds of planes when weights are registered: an
// expansion of the q6_K weights and a decoded-scale plane for q4_K, both
// read by the MMQ GEMM instead of decoding the raw blocks on every tile
// (minfer Features, "GPU — CUDA": the W_exp / W_dsc planes and their memory
// cost). Contents, as declared in mq.h:
//   Q6_K: p = sc_g * (q - 32) per weight (g its 16-value group), as the int8
//         limbs lo = p mod 64 (0..63) and hi = floor(p / 64) (-64..64), planes
//         [N][K]; d per super-block as f32, plane [N][K/256];
//   Q4_K: d * sc_j and dmin * m_j per 32-value sub-block as f32 (exact),
//         planes [N][K/32].
// Both run once per weight matrix, so they are written for clarity: one
// wavefront per Q6_K block, one thread per Q4_K block.
#include "mq_device.h"
#include "mq_launch.h"

namespace mq {
namespace {

// Wavefront b of the grid expands Q6_K block b (row b / nsb); lane l owns
// weights 4l .. 4l + 3 (one 16-value group).
__global__ __launch_bounds__(256) void expand_q6k_kernel(const uint8_t *__restrict__ W, int64_t nblk,
                                                         int nsb, int K, int8_t *__restrict__ lo,
                                                         int8_t *__restrict__ hi, float *__restrict__ dw)
{
    const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= nblk)
        return;
    const int lane = threadIdx.x & 63;
    const uint8_t *blk = W + b * 210;
    const int64_t n = b / nsb, sb = b - n * nsb;
    const int sc = (int)(int8_t)blk[192 + (lane >> 2)];
    uint32_t plo = 0, phi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int w = 4 * lane + e;
        const int g = w >> 7, r = (w >> 5) & 3, i = w & 31;
        const int low4 = (blk[64 * g + 32 * (r & 1) + i] >> (4 * (r >> 1))) & 15;
        const int high2 = (blk[128 + 32 * g + i] >> (2 * r)) & 3;
        const int p = sc * ((low4 | (high2 << 4)) - 32);
        const int h = p >> 6;                  // arithmetic shift: floor(p / 64)
        plo |= (uint32_t)(p - 64 * h) << (8 * e);
        phi |= (uint32_t)(h & 0xff) << (8 * e);
    }
    const int64_t k = n * K + sb * 256 + 4 * lane;
    *reinterpret_cast<uint32_t *>(lo + k) = plo;
    *reinterpret_cast<uint32_t *>(hi + k) = phi;
    if (lane == 0)
        dw[b] = f16_bits_to_f32((uint32_t)blk[208] | ((uint32_t)blk[209] << 8));
}

// Thread b decodes the header of Q4_K block b: eight 6-bit scale codes and
// eight min codes (codes 4..7 take their high bits from the top of bytes
// 0..7), each times the block's f16 d or dmin.
__global__ __launch_bounds__(256) void dsc_q4k_kernel(const uint8_t *__restrict__ W, int64_t nblk,
                                                      float *__restrict__ fw, float *__restrict__ fm)
{
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk)
        return;
    const uint4 h = *reinterpret_cast<const uint4 *>(W + b * 144);
    const float dd = f16_bits_to_f32(h.x);
    const float dm = f16_bits_to_f32(h.x >> 16);
    float s[8], m[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s[j] = dd * (float)((h.y >> (8 * j)) & 63u);
        m[j] = dm * (float)((h.z >> (8 * j)) & 63u);
        s[j + 4] = dd * (float)(((h.w >> (8 * j)) & 15u) | (((h.y >> (8 * j + 6)) & 3u) << 4));
        m[j + 4] = dm * (float)(((h.w >> (8 * j + 4)) & 15u) | (((h.z >> (8 * j + 6)) & 3u) << 4));
    }
    float4 *pw = reinterpret_cast<float4 *>(fw + b * 8);
    float4 *pm = reinterpret_cast<float4 *>(fm + b * 8);
    pw[0] = make_float4(s[0], s[1], s[2], s[3]);
    pw[1] = make_float4(s[4], s[5], s[6], s[7]);
    pm[0] = make_float4(m[0], m[1], m[2], m[3]);
    pm[1] = make_float4(m[4], m[5], m[6], m[7]);
}

} // namespace

hipError_t launch_expand_q6k(const uint8_t *W, int64_t N, int64_t K, int8_t *lo, int8_t *hi, float *dw,
                             hipStream_t st)
{
    const int64_t nblk = N * (K >> 8);
    expand_q6k_kernel<<<dim3((unsigned)((nblk + 3) / 4)), dim3(256), 0, st>>>(W, nblk, (int)(K >> 8), (int)K,
                                                                              lo, hi, dw);
    return hipGetLastError();
}

hipError_t launch_dsc_q4k(const uint8_t *W, int64_t N, int64_t K, float *fw, float *fm, hipStream_t st)
{
    const int64_t nblk = N * (K >> 8);
    dsc_q4k_kernel<<<dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, st>>>(W, nblk, fw, fm);
    return hipGetLastError();
}

} // namespace mq
