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
// The Q6_K expansion also runs once per prefill call at large M (the
// matmul's expansion plan), so it stages its bytes with coalesced dword
// loads; the Q4_K decode runs once per registration, one thread per block.
#include "mq_device.h"
#include "mq_launch.h"

namespace mq {
namespace {

// Wavefront g of the grid expands the XG = 16 Q6_K blocks XG*g ..
// XG*g + XG - 1 (fewer in the last group). A group's 3360 bytes
// (XG * 210, a multiple of 16) start 16-byte aligned when W is, and then the
// wavefront stages them in LDS with 16-byte loads (dword loads when W is
// only 4-byte aligned). Measured on MI355X for 3584 x 18944: one block per
// wavefront 54-69 us (too few bytes in flight), 8 blocks 49 us, 16 blocks
// 41.7 us (4.6 TB/s of reads and writes), 32 blocks 47 us.
// Lane l then owns weights 4l .. 4l + 3 (one 16-value group) of each block,
// read back from LDS as dwords realigned with v_alignbyte (odd blocks start
// 2 bytes into a dword). The last group, when short, is staged as its whole
// dwords plus, for an odd block count, the last block's 2-byte d, so no
// byte past W is read. LDS operations of one wavefront complete in order,
// so its lanes see each other's stores without a barrier.
constexpr int XG = 16;                           // blocks per wavefront
constexpr int XG_WORDS = XG * 210 / 4;           // 840 dwords
__global__ __launch_bounds__(256) void expand_q6k_kernel(const uint8_t *__restrict__ W, int64_t nblk,
                                                         int nsb, int K, int8_t *__restrict__ lo,
                                                         int8_t *__restrict__ hi, float *__restrict__ dw)
{
    __shared__ __align__(16) uint32_t stage[4][XG_WORDS + 4];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t b0 = ((int64_t)blockIdx.x * 4 + wv) * XG;
    if (b0 >= nblk)
        return;
    const int nb = (int)min<int64_t>(XG, nblk - b0);
    const uint8_t *src = W + b0 * 210;
    uint32_t *st = stage[wv];
    if (nb == XG && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
        const uint4 *s16 = reinterpret_cast<const uint4 *>(src);
        constexpr int NC = XG_WORDS / 4;         // 16-byte chunks of the group
        constexpr int NL = (NC + 63) / 64;       // loads per lane
        uint4 v[NL];
#pragma unroll
        for (int u = 0; u < NL; ++u)
            if (u * 64 + lane < NC)
                v[u] = s16[u * 64 + lane];
#pragma unroll
        for (int u = 0; u < NL; ++u)
            if (u * 64 + lane < NC)
                reinterpret_cast<uint4 *>(st)[u * 64 + lane] = v[u];
    } else {
        const int nwords = nb * 210 / 4;         // whole dwords of the group
        for (int j = lane; j < nwords; j += 64)
            st[j] = reinterpret_cast<const uint32_t *>(src)[j];
        if ((nb & 1) && lane == 0)
            st[nwords] = *reinterpret_cast<const uint16_t *>(src + 4 * nwords);
    }
    __builtin_amdgcn_wave_barrier();
    // the 4 bytes at byte offset x of the group
    auto rd32 = [&](int x) {
        const uint32_t a = st[x >> 2], b = st[(x >> 2) + 1];
        return __builtin_amdgcn_alignbyte(b, a, (uint32_t)(x & 3));
    };
    const int w = 4 * lane;
    const int g = w >> 7, r = (w >> 5) & 3, i = w & 31;
    for (int e = 0; e < nb; ++e) {
        const int base = 210 * e;
        const uint32_t ql = rd32(base + 64 * g + 32 * (r & 1) + i) >> (4 * (r >> 1));
        const uint32_t qh = rd32(base + 128 + 32 * g + i) >> (2 * r);
        const int sc = (int)(int8_t)(rd32(base + 192 + (lane >> 2)) & 0xffu);
        uint32_t plo = 0, phi = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int q = (int)((ql >> (8 * k)) & 15u) | (int)(((qh >> (8 * k)) & 3u) << 4);
            const int pv = sc * (q - 32);
            const int h = pv >> 6;             // arithmetic shift: floor(pv / 64)
            plo |= (uint32_t)(pv - 64 * h) << (8 * k);
            phi |= (uint32_t)(h & 0xff) << (8 * k);
        }
        const int64_t b = b0 + e;
        const int64_t n = b / nsb, sb = b - n * nsb;
        const int64_t k0 = n * K + sb * 256 + w;
        *reinterpret_cast<uint32_t *>(lo + k0) = plo;
        *reinterpret_cast<uint32_t *>(hi + k0) = phi;
        if (lane == 0)
            dw[b] = f16_bits_to_f32(rd32(base + 208) & 0xffffu);
    }
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
    const int64_t ngroup = (nblk + XG - 1) / XG;
    expand_q6k_kernel<<<dim3((unsigned)((ngroup + 3) / 4)), dim3(256), 0, st>>>(W, nblk, (int)(K >> 8), (int)K,
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
