// Prefill GEMM for Q6_K weights x per-32 int8 activations (gfx950).
//
// The pages' prefill runs an int8 tensor-core GEMM directly on the raw
// 4-/6-bit quants against the int8 activation plane, with the block scales
// applied after each integer product (minfer Features, "GPU — CUDA": raw-
// nibble int8 GEMMs for q4_K and q6_K). This is a CDNA4 design of that:
//
//   * a 256-thread workgroup computes a 128-token x 128-row output tile as
//     2 x 2 wavefronts of 64 x 64, each 2 x 2 MFMA tiles of 32 x 32;
//   * the K loop moves in half super-blocks (128 values). Each step stages
//     the int8 activations, their per-32 scales and sums, and the weight
//     quants unpacked to int8 (4-bit nibbles, or 6-bit values minus 32) in
//     natural K order into LDS, together with the f32 per-group weight
//     factors (d*sc, dmin*m for Q4_K; d*sc for Q6_K);
//   * the integer dot of every scale group is one int8 MFMA, exact in int32:
//     v_mfma_i32_32x32x32_i8 per 32-value Q4_K sub-block,
//     v_mfma_i32_32x32x16_i8 per 16-value Q6_K group;
//   * the f32 epilogue applies the activation scale times the weight factor
//     (and the Q4_K min term, which uses the activation sums) per group.
//
// MFMA operand layout (32x32xK): lane l supplies row (l % 32) of A and
// column (l % 32) of B, each with K/2 consecutive values starting at
// K/2 * (l / 32); since both operands split K the same way, the products pair
// up whatever order the hardware uses inside a lane. The 32x32 result gives
// lane l column (l % 32) and rows 8*(v/4) + 4*(l/32) + (v%4), v = 0..15.
// Here A = activations (rows = tokens), B = weights (columns = output rows).
#include "mq_device.h"
#include "mq_launch.h"

namespace mq {
namespace {

constexpr int BM = 128;        // tokens per tile
constexpr int BN = 128;        // weight rows per tile
constexpr int BK = 128;        // K values per step (half a super-block)
constexpr int LDA = BK + 16;   // padded LDS row (bytes) against bank conflicts
constexpr int NTHR = 256;

template <bool Q6>
struct Smem {
    int8_t a[BM][LDA];               // activations, int8
    int8_t b[BN][LDA];               // weights, int8 (natural K order)
    float dx[BK / 32][BM];           // activation scale per 32-block
    float sx[BK / 32][BM];           // activation sum (Q4_K only)
    float fw[Q6 ? BK / 16 : BK / 32][BN];   // d*sc per weight scale group
    float fm[BK / 32][BN];           // dmin*m per sub-block (Q4_K only)
};

__device__ __forceinline__ void zero16(int8_t *p)
{
    *reinterpret_cast<v4i *>(p) = v4i{0, 0, 0, 0};
}

// Stage the activation plane slice [t0, t0+BM) x [k0, k0+BK).
template <bool Q6>
__device__ __forceinline__ void stage_act(Smem<Q6> &sm, const int8_t *__restrict__ q,
                                          const float *__restrict__ dx,
                                          const float *__restrict__ sx, int M, int K,
                                          int t0, int k0)
{
    const int tid = threadIdx.x;
    const int nb32 = K >> 5;
#pragma unroll
    for (int i = 0; i < (BM * BK / 16) / NTHR; ++i) {
        const int c = tid + i * NTHR;
        const int row = c >> 3;
        const int col = (c & 7) << 4;
        const int t = t0 + row;
        if (t < M)
            *reinterpret_cast<v4i *>(&sm.a[row][col]) =
                *reinterpret_cast<const v4i *>(q + (int64_t)t * K + k0 + col);
        else
            zero16(&sm.a[row][col]);
    }
    // scales (threads 0..127) and sums (threads 128..255): 4 floats per token
    {
        const int row = tid & (BM - 1);
        const int t = t0 + row;
        const bool sums = tid >= BM;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < M && (!Q6 || !sums))
            v = *reinterpret_cast<const float4 *>((sums ? sx : dx) + (int64_t)t * nb32 + (k0 >> 5));
        float(*dst)[BM] = sums ? sm.sx : sm.dx;
        dst[0][row] = v.x;
        dst[1][row] = v.y;
        dst[2][row] = v.z;
        dst[3][row] = v.w;
    }
}

// Stage Q4_K weights for rows [n0, n0+BN), half hf of super-block sb.
__device__ __forceinline__ void stage_w_q4k(Smem<false> &sm, const uint8_t *__restrict__ W,
                                            int N, int K, int n0, int sb, int hf)
{
    const int tid = threadIdx.x;
    const int64_t rowb = (int64_t)(K >> 8) * 144;
    // quants: per row 64 bytes = 4 chunks of 16 (sub-blocks 4hf..4hf+3)
#pragma unroll
    for (int i = 0; i < (BN * 4) / NTHR; ++i) {
        const int c = tid + i * NTHR;
        const int row = c >> 2;
        const int part = c & 3;
        const int cl = part >> 1;                 // chunk pair within the half
        const int po = (part & 1) << 4;
        const int n = n0 + row;
        int8_t *lo = &sm.b[row][64 * cl + po];    // sub-block 2cl (local), low nibbles
        int8_t *hi = lo + 32;                     // sub-block 2cl+1, high nibbles
        if (n < N) {
            const uint8_t *bp = W + (int64_t)n * rowb + (int64_t)sb * 144;
            const v4i w = *reinterpret_cast<const v4i *>(bp + 16 + 64 * hf + 32 * cl + po);
            *reinterpret_cast<v4i *>(lo) = w & 0x0f0f0f0f;
            *reinterpret_cast<v4i *>(hi) = (w >> 4) & 0x0f0f0f0f;
        } else {
            zero16(lo);
            zero16(hi);
        }
    }
    // block header: d, dmin and the four scale/min codes of this half
    if (tid < BN) {
        const int n = n0 + tid;
        float f[4] = {0.f, 0.f, 0.f, 0.f}, g[4] = {0.f, 0.f, 0.f, 0.f};
        if (n < N) {
            const uint4 hdr = *reinterpret_cast<const uint4 *>(W + (int64_t)n * rowb + (int64_t)sb * 144);
            const float dd = f16_bits_to_f32(hdr.x);
            const float dm = f16_bits_to_f32(hdr.x >> 16);
            const uint32_t scw = hf == 0 ? (hdr.y & 0x3f3f3f3fu)
                                         : ((hdr.w & 0x0f0f0f0fu) | ((hdr.y >> 2) & 0x30303030u));
            const uint32_t mw = hf == 0 ? (hdr.z & 0x3f3f3f3fu)
                                        : (((hdr.w >> 4) & 0x0f0f0f0fu) | ((hdr.z >> 2) & 0x30303030u));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[j] = dd * (float)((scw >> (8 * j)) & 0xffu);
                g[j] = dm * (float)((mw >> (8 * j)) & 0xffu);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sm.fw[j][tid] = f[j];
            sm.fm[j][tid] = g[j];
        }
    }
}

// q (0..63 per byte) -> q - 32 as int8 per byte.
__device__ __forceinline__ uint32_t q6_center(uint32_t qv)
{
    uint32_t v = qv ^ 0x20202020u;          // 6-bit two's complement of q - 32
    const uint32_t sgn = v & 0x20202020u;
    return v | (sgn << 1) | (sgn << 2);     // sign-extend bit 5 into bits 6, 7
}

// Stage Q6_K weights for rows [n0, n0+BN), half g of super-block sb
// (weights 128g .. 128g+127 of the block).
__device__ __forceinline__ void stage_w_q6k(Smem<true> &sm, const uint8_t *__restrict__ W,
                                            int N, int K, int n0, int sb, int g)
{
    const int tid = threadIdx.x;
    const int64_t rowb = (int64_t)(K >> 8) * 210;
    const int row = tid >> 1;
    const int hh = tid & 1;
    const int n = n0 + row;
    uint32_t qr[4][4];
    float f[8];
    if (n < N) {
        const uint8_t *bp = W + (int64_t)n * rowb + (int64_t)sb * 210;
        uint32_t l0[4], l1[4], h[4];
        load_dwords_a2<4>(bp + 64 * g + 16 * hh, l0);
        load_dwords_a2<4>(bp + 64 * g + 32 + 16 * hh, l1);
        load_dwords_a2<4>(bp + 128 + 32 * g + 16 * hh, h);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qr[0][i] = q6_center((l0[i] & 0x0f0f0f0fu) | ((h[i] << 4) & 0x30303030u));
            qr[1][i] = q6_center((l1[i] & 0x0f0f0f0fu) | ((h[i] << 2) & 0x30303030u));
            qr[2][i] = q6_center(((l0[i] >> 4) & 0x0f0f0f0fu) | (h[i] & 0x30303030u));
            qr[3][i] = q6_center(((l1[i] >> 4) & 0x0f0f0f0fu) | ((h[i] >> 2) & 0x30303030u));
        }
        if (hh == 0) {
            uint32_t sc[2];
            load_dwords_a2<2>(bp + 192 + 8 * g, sc);
            const float dd = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(bp + 208));
#pragma unroll
            for (int j = 0; j < 8; ++j)
                f[j] = dd * (float)(int)(int8_t)(sc[j >> 2] >> (8 * (j & 3)));
        }
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qr[r][i] = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            f[j] = 0.0f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        *reinterpret_cast<v4i *>(&sm.b[row][32 * r + 16 * hh]) =
            v4i{(int)qr[r][0], (int)qr[r][1], (int)qr[r][2], (int)qr[r][3]};
    if (hh == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            sm.fw[j][row] = f[j];
    }
}

template <bool Q6>
__global__ __launch_bounds__(NTHR, 2) void gemm_kernel(
    const uint8_t *__restrict__ W, const int8_t *__restrict__ q,
    const float *__restrict__ dx, const float *__restrict__ sx, int M, int N,
    int K, int tiles_m, float *__restrict__ out)
{
    __shared__ Smem<Q6> sm;
    const int tile_m = blockIdx.x % tiles_m;
    const int tile_n = blockIdx.x / tiles_m;
    const int t0 = tile_m * BM;
    const int n0 = tile_n * BN;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave & 1;          // 64-token half of the tile
    const int wn = wave >> 1;         // 64-row half of the tile
    const int lr = lane & 31;         // operand row / result column
    const int lh = lane >> 5;         // K half / result row group

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[a][b][v] = 0.0f;

    const int nsteps = K / BK;
    for (int st = 0; st < nsteps; ++st) {
        const int k0 = st * BK;
        __syncthreads();                       // previous step's reads done
        stage_act<Q6>(sm, q, dx, sx, M, K, t0, k0);
        if constexpr (Q6)
            stage_w_q6k(sm, W, N, K, n0, st >> 1, st & 1);
        else
            stage_w_q4k(sm, W, N, K, n0, st >> 1, st & 1);
        __syncthreads();

        if constexpr (!Q6) {
#pragma unroll
            for (int j = 0; j < BK / 32; ++j) {
                v4i af[2], bf[2];
#pragma unroll
                for (int a = 0; a < 2; ++a)
                    af[a] = *reinterpret_cast<const v4i *>(&sm.a[wm * 64 + a * 32 + lr][32 * j + 16 * lh]);
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    bf[b] = *reinterpret_cast<const v4i *>(&sm.b[wn * 64 + b * 32 + lr][32 * j + 16 * lh]);
                v16i I[2][2];
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        I[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], v16i{}, 0, 0, 0);
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    float dxv[16], sxv[16];
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int tl = wm * 64 + a * 32 + 8 * g4 + 4 * lh;
                        const float4 d4 = *reinterpret_cast<const float4 *>(&sm.dx[j][tl]);
                        const float4 s4 = *reinterpret_cast<const float4 *>(&sm.sx[j][tl]);
                        dxv[4 * g4 + 0] = d4.x; dxv[4 * g4 + 1] = d4.y;
                        dxv[4 * g4 + 2] = d4.z; dxv[4 * g4 + 3] = d4.w;
                        sxv[4 * g4 + 0] = s4.x; sxv[4 * g4 + 1] = s4.y;
                        sxv[4 * g4 + 2] = s4.z; sxv[4 * g4 + 3] = s4.w;
                    }
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        const int nl = wn * 64 + b * 32 + lr;
                        const float fw = sm.fw[j][nl];
                        const float fm = -sm.fm[j][nl];
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            float t = fmaf((float)I[a][b][v], dxv[v] * fw, acc[a][b][v]);
                            acc[a][b][v] = fmaf(sxv[v], fm, t);
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < BK / 16; ++j) {
                long af[2], bf[2];
#pragma unroll
                for (int a = 0; a < 2; ++a)
                    af[a] = *reinterpret_cast<const long *>(&sm.a[wm * 64 + a * 32 + lr][16 * j + 8 * lh]);
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    bf[b] = *reinterpret_cast<const long *>(&sm.b[wn * 64 + b * 32 + lr][16 * j + 8 * lh]);
                v16i I[2][2];
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        I[a][b] = __builtin_amdgcn_mfma_i32_32x32x16_i8(af[a], bf[b], v16i{}, 0, 0, 0);
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    float dxv[16];
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int tl = wm * 64 + a * 32 + 8 * g4 + 4 * lh;
                        const float4 d4 = *reinterpret_cast<const float4 *>(&sm.dx[j >> 1][tl]);
                        dxv[4 * g4 + 0] = d4.x; dxv[4 * g4 + 1] = d4.y;
                        dxv[4 * g4 + 2] = d4.z; dxv[4 * g4 + 3] = d4.w;
                    }
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        const int nl = wn * 64 + b * 32 + lr;
                        const float fw = sm.fw[j][nl];
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            acc[a][b][v] = fmaf((float)I[a][b][v], dxv[v] * fw, acc[a][b][v]);
                    }
                }
            }
        }
    }

    // store: lane owns column n0 + nl and rows t0 + tl (+ v layout)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int n = n0 + wn * 64 + b * 32 + lr;
            if (n < N) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int t = t0 + wm * 64 + a * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                    if (t < M)
                        out[(int64_t)t * N + n] = acc[a][b][v];
                }
            }
        }
    }
}

template <bool Q6>
hipError_t launch_gemm(const uint8_t *W, const int8_t *q, const float *d,
                       const float *s, int M, int N, int K, float *out,
                       hipStream_t st)
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int64_t grid = (int64_t)tiles_m * tiles_n;
    gemm_kernel<Q6><<<dim3((unsigned)grid), dim3(NTHR), 0, st>>>(W, q, d, s, M, N, K, tiles_m, out);
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemm_q6k(const uint8_t *W, const int8_t *q, const float *d,
                           int M, int N, int K, float *out, hipStream_t st)
{
    return launch_gemm<true>(W, q, d, nullptr, M, N, K, out, st);
}

} // namespace mq
