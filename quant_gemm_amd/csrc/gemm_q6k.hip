// Prefill GEMM for Q6_K weights x per-32 int8 activations (gfx950).
//
// The pages' prefill runs an int8 tensor-core GEMM on the raw quants for
// q6_K as for q4_K (minfer Features, "GPU — CUDA": raw-nibble int8 GEMMs
// for q4_K and q6_K). Q6_K has an int8 scale per 16 values, so one int8
// product per 32-value activation block would mix two scales. Here the scale
// is folded into the weights exactly: each weight becomes
//     p = sc * (q - 32)  in [-4064, 4096],  split as  p = 64 * hi + lo,
// lo = p & 63 in [0, 63] and hi = p >> 6 in [-64, 64], both int8. Two
// v_mfma_i32_32x32x32_i8 per 32-value block (one per limb) give
//     J = 64 * I_hi + I_lo = sum_k sc_k * (q_k - 32) * x_k
// exactly in int32 (|J| <= 32 * 4096 * 127 < 2^31). The result is
//     out[t, n] = sum over super-blocks s of d[n, s] * sum_b d_x[t, b] * J_b,
// and d changes only once per 256 values, so each accumulator is kept in
// units of its row's current d: acc' += d_x[t] * J per 32 values (combine,
// convert, fma: 3 VALU operations), and at each super-block whose d is
// nonzero acc' is multiplied by d_old / d_new once (16 operations per row
// tile per 256 values); the stored result is acc' * d. A super-block with
// d = 0 contributes nothing: its limbs are written as zeros and the scale
// is kept. Each rescale rounds twice (the quotient and the product), at
// most 2 * K/256 * 2^-24 relative on the running sum.
//
// Tiling and staging follow the Q4_K kernel: a 256-thread workgroup computes
// 128 tokens x 128 rows as 4 wavefronts of 32 tokens x 128 rows (1 x 4 MFMA
// tiles of 32 x 32); K moves in steps of 128 values (half a super-block:
// weights 128g .. 128g+127). Activations arrive by global->LDS DMA into
// XOR-swizzled double buffers. The weights are decoded to limbs on the way
// into LDS (their 210-byte blocks are only 2-byte aligned, so they are read
// with aligned dword loads realigned in registers): the limb planes use one
// buffer, written between two barriers.
//
// Expansion planes: a second kernel reads the two limbs and d from planes
// built once at registration (mq_expand_q6k) instead of decoding the raw
// blocks on every tile, as the pages' q6_K expansion planes do (minfer
// Features, "GPU — CUDA"). With nothing to decode it stages everything by
// DMA into double-buffered 64-value steps (see "planes GEMM" below).
//
// MFMA operand layout (32x32x32): lane l supplies row (l % 32) of A and
// column (l % 32) of B, 16 consecutive K values from 16 * (l / 32) each;
// both operands split K alike. The result gives lane l column (l % 32) and
// rows 8*(v/4) + 4*(l/32) + (v%4). A = activations, B = weight limbs.
#include "mq_device.h"
#include "mq_launch.h"

#include <type_traits>

namespace mq {
namespace {

// Workgroup tile: WM x WN wavefronts, each 1 x TN MFMA tiles of 32 x 32.
#ifndef MQ_Q6K_TN
#define MQ_Q6K_TN 4
#define MQ_Q6K_WM 4
#define MQ_Q6K_WN 1
#endif
constexpr int TM = 1, TN = MQ_Q6K_TN, WM = MQ_Q6K_WM, WN = MQ_Q6K_WN;
constexpr int BM = 32 * TM * WM;            // tokens per tile
constexpr int BN = 32 * TN * WN;            // rows per tile
constexpr int BK = 128;
constexpr int NWAVES = WM * WN;
constexpr int NTHR = 64 * NWAVES;
// int8 ops per second of one resident workgroup, for the split-K choice
constexpr double Q6K_SLOT_OPS = 0.6e12;
constexpr int A_CHUNKS = BM * BK / 16;      // 16-byte activation chunks per step
static_assert(A_CHUNKS % (64 * NWAVES) == 0, "DMA split");
static_assert(NTHR == 2 * BN && NTHR >= BM, "one thread per (row, half) and per token");

// LDS. 16-byte chunk c of row r sits in slot r*8 + (c ^ ((r >> 1) & 7)) in
// the activation tiles and in both limb planes: sixteen consecutive 128-byte
// rows reading one chunk fall in sixteen different 4-bank groups.
struct alignas(16) ActStage {
    int8_t a[A_CHUNKS * 16];
    float dx[BK / 32][BM];
};
struct alignas(16) WgtStage {
    int8_t lo[BN * BK];
    int8_t hi[BN * BK];
    float dw[BN];                            // d of the row's super-block
};

__device__ __forceinline__ int slot8(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Activation tile of step st by DMA; rows past M read the last valid row.
__device__ __forceinline__ void issue_act(ActStage &s, const int8_t *__restrict__ q, int M,
                                          int K, int t0, int st, int wave, int lane)
{
    const int k0 = st * BK;
#pragma unroll
    for (int ii = 0; ii < A_CHUNKS / 64 / NWAVES; ++ii) {
        const int i = wave * (A_CHUNKS / 64 / NWAVES) + ii;
        const int p = 64 * i + lane;
        const int r = p >> 3;
        const int c = (p & 7) ^ ((r >> 1) & 7);
        const int t = min(t0 + r, M - 1);
        dma16(q + (int64_t)t * K + k0 + 16 * c, s.a + 1024 * i);
    }
}

// Expansion planes of the weights: limbs lo / hi [N][K], d [N][K/256].
struct Planes {
    const int8_t *lo, *hi;
    const float *dw;
};

// One thread's raw share of a step: row n0 + tid/2, half hh = tid & 1 of
// the 128 weights (positions 32r + 16hh + i, r = 0..3, i = 0..15). The
// fields start 2 bytes into a dword when the block does; the aligned dwords
// covering them are kept as loaded and realigned only after the step's
// compute, so the loads stay in flight during it.
struct Raw {
    uint32_t w0[5], w1[5], wh[5], ws[3];
    uint32_t sh;                             // 0 or 2: byte offset of the fields in their dwords
    uint32_t dbits;
    float4 ds;                               // 4 activation scales of token tid (tid < BM)
};
template <int n>
__device__ __forceinline__ void load_dw(const uint8_t *p, uint32_t (&w)[n + 1], uint32_t sh)
{
    const uint32_t *b = reinterpret_cast<const uint32_t *>(p - sh);   // stays a global pointer
#pragma unroll
    for (int i = 0; i < n; ++i)
        w[i] = b[i];
    // the dword past the field only when the field straddles one; otherwise a
    // dword inside the field (ignored by realign), so no load leaves the block
    w[n] = b[sh ? n : n - 1];
}

template <int n>
__device__ __forceinline__ void realign(const uint32_t (&w)[n + 1], uint32_t sh, uint32_t (&o)[n])
{
#pragma unroll
    for (int i = 0; i < n; ++i)
        o[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
}

__device__ __forceinline__ void load_raw(Raw &p, const uint8_t *__restrict__ W,
                                         const float *__restrict__ dx, int M, int N, int K,
                                         int t0, int n0, int st)
{
    const int tid = threadIdx.x;
    const int row = tid >> 1, hh = tid & 1;
    const int g = st & 1;
    const int n = min(n0 + row, N - 1);
    // Fields start at block offset + an even number of bytes; the block
    // offset is 0 or 2 mod 4, so all fields share the dword phase sh.
    // Reads stay within [field - 2, field end + 2), inside the block.
    const uint8_t *bp = W + (int64_t)n * ((K >> 8) * 210) + (int64_t)(st >> 1) * 210;
    p.sh = (uint32_t)(reinterpret_cast<uintptr_t>(bp) & 3u);
    load_dw<4>(bp + 64 * g + 16 * hh, p.w0, p.sh);
    load_dw<4>(bp + 64 * g + 32 + 16 * hh, p.w1, p.sh);
    load_dw<4>(bp + 128 + 32 * g + 16 * hh, p.wh, p.sh);
    load_dw<2>(bp + 192 + 8 * g, p.ws, p.sh);
    p.dbits = *reinterpret_cast<const uint16_t *>(bp + 208);
    const int t = min(t0 + (tid & (BM - 1)), M - 1);
    p.ds = *reinterpret_cast<const float4 *>(dx + (int64_t)t * (K >> 5) + (st * BK >> 5));
}

typedef short v2s __attribute__((ext_vector_type(2)));

// Four 6-bit quants (bytes of qv, 0..63) times the int8 scale s, split into
// the low limb (p & 63) and the high limb (p >> 6), four bytes each.
__device__ __forceinline__ void limbs4(uint32_t qv, int s, uint32_t &lo, uint32_t &hi)
{
    // bytes 0, 2 and bytes 1, 3 as 16-bit lanes
    const uint32_t ea = __builtin_amdgcn_perm(0u, qv, 0x0c020c00u);
    const uint32_t eb = __builtin_amdgcn_perm(0u, qv, 0x0c030c01u);
    const v2s s2 = {(short)s, (short)s};
    const v2s c32 = {32, 32};
    const v2s pa = (__builtin_bit_cast(v2s, ea) - c32) * s2;
    const v2s pb = (__builtin_bit_cast(v2s, eb) - c32) * s2;
    const v2s m63 = {63, 63};
    const uint32_t la = __builtin_bit_cast(uint32_t, (v2s)(pa & m63));
    const uint32_t lb = __builtin_bit_cast(uint32_t, (v2s)(pb & m63));
    const uint32_t ha = __builtin_bit_cast(uint32_t, (v2s)(pa >> (short)6));
    const uint32_t hb = __builtin_bit_cast(uint32_t, (v2s)(pb >> (short)6));
    // interleave back to byte order w0, w1, w2, w3
    lo = __builtin_amdgcn_perm(lb, la, 0x06020400u);
    hi = __builtin_amdgcn_perm(hb, ha, 0x06020400u);
}

__device__ __forceinline__ void store_act_scales(ActStage &a, const float4 &ds, int M, int t0)
{
    const int tid = threadIdx.x;
    const bool tok = t0 + (tid & (BM - 1)) < M;
    const float4 v = tok ? ds : make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < BM) {
        a.dx[0][tid] = v.x;
        a.dx[1][tid] = v.y;
        a.dx[2][tid] = v.z;
        a.dx[3][tid] = v.w;
    }
}

__device__ __forceinline__ void store_raw(WgtStage &w, ActStage &a, const Raw &p, int M, int N,
                                          int t0, int n0)
{
    const int tid = threadIdx.x;
    const int row = tid >> 1, hh = tid & 1;
    // rows past N and super-blocks with d = 0 (either sign) get zero limbs
    const bool rok = n0 + row < N && (p.dbits & 0x7fffu) != 0;
    uint32_t l0[4], l1[4], h[4], sc[2];
    realign<4>(p.w0, p.sh, l0);
    realign<4>(p.w1, p.sh, l1);
    realign<4>(p.wh, p.sh, h);
    realign<2>(p.ws, p.sh, sc);
    // scales of the four 16-value groups 2r + hh, r = 0..3
    int s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        s[r] = rok ? (int)(int8_t)(sc[r >> 1] >> (16 * (r & 1) + 8 * hh)) : 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t l = r & 1 ? l1[i] : l0[i];
            const uint32_t nib = (r >> 1 ? (l >> 4) : l) & 0x0f0f0f0fu;
            const uint32_t hb = ((r == 0 ? h[i] << 4 : r == 1 ? h[i] << 2 : r == 2 ? h[i] : h[i] >> 2)) &
                                0x30303030u;
            limbs4(nib | hb, s[r], lo[i], hi[i]);
        }
        const int c = 2 * r + hh;            // 16-byte chunk of the row
        *reinterpret_cast<v4i *>(w.lo + 16 * slot8(row, c)) = v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
        *reinterpret_cast<v4i *>(w.hi + 16 * slot8(row, c)) = v4i{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    // every thread consumes its loaded values (only some store them), so no
    // load into these registers is left pending into the next step
    const float dwv = rok ? f16_bits_to_f32(p.dbits) : 0.0f;   // 0: limbs zeroed, scale kept
    if (hh == 0)
        w.dw[row] = dwv;
    store_act_scales(a, p.ds, M, t0);
}

// FIRST: the step opens a super-block, so each row tile moves its
// accumulator to the new d (cur[b]: the d the accumulator is counted in).
template <bool FIRST>
__device__ __forceinline__ void compute_step(const ActStage &a, const WgtStage &w,
                                             v16f (&acc)[TN], float (&cur)[TN], int wm, int wn, int lr,
                                             int lh)
{
    if constexpr (FIRST) {
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const float dn = w.dw[(wn * TN + b) * 32 + lr];
            if (dn != 0.0f) {
                const float f = cur[b] / dn;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[b][v] *= f;
                cur[b] = dn;
            }
        }
    }
    if constexpr (TN == 4) {
        // The two limb MFMAs of the next tile are issued before each tile's
        // epilogue reads its own (two tiles in flight), and the next sub-block's
        // first tile before the last tile's epilogue: at the step's last
        // sub-block that product repeats tile 0 of the same sub-block and is not
        // used (1 of the step's 16 MFMA pairs), so that every sub-block runs the
        // same rolled loop body; the stages are pinned by scheduling barriers
        // (measured 3% faster than each tile's MFMAs followed at once by its
        // epilogue). Skipping that pair, by a branch or by peeling the last
        // sub-block, takes the kernel past 256 registers (99 to 119 spilled),
        // and the MFMA pipe is not what bounds it. The expansion-plane kernel
        // below has no such pair.
        const int tr = wm * 32 + lr;
        auto mm = [&](int j, int b, const v4i &afx, v16i &il, v16i &ih) {
            const int r = (wn * TN + b) * 32 + lr;
            const v4i lo = *reinterpret_cast<const v4i *>(w.lo + 16 * slot8(r, 2 * j + lh));
            const v4i hi = *reinterpret_cast<const v4i *>(w.hi + 16 * slot8(r, 2 * j + lh));
            il = __builtin_amdgcn_mfma_i32_32x32x32_i8(afx, lo, v16i{}, 0, 0, 0);
            ih = __builtin_amdgcn_mfma_i32_32x32x32_i8(afx, hi, v16i{}, 0, 0, 0);
        };
        auto epi = [&](int b, const v16i &il, const v16i &ih, const float (&dv)[16]) {
    #pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int J = (ih[v] << 6) + il[v];
                acc[b][v] = fmaf((float)J, dv[v], acc[b][v]);
            }
        };
        v4i af = *reinterpret_cast<const v4i *>(a.a + 16 * slot8(tr, lh));
        v16i pl, ph, ql, qh;
        mm(0, 0, af, pl, ph);
    #pragma unroll 1
        for (int j = 0; j < BK / 32; ++j) {
            float dv[16];
    #pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 d4 = *reinterpret_cast<const float4 *>(&a.dx[j][wm * 32 + 8 * g4 + 4 * lh]);
                dv[4 * g4 + 0] = d4.x;
                dv[4 * g4 + 1] = d4.y;
                dv[4 * g4 + 2] = d4.z;
                dv[4 * g4 + 3] = d4.w;
            }
            const int jn = min(j + 1, BK / 32 - 1);
            const v4i af_n = *reinterpret_cast<const v4i *>(a.a + 16 * slot8(tr, 2 * jn + lh));
            mm(j, 1, af, ql, qh);
            __builtin_amdgcn_sched_barrier(0);
            epi(0, pl, ph, dv);
            __builtin_amdgcn_sched_barrier(0);
            mm(j, 2, af, pl, ph);
            __builtin_amdgcn_sched_barrier(0);
            epi(1, ql, qh, dv);
            __builtin_amdgcn_sched_barrier(0);
            mm(j, 3, af, ql, qh);
            __builtin_amdgcn_sched_barrier(0);
            epi(2, pl, ph, dv);
            __builtin_amdgcn_sched_barrier(0);
            mm(jn, 0, af_n, pl, ph);
            __builtin_amdgcn_sched_barrier(0);
            epi(3, ql, qh, dv);
            __builtin_amdgcn_sched_barrier(0);
            af = af_n;
        }
    } else {
    #pragma unroll 1
        for (int j = 0; j < BK / 32; ++j) {
            const int tr = wm * 32 + lr;
            const v4i af = *reinterpret_cast<const v4i *>(a.a + 16 * slot8(tr, 2 * j + lh));
            float dv[16];
    #pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 d4 = *reinterpret_cast<const float4 *>(&a.dx[j][wm * 32 + 8 * g4 + 4 * lh]);
                dv[4 * g4 + 0] = d4.x;
                dv[4 * g4 + 1] = d4.y;
                dv[4 * g4 + 2] = d4.z;
                dv[4 * g4 + 3] = d4.w;
            }
    #pragma unroll
            for (int b = 0; b < TN; ++b) {
                const int r = (wn * TN + b) * 32 + lr;
                const v4i blo = *reinterpret_cast<const v4i *>(w.lo + 16 * slot8(r, 2 * j + lh));
                const v4i bhi = *reinterpret_cast<const v4i *>(w.hi + 16 * slot8(r, 2 * j + lh));
                const v16i il = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, blo, v16i{}, 0, 0, 0);
                const v16i ih = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bhi, v16i{}, 0, 0, 0);
    #pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int J = (ih[v] << 6) + il[v];
                    acc[b][v] = fmaf((float)J, dv[v], acc[b][v]);
                }
            }
        }
    }
}

__global__ __launch_bounds__(NTHR, 2) void gemm_q6k_kernel(
    const uint8_t *__restrict__ W, const int8_t *__restrict__ q,
    const float *__restrict__ dx, int M, int N, int K, int tiles_m, int nsplit,
    float *__restrict__ out)
{
    __shared__ ActStage A0, A1;
    __shared__ WgtStage B;
    // blockIdx = split * tiles + tile (tile_order maps tile to tile_m and
    // tile_n); split s of nsplit
    // covers the super-blocks [s*P/nsplit, (s+1)*P/nsplit) of P = K/256 and,
    // when nsplit > 1, writes its partial sums to out + s*M*N.
    const int tiles = gridDim.x / nsplit;
    const int split = blockIdx.x / tiles;
    const int tile = blockIdx.x - split * tiles;
    int tile_m, tile_n;
    tile_order(tile, tiles_m, tiles / tiles_m, tile_m, tile_n);
    const int pairs = K >> 8;
    const int st_begin = 2 * (int)((int64_t)split * pairs / nsplit);
    const int st_end = 2 * (int)((int64_t)(split + 1) * pairs / nsplit);
    float *dst = out + (int64_t)split * M * N;
    const int t0 = tile_m * BM;
    const int n0 = tile_n * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: DMA bases in SGPRs
    const int wm = wave % WM, wn = wave / WM;
    const int lr = lane & 31, lh = lane >> 5;

    v16f acc[TN];
    float cur[TN];
#pragma unroll
    for (int b = 0; b < TN; ++b) {
        cur[b] = 1.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[b][v] = 0.0f;
    }

    // The step range is even (whole super-blocks): steps alternate the
    // activation buffers A0, A1.
    Raw p;
    issue_act(A0, q, M, K, t0, st_begin, wave, lane);
    load_raw(p, W, dx, M, N, K, t0, n0, st_begin);
    wait_vm<0>();
    store_raw(B, A0, p, M, N, t0, n0);
    __syncthreads();
    for (int st = st_begin; st < st_end; st += 2) {
        // register loads before the DMA: any wait the compiler puts in front
        // of them then has no DMA in flight to wait for
        load_raw(p, W, dx, M, N, K, t0, n0, st + 1);
        issue_act(A1, q, M, K, t0, st + 1, wave, lane);
        compute_step<true>(A0, B, acc, cur, wm, wn, lr, lh);
        __syncthreads();                      // limb planes of step st consumed
        wait_vm<0>();
        store_raw(B, A1, p, M, N, t0, n0);
        __syncthreads();
        const bool more = st + 2 < st_end;
        if (more) {
            load_raw(p, W, dx, M, N, K, t0, n0, st + 2);
            issue_act(A0, q, M, K, t0, st + 2, wave, lane);
        }
        compute_step<false>(A1, B, acc, cur, wm, wn, lr, lh);
        __syncthreads();
        if (more) {
            wait_vm<0>();
            store_raw(B, A0, p, M, N, t0, n0);
            __syncthreads();
        }
    }

#pragma unroll
    for (int b = 0; b < TN; ++b) {
        const int n = n0 + (wn * TN + b) * 32 + lr;
        if (n < N) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = t0 + wm * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                if (t < M)
                    dst[(int64_t)t * N + n] = acc[b][v] * cur[b];
            }
        }
    }
}

// ---------------------------------------------------------------- planes GEMM
// The expansion planes need no decoding, so their GEMM stages everything by
// global->LDS DMA (the pages stage the W_exp planes with asynchronous
// copies: minfer Features, "GPU — CUDA"): K moves in steps of 64 values
// through two stages, each holding the step's activation tile, both limb
// tiles, the activation scales and (at super-block starts) the rows' d.
// While the wavefronts compute on one stage the DMA fills the other, with
// one barrier per step. The planes hold the limbs of a super-block with
// d = 0 as they are; in a super-block where one of its rows has d = 0, a
// wavefront zeroes those rows' limbs in the stage before it reads them
// (every wavefront that reads a row zeroes it itself, so no barrier is
// needed), as the raw-block kernel writes them.
//
// LDS rows are 64 bytes (4 chunks of 16); chunk c of row r sits in slot
// 4 r + (c ^ ((r >> 2) & 3)), so the 16 rows one MFMA operand read touches
// in a cycle fall in distinct banks.
constexpr int XBK = 64;
constexpr int XSUB = XBK / 32;               // 32-value sub-blocks per step
struct alignas(16) XStage {
    int8_t a[BM * XBK];
    int8_t lo[BN * XBK];
    int8_t hi[BN * XBK];
    float dx[XSUB][BM];
    float dw[BN];
};

__device__ __forceinline__ int slot4(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// The DMA of a stage: 64-lane instructions i = wave + NWAVES * ii over each
// array; every lane keeps the source address of its share of each array
// for step 0 (the step adds 64 values, 2 activation scales and, every 4
// steps, 1 super-block).
constexpr int XA_I = BM * 4 / 64;            // activation tile: 16-byte chunks / 64
constexpr int XW_I = BN * 4 / 64;            // one limb tile
constexpr int XD_I = XSUB * BM / 64;         // activation scales (dwords)
constexpr int XE_I = BN / 64;                // rows' d (dwords)
static_assert(XA_I * 64 == BM * 4 && XW_I * 64 == BN * 4 && XD_I * 64 == XSUB * BM && XE_I * 64 == BN,
              "whole DMA instructions");
template <int I>
constexpr int per_wave() { return (I + NWAVES - 1) / NWAVES; }

struct XSrc {
    const int8_t *a[per_wave<XA_I>()];
    const int8_t *lo[per_wave<XW_I>()];
    const int8_t *hi[per_wave<XW_I>()];
    const float *dx[per_wave<XD_I>()];
    const float *dw[per_wave<XE_I>()];
};

__device__ __forceinline__ XSrc x_src(const Planes &E, const int8_t *__restrict__ q, const float *__restrict__ dx,
                                      int M, int N, int K, int t0, int n0, int wave, int lane)
{
    XSrc S;
    auto chunk = [&](int i, int &r, int &c) {
        const int p = 64 * i + lane;
        r = p >> 2;
        c = (p & 3) ^ ((r >> 2) & 3);
    };
#pragma unroll
    for (int ii = 0; ii < per_wave<XA_I>(); ++ii) {
        int r, c;
        chunk(wave + NWAVES * ii, r, c);
        S.a[ii] = q + (int64_t)min(t0 + r, M - 1) * K + 16 * c;
    }
#pragma unroll
    for (int ii = 0; ii < per_wave<XW_I>(); ++ii) {
        int r, c;
        chunk(wave + NWAVES * ii, r, c);
        const int64_t o = (int64_t)min(n0 + r, N - 1) * K + 16 * c;
        S.lo[ii] = E.lo + o;
        S.hi[ii] = E.hi + o;
    }
#pragma unroll
    for (int ii = 0; ii < per_wave<XD_I>(); ++ii) {
        const int p = 64 * (wave + NWAVES * ii) + lane;
        S.dx[ii] = dx + (int64_t)min(t0 + p % BM, M - 1) * (K >> 5) + p / BM;
    }
#pragma unroll
    for (int ii = 0; ii < per_wave<XE_I>(); ++ii) {
        const int r = 64 * (wave + NWAVES * ii) + lane;
        S.dw[ii] = E.dw + (int64_t)min(n0 + r, N - 1) * (K >> 8);
    }
    return S;
}

__device__ __forceinline__ void x_issue(XStage &S, const XSrc &src, int st, int wave)
{
    const int64_t k0 = (int64_t)st * XBK;
#pragma unroll
    for (int ii = 0; ii < per_wave<XA_I>(); ++ii) {
        const int i = wave + NWAVES * ii;
        if (XA_I % NWAVES == 0 || i < XA_I)  // wavefront-uniform
            dma16(src.a[ii] + k0, S.a + 1024 * i);
    }
#pragma unroll
    for (int ii = 0; ii < per_wave<XW_I>(); ++ii) {
        const int i = wave + NWAVES * ii;
        if (XW_I % NWAVES == 0 || i < XW_I) {
            dma16(src.lo[ii] + k0, S.lo + 1024 * i);
            dma16(src.hi[ii] + k0, S.hi + 1024 * i);
        }
    }
#pragma unroll
    for (int ii = 0; ii < per_wave<XD_I>(); ++ii) {
        const int i = wave + NWAVES * ii;
        if (XD_I % NWAVES == 0 || i < XD_I)
            dma4(src.dx[ii] + XSUB * st, &S.dx[0][0] + 64 * i);
    }
    if ((st & 3) == 0) {                     // a super-block starts: the rows' d
#pragma unroll
        for (int ii = 0; ii < per_wave<XE_I>(); ++ii) {
            const int i = wave + NWAVES * ii;
            if (XE_I % NWAVES == 0 || i < XE_I)
                dma4(src.dw[ii] + (st >> 2), S.dw + 64 * i);
        }
    }
}

// One step on a stage: for each sub-block, each tile's two limb MFMAs, then
// (while they run) the next tile's limb reads from LDS, then the tile's
// epilogue (combine the limbs, convert, fma with the activation scale). The
// sub-block loop stays rolled, which keeps the MFMA results of one tile at
// a time in registers (164 VGPRs, three workgroups per CU). The empty asm
// statements hold each epilogue in its place: without them the compiler
// moves every epilogue of the step behind all its MFMAs (251 VGPRs).
// Measured on MI355X: the read-ahead cuts the wait cycles by a quarter,
// about 2% of the kernel's time.
__device__ __forceinline__ void x_compute(const XStage &S, v16f (&acc)[TN], int wm, int wn, int lr, int lh)
{
    const int tr = wm * 32 + lr;
    auto ld_w = [&](int j, int b, v4i &lo, v4i &hi) {
        const int r = (wn * TN + b) * 32 + lr;
        lo = *reinterpret_cast<const v4i *>(S.lo + 16 * slot4(r, 2 * j + lh));
        hi = *reinterpret_cast<const v4i *>(S.hi + 16 * slot4(r, 2 * j + lh));
    };
    auto ld_dv = [&](int j, float (&dv)[16]) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const float4 d4 = *reinterpret_cast<const float4 *>(&S.dx[j][wm * 32 + 8 * g4 + 4 * lh]);
            dv[4 * g4 + 0] = d4.x;
            dv[4 * g4 + 1] = d4.y;
            dv[4 * g4 + 2] = d4.z;
            dv[4 * g4 + 3] = d4.w;
        }
    };
    v4i lo, hi;
    ld_w(0, 0, lo, hi);
#pragma unroll 1
    for (int j = 0; j < XSUB; ++j) {
        const v4i af = *reinterpret_cast<const v4i *>(S.a + 16 * slot4(tr, 2 * j + lh));
        float dv[16];
        ld_dv(j, dv);
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const v16i il = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, lo, v16i{}, 0, 0, 0);
            const v16i ih = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, hi, v16i{}, 0, 0, 0);
            if (b + 1 < TN)
                ld_w(j, b + 1, lo, hi);
            else if (j + 1 < XSUB)
                ld_w(j + 1, 0, lo, hi);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int J = (ih[v] << 6) + il[v];
                acc[b][v] = fmaf((float)J, dv[v], acc[b][v]);
            }
#pragma unroll
            for (int v = 0; v < 16; ++v)
                asm volatile("" : "+v"(acc[b][v]));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// A step: wait for this stage's DMA (own, then everyone's through the
// barrier, which also ends every wavefront's reads of the other stage),
// start the next step's DMA into the other stage, then compute. FIRST: the
// step opens a super-block, so each row tile moves its accumulator to the
// new d (cur[b]: the d the accumulator is counted in).
template <bool FIRST>
__device__ __forceinline__ void x_step(XStage &S, XStage &Snext, const XSrc &src, int st, int st_end,
                                       v16f (&acc)[TN], float (&cur)[TN], bool (&zr)[TN], bool &mask, int wave,
                                       int wm, int wn, int lr, int lh)
{
    wait_vm<0>();
    __syncthreads();
    if (st + 1 < st_end)
        x_issue(Snext, src, st + 1, wave);
    if constexpr (FIRST) {
        bool any = false;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const float dn = S.dw[(wn * TN + b) * 32 + lr];
            zr[b] = dn == 0.0f;
            any |= zr[b];
            if (dn != 0.0f) {
                const float f = cur[b] / dn;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[b][v] *= f;
                cur[b] = dn;
            }
        }
        mask = __any(any);
    }
    if (mask) {                              // rare: zero the limbs this lane reads of rows with d = 0
        const v4i z = {0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            if (zr[b]) {
                const int r = (wn * TN + b) * 32 + lr;
#pragma unroll
                for (int j = 0; j < XSUB; ++j) {
                    *reinterpret_cast<v4i *>(S.lo + 16 * slot4(r, 2 * j + lh)) = z;
                    *reinterpret_cast<v4i *>(S.hi + 16 * slot4(r, 2 * j + lh)) = z;
                }
            }
        }
    }
    x_compute(S, acc, wm, wn, lr, lh);
}

__global__ __launch_bounds__(NTHR, 2) void gemm_q6k_planes_kernel(
    const Planes E, const int8_t *__restrict__ q, const float *__restrict__ dx, int M, int N, int K,
    int tiles_m, int nsplit, float *__restrict__ out)
{
    __shared__ XStage S0, S1;
    const int tiles = gridDim.x / nsplit;
    const int split = blockIdx.x / tiles;
    const int tile = blockIdx.x - split * tiles;
    int tile_m, tile_n;
    tile_order(tile, tiles_m, tiles / tiles_m, tile_m, tile_n);
    const int sbs = K >> 8;                  // super-blocks; 4 steps each
    const int st_begin = 4 * (int)((int64_t)split * sbs / nsplit);
    const int st_end = 4 * (int)((int64_t)(split + 1) * sbs / nsplit);
    float *dst = out + (int64_t)split * M * N;
    const int t0 = tile_m * BM;
    const int n0 = tile_n * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: DMA bases in SGPRs
    const int wm = wave % WM, wn = wave / WM;
    const int lr = lane & 31, lh = lane >> 5;

    v16f acc[TN];
    float cur[TN];
    bool zr[TN];
    bool mask = false;
#pragma unroll
    for (int b = 0; b < TN; ++b) {
        cur[b] = 1.0f;
        zr[b] = false;
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[b][v] = 0.0f;
    }
    const XSrc src = x_src(E, q, dx, M, N, K, t0, n0, wave, lane);
    if (st_begin < st_end)
        x_issue(S0, src, st_begin, wave);
#pragma unroll 1
    for (int st = st_begin; st < st_end; st += 4) {   // whole super-blocks: stages S0, S1, S0, S1
        x_step<true>(S0, S1, src, st, st_end, acc, cur, zr, mask, wave, wm, wn, lr, lh);
        x_step<false>(S1, S0, src, st + 1, st_end, acc, cur, zr, mask, wave, wm, wn, lr, lh);
#pragma unroll 1
        for (int k = 2; k < 4; k += 2) {          // rolled: one copy of the S0, S1 pair
            x_step<false>(S0, S1, src, st + k, st_end, acc, cur, zr, mask, wave, wm, wn, lr, lh);
            x_step<false>(S1, S0, src, st + k + 1, st_end, acc, cur, zr, mask, wave, wm, wn, lr, lh);
        }
    }

#pragma unroll
    for (int b = 0; b < TN; ++b) {
        const int n = n0 + (wn * TN + b) * 32 + lr;
        if (n < N) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = t0 + wm * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                if (t < M)
                    dst[(int64_t)t * N + n] = acc[b][v] * cur[b];
            }
        }
    }
}

} // namespace

namespace {
// K ranges of a launch (see gemm_splits); tiles of BM x BN outputs. The
// expansion-plane GEMM takes the same choice, so both give one result.
int nsplit_for(int M, int N, int K)
{
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return gemm_splits(tiles, BM * BN, K >> 8, M, N, K, Q6K_SLOT_OPS);
}
} // namespace

#ifdef MQ_Q6K_SMALL
int splits_gemm_q6k_small(int M, int N, int K) { return nsplit_for(M, N, K); }
hipError_t launch_gemm_q6k_small(const uint8_t *W, const int8_t *q, const float *d,
                                 int M, int N, int K, float *out, const Ws &ws, hipStream_t st)
#else
int splits_gemm_q6k(int M, int N, int K) { return nsplit_for(M, N, K); }
hipError_t launch_gemm_q6k(const uint8_t *W, const int8_t *q, const float *d,
                           int M, int N, int K, float *out, const Ws &ws, hipStream_t st)
#endif
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int nsplit = ws.ptr ? nsplit_for(M, N, K) : 1;
    return run_split_k(nsplit, (int64_t)M * N, out, ws, st, [&](float *dst) {
        launch(gemm_q6k_kernel, dim3((unsigned)(tiles * nsplit)), dim3(NTHR), 0, st, W, q, d, M, N, K, tiles_m,
                                                                                 nsplit, dst);
        return hipGetLastError();
    });
}

#ifdef MQ_Q6K_SMALL
hipError_t launch_gemm_q6k_x_small(const int8_t *lo, const int8_t *hi, const float *dw, const int8_t *q,
                                   const float *d, int M, int N, int K, float *out, const Ws &ws,
                                   hipStream_t st)
#else
hipError_t launch_gemm_q6k_x(const int8_t *lo, const int8_t *hi, const float *dw, const int8_t *q,
                             const float *d, int M, int N, int K, float *out, const Ws &ws, hipStream_t st)
#endif
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int nsplit = ws.ptr ? nsplit_for(M, N, K) : 1;
    const Planes E{lo, hi, dw};
    return run_split_k(nsplit, (int64_t)M * N, out, ws, st, [&](float *dst) {
        launch(gemm_q6k_planes_kernel, dim3((unsigned)(tiles * nsplit)), dim3(NTHR), 0, st, E, q, d, M, N, K, tiles_m,
               nsplit, dst);
        return hipGetLastError();
    });
}

} // namespace mq
