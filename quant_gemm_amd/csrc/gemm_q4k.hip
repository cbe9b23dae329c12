// Prefill GEMM for Q4_K (and, built with MQ_Q5K, Q5_K) weights x per-32
// int8 activations (gfx950).
//
// The pages' prefill runs an int8 tensor-core GEMM on the raw 4-bit quants
// against the int8 activation plane, with the block scales applied after
// each integer product (minfer Features, "GPU — CUDA": raw-nibble int8 GEMMs
// for q4_K and q6_K). This is a CDNA4 design of that step. Q5_K (listed with
// the k-quants the pages' decode path serves, minfer Support Matrix,
// "Supported Quantization Formats") has the same header and sub-blocks plus
// a plane of fifth bits: its quants 0..31 are still exact int8 operands, so
// the same kernel runs it with one more DMA'd tile (32 bytes of high bits
// per row and step) merged into the B operand.
//
// Decoded-scale planes (DSC): the Q4_K kernel can instead take the per
// sub-block factors d*sc and dmin*m from f32 planes built once at
// registration (mq_dsc_q4k; the pages' q4_K decoded-scale plane, minfer
// Features, "GPU — CUDA"), so no block header is decoded per tile.
//
// Tiling. A 256-thread workgroup computes 128 tokens x 128 weight rows as
// 4 wavefronts of 32 tokens x 128 rows, each 1 x 4 MFMA tiles of 32 x 32.
// The K loop moves in half super-blocks (128 values = 4 sub-blocks of 32).
//
// Staging. Each step's slice goes into one of two LDS buffers: the int8
// activations and the weights' raw quant bytes (64 per row: one 16-byte
// chunk holds positions 16h..16h+15 of two sub-blocks, as low and high
// nibbles) by global->LDS DMA (no registers, no LDS store instructions); the
// per-32 activation scales and sums and, per row and sub-block, the f32
// factors d*sc and dmin*m decoded from the block header through registers.
// The loads for step s+1 are issued before step s is computed and fill the
// other buffer, so one barrier per step suffices.
//
// Arithmetic. Every 32-value sub-block is one v_mfma_i32_32x32x32_i8 (exact
// int32 dot of the 4-bit quants with the int8 activations). The f32
// epilogue then adds, per token t, row n and sub-block j,
//     d_x[t,j] * (d*sc_j)[n] * I  -  s_x[t,j] * (dmin*m_j)[n]
// (the min term uses the activation block sums). The first term is a
// per-element scaling (3 VALU operations: convert, scale product, fma); the
// second is a rank-4 product per step, summed on the bf16 matrix cores from
// three-limb splits of both f32 factors (f32 accuracy; see limbs4). On
// gfx950 the VALU part, not the int8 MFMA, bounds the kernel: 3 VALU
// operations per token, row and sub-block against 32 int8 MACs.
//
// MFMA operand layout (32x32x32): lane l supplies row (l % 32) of A and
// column (l % 32) of B, 16 consecutive K values from 16 * (l / 32) each;
// both operands split K alike, so products pair up whatever order the
// hardware uses within a lane. The result gives lane l column (l % 32) and
// rows 8*(v/4) + 4*(l/32) + (v%4), v = 0..15. A = activations (rows =
// tokens), B = weights (columns = output rows).
#include "mq_device.h"
#include "mq_launch.h"
#include "quant_core.h"

namespace mq {
namespace {

// Workgroup tile: WM x WN wavefronts, each TM x TN MFMA tiles of 32 x 32.
// One wavefront owns 32 tokens x 128 rows: each activation scale/sum read
// from LDS then serves four row tiles (measured fastest on MI355X among
// 64x64, 32x64 and 64x32 wave tiles).
#ifndef MQ_Q5K
#define MQ_Q5K 0
#endif
constexpr bool Q5 = MQ_Q5K;
constexpr int BLK_BYTES = Q5 ? 176 : 144; // super-block size
constexpr int QS_OFF = Q5 ? 48 : 16;      // offset of the 128 low-nibble bytes
#ifndef MQ_Q4K_TM
#define MQ_Q4K_TM 1
#define MQ_Q4K_TN 4
#define MQ_Q4K_WM 4
#define MQ_Q4K_WN 1
#define MQ_Q4K_OCC 2
#endif
constexpr int TM = MQ_Q4K_TM;             // 32-token tiles per wavefront
constexpr int TN = MQ_Q4K_TN;             // 32-row tiles per wavefront
constexpr int WM = MQ_Q4K_WM;             // wavefronts along tokens
constexpr int WN = MQ_Q4K_WN;             // wavefronts along rows
constexpr int BM = 32 * TM * WM;          // tokens per tile
constexpr int BN = 32 * TN * WN;          // weight rows per tile
constexpr int BK = 128;                   // K values per step
constexpr int NWAVES = WM * WN;
constexpr int NTHR = 64 * NWAVES;
// int8 ops per second of one resident workgroup (about 500 TOPS over 512
// resident workgroups), for the split-K choice
constexpr double Q4K_SLOT_OPS = Q5 ? 0.85e12 : 1.0e12;
constexpr int A_CHUNKS = BM * BK / 16;      // 16-byte activation chunks per step
constexpr int Q_CHUNKS = BN * BK / 2 / 16;  // 16-byte raw quant chunks per step
constexpr int H_CHUNKS = Q5 ? BN * 2 : 0;   // 16-byte high-bit chunks per step (Q5_K)
static_assert(A_CHUNKS % (64 * NWAVES) == 0 && Q_CHUNKS % (64 * NWAVES) == 0 &&
              H_CHUNKS % (64 * NWAVES) == 0, "DMA split");
static_assert(NTHR >= 2 * BM && NTHR >= BN, "side loads need one thread per row");

// LDS layout of one step. The activation and quant tiles are filled by
// global->LDS DMA, 64 lanes x 16 bytes per instruction into consecutive
// slots, so they hold 16-byte chunks in a permuted order instead of padded
// rows: chunk c of row r sits in slot  r*8 + (c ^ ((r >> 1) & 7))
// (activations, 8 chunks per row) or  r*4 + (c ^ ((r >> 2) & 3))  (quants,
// 4 per row). Sixteen consecutive rows reading the same chunk (the lanes an
// LDS read serves together) then hit sixteen different 4-bank groups; with
// c ^ (r & 7) for the 128-byte rows, rows r and r + 8 shared one (2-way
// conflicts, 14.7M conflict cycles per launch at 3314 x 18944 x 3584). Q5_K's high bits (the block's whole qh[32], of which a step
// uses 4 bit positions) sit in slot  r*2 + (c ^ ((r >> 2) & 1)).
struct alignas(16) Stage {
    int8_t a[A_CHUNKS * 16];
    uint8_t qs[Q_CHUNKS * 16];
    uint8_t qh[Q5 ? H_CHUNKS * 16 : 16];
    float dx[BK / 32][BM];
    float fw[BK / 32][BN];
    // bf16 limbs of s_x for the step's 4 sub-blocks (see limbs4), part p of
    // token t at sxl[p][t]: 16-byte strides, so a wavefront's reads of one
    // part hit consecutive banks
    uint4 sxl[2][BM];
    uint4 fml[2][BN];       // bf16 limbs of -(dmin*m_j), the same way
};

// The min term  -sum_j s_x[t,j] * (dmin*m_j)[n]  is a contraction over the
// sub-blocks, so it runs on the bf16 matrix cores instead of the VALU. Each
// f32 factor is split into three bf16 limbs, x = x1 + x2 + x3 up to 2^-27
// relative (each limb the nearest bf16 of what the previous ones left), and
// the eight limb products other than x3*y3 are summed with f32 accumulation:
// the same accuracy as one f32 multiply-add per sub-block. A record holds,
// for one token or row, the limbs of the step's 4 sub-blocks as bf16 pairs:
// part 0 = {x1 j0j1, x1 j2j3, x2 j0j1, x2 j2j3}, part 1 = {x3 j0j1, x3 j2j3, 0, 0}.
__device__ __forceinline__ void limbs4(const float (&x)[4], uint4 &r0, uint4 &r1)
{
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        bf16_limbs3(x[j], h[j], m[j], l[j]);
    r0 = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), m[0] | (m[1] << 16), m[2] | (m[3] << 16));
    r1 = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), 0u, 0u);
}

// Weight row r (0..BN-1) of a tile. Plain GEMM: row n0 + r of W. Gate|up
// (FFN): rows 0..63 are the gate rows n0..n0+63 (W) and rows 64..127 the up
// rows n0..n0+63 (W2), so that a lane's tiles b and b+2 hold g and u of the
// same output column. Rows past N read the last row (never stored).
struct WRows {
    const uint8_t *W, *W2;
    int n0, N;
    int64_t rowb;
    template <bool FFN>
    __device__ __forceinline__ const uint8_t *row(int r) const
    {
        if (FFN)
            return (r < 64 ? W : W2) + (int64_t)min(n0 + (r & 63), N - 1) * rowb;
        return W + (int64_t)min(n0 + r, N - 1) * rowb;
    }
    template <bool FFN>
    __device__ __forceinline__ bool valid(int r) const
    {
        return (FFN ? n0 + (r & 63) : n0 + r) < N;
    }
};

__device__ __forceinline__ int a_slot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }
__device__ __forceinline__ int q_slot(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }
__device__ __forceinline__ int h_slot(int r, int c) { return r * 2 + (c ^ ((r >> 2) & 1)); }

// Start the DMA of step st's activation and quant tiles into s. Rows past M
// or N read the last valid row instead: their results are never stored.
template <bool FFN>
__device__ __forceinline__ void issue_tiles(Stage &s, const WRows &rows,
                                            const int8_t *__restrict__ q, int M, int K,
                                            int t0, int st, int wave, int lane)
{
    const int k0 = st * BK;
    const int sb = st >> 1, hf = st & 1;
#pragma unroll
    for (int ii = 0; ii < A_CHUNKS / 64 / NWAVES; ++ii) {
        const int i = wave * (A_CHUNKS / 64 / NWAVES) + ii;
        const int p = 64 * i + lane;
        const int r = p >> 3;
        const int c = (p & 7) ^ ((r >> 1) & 7);
        const int t = min(t0 + r, M - 1);
        dma16(q + (int64_t)t * K + k0 + 16 * c, s.a + 1024 * i);
    }
#pragma unroll
    for (int ii = 0; ii < Q_CHUNKS / 64 / NWAVES; ++ii) {
        const int i = wave * (Q_CHUNKS / 64 / NWAVES) + ii;
        const int p = 64 * i + lane;
        const int r = p >> 2;
        const int c = (p & 3) ^ ((r >> 2) & 3);
        dma16(rows.row<FFN>(r) + (int64_t)sb * BLK_BYTES + QS_OFF + 64 * hf + 16 * c, s.qs + 1024 * i);
    }
    if constexpr (Q5) {
#pragma unroll
        for (int ii = 0; ii < H_CHUNKS / 64 / NWAVES; ++ii) {
            const int i = wave * (H_CHUNKS / 64 / NWAVES) + ii;
            const int p = 64 * i + lane;
            const int r = p >> 1;
            const int c = (p & 1) ^ ((r >> 2) & 1);
            dma16(rows.row<FFN>(r) + (int64_t)sb * BLK_BYTES + 16 + 16 * c, s.qh + 1024 * i);
        }
    }
}

// The per-row block header and the per-token scales / sums of a step pass
// through registers (they are decoded or transposed on the way into LDS).
// Loads always read a valid row (clamped); rows past M or N are zeroed when
// stored, so their contributions vanish.
struct Side {
    uint4 hdr;      // block header of row n0 + tid (tid < BN)
    float4 fw, fm;  // DSC: d*sc_j and dmin*m_j of the step's 4 sub-blocks, row n0 + tid
    float4 ds;      // 4 scales (tid < BM) or 4 sums (tid >= BM) of token t0 + tid % BM
};

// Decoded-scale planes fw / fm [N][K/32] (DSC) or none.
struct Dsc {
    const float *fw, *fm;
};

template <bool FFN, bool DSC>
__device__ __forceinline__ void load_side(Side &p, const WRows &rows, const Dsc &dsc,
                                          const float *__restrict__ dx,
                                          const float *__restrict__ sx, int M, int K,
                                          int t0, int st)
{
    const int tid = threadIdx.x;
    const int k0 = st * BK;
    if (tid < BN) {
        if constexpr (DSC) {
            const int64_t i = (int64_t)min(rows.n0 + tid, rows.N - 1) * (K >> 5) + (k0 >> 5);
            p.fw = *reinterpret_cast<const float4 *>(dsc.fw + i);
            p.fm = *reinterpret_cast<const float4 *>(dsc.fm + i);
        } else {
            p.hdr = *reinterpret_cast<const uint4 *>(rows.row<FFN>(tid) + (int64_t)(st >> 1) * BLK_BYTES);
        }
    }
    if (tid < 2 * BM) {
        const int t = min(t0 + (tid & (BM - 1)), M - 1);
        const float *src = tid < BM ? dx : sx;
        p.ds = *reinterpret_cast<const float4 *>(src + (int64_t)t * (K >> 5) + (k0 >> 5));
    }
}

template <bool FFN, bool DSC>
__device__ __forceinline__ void store_side(Stage &s, const Side &p, const WRows &rows, int st, int M,
                                           int t0)
{
    const int tid = threadIdx.x;
    const int hf = st & 1;
    const int row = tid & (BM - 1);
    const bool tok = t0 + row < M;
    if (tid < BM) {
        s.dx[0][row] = tok ? p.ds.x : 0.0f;
        s.dx[1][row] = tok ? p.ds.y : 0.0f;
        s.dx[2][row] = tok ? p.ds.z : 0.0f;
        s.dx[3][row] = tok ? p.ds.w : 0.0f;
    } else if (tid < 2 * BM) {
        const float x[4] = {tok ? p.ds.x : 0.0f, tok ? p.ds.y : 0.0f, tok ? p.ds.z : 0.0f,
                            tok ? p.ds.w : 0.0f};
        limbs4(x, s.sxl[0][row], s.sxl[1][row]);
    }
    if (DSC && tid < BN) {
        const bool ok = rows.valid<FFN>(tid);
        const float fw[4] = {p.fw.x, p.fw.y, p.fw.z, p.fw.w};
        const float fm[4] = {ok ? -p.fm.x : 0.0f, ok ? -p.fm.y : 0.0f, ok ? -p.fm.z : 0.0f,
                             ok ? -p.fm.w : 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s.fw[j][tid] = ok ? fw[j] : 0.0f;
        limbs4(fm, s.fml[0][tid], s.fml[1][tid]);
    } else if (tid < BN) {
        // header: f16 d | f16 dmin | 12 bytes of 6-bit codes. Codes j = 0..3
        // are bytes 0..3 (scale) and 4..7 (min) masked to 6 bits; codes
        // 4..7 take their low 4 bits from bytes 8..11 and their high 2 bits
        // from the top of bytes 0..3 (scale) or 4..7 (min).
        const uint4 h = rows.valid<FFN>(tid) ? p.hdr : make_uint4(0, 0, 0, 0);
        const float dd = f16_bits_to_f32(h.x);
        const float dm = f16_bits_to_f32(h.x >> 16);
        const uint32_t scw = hf == 0 ? (h.y & 0x3f3f3f3fu)
                                     : ((h.w & 0x0f0f0f0fu) | ((h.y >> 2) & 0x30303030u));
        const uint32_t mw = hf == 0 ? (h.z & 0x3f3f3f3fu)
                                    : (((h.w >> 4) & 0x0f0f0f0fu) | ((h.z >> 2) & 0x30303030u));
        float fm[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s.fw[j][tid] = dd * (float)((scw >> (8 * j)) & 0xffu);
            fm[j] = -(dm * (float)((mw >> (8 * j)) & 0xffu));
        }
        limbs4(fm, s.fml[0][tid], s.fml[1][tid]);
    }
}

// HF: which half super-block the step covers (its sub-blocks are 4 HF + j).
template <int HF>
__device__ __forceinline__ void compute_step(const Stage &s, v16f (&acc)[TM][TN], int wm, int wn,
                                             int lr, int lh)
{
    if constexpr (TM == 1 && TN == 4) {
        // The main configuration (Q4_K and Q5_K) rolls its int8 MFMAs under
        // the epilogue (Q5_K measured 1016 against 1067 us without): two
        // 32x32 tiles are in flight, and each tile's MFMA for the sub-block is
        // issued as soon as the epilogue before it has read its register
        // buffer; the next sub-block's activation fragment, weight factors
        // and (at the chunk change) quant chunks are read from LDS while the
        // current epilogue runs. The nibbles are unpacked right before each
        // MFMA. The arithmetic per output is unchanged (same products, same
        // order): measured 4% faster than issuing a sub-block's four MFMAs
        // together. Each stage is pinned by a scheduling barrier.
        const int tr = wm * 32 + lr;
        const int tl0 = wm * 32 + 4 * lh;
        auto ld_raw = [&](int cl, v4i (&raw)[TN]) {
#pragma unroll
            for (int b = 0; b < TN; ++b)
                raw[b] = *reinterpret_cast<const v4i *>(s.qs + 16 * q_slot((wn * TN + b) * 32 + lr, 2 * cl + lh));
        };
        auto ld_dv = [&](int j, float (&dv)[16]) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const float4 d4 = *reinterpret_cast<const float4 *>(&s.dx[j][tl0 + 8 * g4]);
                dv[4 * g4] = d4.x;
                dv[4 * g4 + 1] = d4.y;
                dv[4 * g4 + 2] = d4.z;
                dv[4 * g4 + 3] = d4.w;
            }
        };
        auto ld_fw = [&](int j, float (&fw)[TN]) {
#pragma unroll
            for (int b = 0; b < TN; ++b)
                fw[b] = s.fw[j][(wn * TN + b) * 32 + lr];
        };
        // tile b's nibbles for sub-block parity h (low / high half of its
        // chunk); for Q5_K merged with bit 4 HF + j of the lane's 16
        // high-bit bytes of the tile, rotated to bit 4 (j the sub-block
        // within the step; the bytes are re-read from LDS per use to stay
        // within 256 VGPRs)
        auto nib = [&](const v4i (&r)[TN], int h, int b, int j) {
            v4i v = h ? ((r[b] >> 4) & 0x0f0f0f0f) : (r[b] & 0x0f0f0f0f);
            if constexpr (Q5) {
                const v4i hq = *reinterpret_cast<const volatile v4i *>(
                    s.qh + 16 * h_slot((wn * TN + b) * 32 + lr, lh));
                const int rot = (4 * HF + j + 28) & 31;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] |= (int)(__builtin_rotateright32((uint32_t)hq[e], rot) & 0x10101010u);
            }
            return v;
        };
        auto epi = [&](int b, const v16i &I, const float (&dv)[16], float f) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[0][b][v] = fmaf((float)I[v], dv[v] * f, acc[0][b][v]);
        };
        v4i raw[TN];
        ld_raw(0, raw);
        v4i af = *reinterpret_cast<const v4i *>(s.a + 16 * a_slot(tr, lh));
        float dv[16], fw[TN];
        ld_fw(0, fw);
        v16i X = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, nib(raw, 0, 0, 0), v16i{}, 0, 0, 0);
        v16i Y = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, nib(raw, 0, 1, 0), v16i{}, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int h = j & 1;
            v4i af_n = af, raw_n[TN];
            float fw_n[TN];
            ld_dv(j, dv);
            if (j < 3) {
                af_n = *reinterpret_cast<const v4i *>(s.a + 16 * a_slot(tr, 2 * (j + 1) + lh));
                ld_fw(j + 1, fw_n);
                if (j == 1)
                    ld_raw(1, raw_n);
            }
            __builtin_amdgcn_sched_barrier(0);
            epi(0, X, dv, fw[0]);
            X = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, nib(raw, h, 2, j), v16i{}, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            epi(1, Y, dv, fw[1]);
            Y = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, nib(raw, h, 3, j), v16i{}, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            epi(2, X, dv, fw[2]);
            if (j < 3)   // the next sub-block: high nibbles of this chunk, or the next chunk
                X = __builtin_amdgcn_mfma_i32_32x32x32_i8(af_n, nib(j == 1 ? raw_n : raw, h ^ 1, 0, j + 1), v16i{}, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            epi(3, Y, dv, fw[3]);
            if (j < 3) {
                Y = __builtin_amdgcn_mfma_i32_32x32x32_i8(af_n, nib(j == 1 ? raw_n : raw, h ^ 1, 1, j + 1), v16i{}, 0, 0, 0);
                af = af_n;
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    fw[b] = fw_n[b];
                    if (j == 1)
                        raw[b] = raw_n[b];
                }
            }
        }
    } else {
    #pragma unroll 1
        for (int cl = 0; cl < 2; ++cl) {
            v4i raw[TN];
    #pragma unroll
            for (int b = 0; b < TN; ++b) {
                const int r = (wn * TN + b) * 32 + lr;
                raw[b] = *reinterpret_cast<const v4i *>(s.qs + 16 * q_slot(r, 2 * cl + lh));
            }
    #pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int j = 2 * cl + h;            // sub-block within the step
                v4i bf[TN], af[TM];
    #pragma unroll
                for (int b = 0; b < TN; ++b)
                    bf[b] = h ? ((raw[b] >> 4) & 0x0f0f0f0f) : (raw[b] & 0x0f0f0f0f);
                if constexpr (Q5) {
                    // Q5_K: this lane's 16 high-bit bytes (positions 16 lh.. of
                    // the row's sub-blocks), read per sub-block to keep registers
                    // free; bit 4 HF + j of every byte rotated to bit 4
                    const int rot = (4 * HF + j + 28) & 31;
    #pragma unroll
                    for (int b = 0; b < TN; ++b) {
                        const v4i hq = *reinterpret_cast<const volatile v4i *>(
                            s.qh + 16 * h_slot((wn * TN + b) * 32 + lr, lh));
    #pragma unroll
                        for (int e = 0; e < 4; ++e)
                            bf[b][e] |= (int)(__builtin_rotateright32((uint32_t)hq[e], rot) & 0x10101010u);
                    }
                }
    #pragma unroll
                for (int a = 0; a < TM; ++a) {
                    const int r = (wm * TM + a) * 32 + lr;
                    af[a] = *reinterpret_cast<const v4i *>(s.a + 16 * a_slot(r, 2 * j + lh));
                }
                v16i I[TM][TN];
                // raised wave priority while the MFMAs issue, so that they are
                // not queued behind the other wavefront's epilogue (measured +1.5%)
                __builtin_amdgcn_s_setprio(1);
    #pragma unroll
                for (int a = 0; a < TM; ++a)
    #pragma unroll
                    for (int b = 0; b < TN; ++b)
                        I[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], v16i{}, 0, 0, 0);
                __builtin_amdgcn_s_setprio(0);
                float fw[TN];
    #pragma unroll
                for (int b = 0; b < TN; ++b)
                    fw[b] = s.fw[j][(wn * TN + b) * 32 + lr];
    #pragma unroll
                for (int a = 0; a < TM; ++a) {
    #pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int tl = (wm * TM + a) * 32 + 8 * g4 + 4 * lh;
                        const float4 d4 = *reinterpret_cast<const float4 *>(&s.dx[j][tl]);
                        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
    #pragma unroll
                        for (int b = 0; b < TN; ++b) {
    #pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int v = 4 * g4 + r;
                                acc[a][b][v] = fmaf((float)I[a][b][v], dv[r] * fw[b], acc[a][b][v]);
                            }
                        }
                    }
                }
            }
        }
    }
    // Min term of the step's 4 sub-blocks: two 32x32x16 bf16 MFMAs per tile,
    // issued after the step's last epilogue, so that they run while the
    // wavefront moves on to the next step's staging instead of holding up
    // the first epilogue that reads the accumulators they write (measured
    // 1.5-2% faster than at the start of the step).
    // K slot 8*lh + e pairs element e of the A and B operands; lane half 0
    // carries x1*y1, x1*y2 (first MFMA) and x2*y2, x3*y1 (second), lane
    // half 1 x2*y1, x1*y3 and x2*y3, x3*y2, for j = 0..3 each.
    {
        v4i A0[TM], A1[TM];
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            const int t = (wm * TM + a) * 32 + lr;
            const uint4 r0 = s.sxl[0][t], r1 = s.sxl[1][t];
            A0[a] = v4i{(int)(lh ? r0.z : r0.x), (int)(lh ? r0.w : r0.y), (int)r0.x, (int)r0.y};
            A1[a] = v4i{(int)r0.z, (int)r0.w, (int)r1.x, (int)r1.y};
        }
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const int n = (wn * TN + b) * 32 + lr;
            const uint4 q0 = s.fml[0][n], q1 = s.fml[1][n];
            const uint32_t y2a = lh ? q1.x : q0.z, y2b = lh ? q1.y : q0.w;   // y2 | y3
            const v4i B0 = {(int)q0.x, (int)q0.y, (int)y2a, (int)y2b};
            const v4i B1 = {(int)y2a, (int)y2b, (int)(lh ? q0.z : q0.x), (int)(lh ? q0.w : q0.y)};
#pragma unroll
            for (int a = 0; a < TM; ++a) {
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(v8bf, A0[a]), __builtin_bit_cast(v8bf, B0), acc[a][b], 0, 0, 0);
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(v8bf, A1[a]), __builtin_bit_cast(v8bf, B1), acc[a][b], 0, 0, 0);
            }
        }
    }
}

// Max / sum over the 32 lanes of each wavefront half, result in all of them:
// DPP within 16-lane rows, then one swap of the row pairs.
__device__ __forceinline__ float half_max(float v)
{
    v = fmaxf(v, dpp_move<0xb1>(v));
    v = fmaxf(v, dpp_move<0x4e>(v));
    v = fmaxf(v, dpp_move<0x141>(v));
    v = fmaxf(v, dpp_move<0x140>(v));
    return fmaxf(v, __shfl_xor(v, 16));
}
__device__ __forceinline__ int half_sum(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, true);
    return v + __shfl_xor(v, 16);
}

// SiLU(g) * u as the SwiGLU producer computes it (f64 SiLU rounded once,
// f32 product).
__device__ __forceinline__ float swiglu1(float g, float u)
{
    const double g64 = (double)g;
    return (float)(g64 / (1.0 + exp(-g64))) * u;
}

// Plain: out (or a split-K partial plane) = the f32 result. FFN (W = gate,
// W2 = up, tiles of 64 output columns): y = SiLU(g) * u per output, written
// as its int8 plane qo / do_ / so (and y itself when y != nullptr).
template <bool FFN, bool DSC>
__global__ __launch_bounds__(NTHR, MQ_Q4K_OCC) void gemm_q4k_kernel(
    const uint8_t *__restrict__ W, const uint8_t *__restrict__ W2, const Dsc dsc, const int8_t *__restrict__ q,
    const float *__restrict__ dx, const float *__restrict__ sx, int M, int N,
    int K, int tiles_m, int nsplit, float *__restrict__ out, int8_t *__restrict__ qo,
    float *__restrict__ do_, float *__restrict__ so)
{
    __shared__ Stage S0, S1;
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
    const int n0 = tile_n * (FFN ? BN / 2 : BN);
    const WRows rows{W, W2, n0, N, (int64_t)(K >> 8) * BLK_BYTES};
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: DMA bases in SGPRs
    const int wm = wave % WM, wn = wave / WM;
    const int lr = lane & 31, lh = lane >> 5;

    v16f acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[a][b][v] = 0.0f;

    // The step range is even (whole super-blocks): steps alternate S0, S1.
    Side p;
    issue_tiles<FFN>(S0, rows, q, M, K, t0, st_begin, wave, lane);
    load_side<FFN, DSC>(p, rows, dsc, dx, sx, M, K, t0, st_begin);
    wait_vm<0>();
    store_side<FFN, DSC>(S0, p, rows, st_begin, M, t0);
    __syncthreads();
    for (int st = st_begin; st < st_end; st += 2) {
        issue_tiles<FFN>(S1, rows, q, M, K, t0, st + 1, wave, lane);
        load_side<FFN, DSC>(p, rows, dsc, dx, sx, M, K, t0, st + 1);
        compute_step<0>(S0, acc, wm, wn, lr, lh);
        wait_vm<0>();
        store_side<FFN, DSC>(S1, p, rows, st + 1, M, t0);
        __syncthreads();
        const bool more = st + 2 < st_end;
        if (more) {
            issue_tiles<FFN>(S0, rows, q, M, K, t0, st + 2, wave, lane);
            load_side<FFN, DSC>(p, rows, dsc, dx, sx, M, K, t0, st + 2);
        }
        compute_step<1>(S1, acc, wm, wn, lr, lh);
        if (more) {
            wait_vm<0>();
            store_side<FFN, DSC>(S0, p, rows, st + 2, M, t0);
        }
        __syncthreads();
    }

    if constexpr (FFN) {
        static_assert(TM == 1 && TN == 4 && WN == 1, "gate|up tiles: b and b + 2 share columns");
        // y for (token t, column n): tiles b = 0, 1 hold g, tiles b + 2 the u of
        // the same columns. A 32-value block of the plane is one tile row:
        // lanes lr = 0..31 of one half (lh) at one v, combined across lanes.
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int n = n0 + 32 * b + lr;
            float y[16];
#pragma unroll
            for (int v = 0; v < 16; ++v)
                y[v] = swiglu1(acc[0][b][v], acc[0][b + 2][v]);
            float amax[16];
#pragma unroll
            for (int v = 0; v < 16; ++v)
                amax[v] = fabsf(y[v]);
#pragma unroll
            for (int v = 0; v < 16; ++v)
                amax[v] = half_max(amax[v]);
            float db[16], rdb[16], qf[16];
            bool slow = false;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                db[v] = q_scale(amax[v]);
                rdb[v] = q_recip(db[v]);
                const bool zero = db[v] == 0.0f;
                const float t = y[v] * rdb[v];
                const float r = __builtin_rintf(t);
                slow |= !zero && (db[v] < 0x1p-100f || q_near_half(t, r));
                qf[v] = fminf(fmaxf(r, -127.0f), 127.0f);
            }
            if (__any(slow)) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const bool zero = db[v] == 0.0f;
                    const float t = y[v] * rdb[v];
                    if (!zero && (db[v] < 0x1p-100f || q_near_half(t, __builtin_rintf(t))))
                        qf[v] = q_clamp_round(y[v] / db[v]);
                }
            }
            int sum[16];
#pragma unroll
            for (int v = 0; v < 16; ++v)
                sum[v] = (int)qf[v];
#pragma unroll
            for (int v = 0; v < 16; ++v)
                sum[v] = half_sum(sum[v]);
            if (n < N) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int t = t0 + wm * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                    if (t < M) {
                        qo[(int64_t)t * N + n] = (int8_t)(int)qf[v];
                        if (out)
                            out[(int64_t)t * N + n] = y[v];
                        if (lr == 0) {
                            const int64_t blk = (int64_t)t * (N >> 5) + (n >> 5);
                            do_[blk] = db[v];
                            so[blk] = db[v] * (float)sum[v];
                        }
                    }
                }
            }
        }
        return;
    }
#pragma unroll
    for (int a = 0; a < TM; ++a) {
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const int n = n0 + (wn * TN + b) * 32 + lr;
            if (n < N) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int t = t0 + (wm * TM + a) * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                    if (t < M)
                        dst[(int64_t)t * N + n] = acc[a][b][v];
                }
            }
        }
    }
}

} // namespace

namespace {
// K ranges of a launch (see gemm_splits); tiles of BM x BN outputs
int nsplit_for(int M, int N, int K)
{
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return gemm_splits(tiles, BM * BN, K >> 8, M, N, K, Q4K_SLOT_OPS);
}
} // namespace

#if MQ_Q5K && defined(MQ_Q4K_SMALL)
int splits_gemm_q5k_small(int M, int N, int K) { return nsplit_for(M, N, K); }
hipError_t launch_gemm_q5k_small(const uint8_t *W, const int8_t *q, const float *d,
                                 const float *s, int M, int N, int K, float *out,
                                 const Ws &ws, hipStream_t st)
#elif MQ_Q5K
int splits_gemm_q5k(int M, int N, int K) { return nsplit_for(M, N, K); }
hipError_t launch_gemm_q5k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           const Ws &ws, hipStream_t st)
#elif defined(MQ_Q4K_SMALL)
int splits_gemm_q4k_small(int M, int N, int K) { return nsplit_for(M, N, K); }
hipError_t launch_gemm_q4k_small(const uint8_t *W, const int8_t *q, const float *d,
                                 const float *s, int M, int N, int K, float *out,
                                 const Ws &ws, hipStream_t st)
#else
int splits_gemm_q4k(int M, int N, int K) { return nsplit_for(M, N, K); }
hipError_t launch_gemm_q4k(const uint8_t *W, const int8_t *q, const float *d,
                           const float *s, int M, int N, int K, float *out,
                           const Ws &ws, hipStream_t st)
#endif
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int nsplit = ws.ptr ? nsplit_for(M, N, K) : 1;
    return run_split_k(nsplit, (int64_t)M * N, out, ws, st, [&](float *dst) {
        launch(gemm_q4k_kernel<false, false>, dim3((unsigned)(tiles * nsplit)), dim3(NTHR), 0, st, 
            W, nullptr, Dsc{nullptr, nullptr}, q, d, s, M, N, K, tiles_m, nsplit, dst, nullptr, nullptr, nullptr);
        return hipGetLastError();
    });
}

#if !MQ_Q5K
#ifdef MQ_Q4K_SMALL
hipError_t launch_gemm_q4k_dsc_small(const uint8_t *W, const float *fw, const float *fm, const int8_t *q,
                                     const float *d, const float *s, int M, int N, int K, float *out,
                                     const Ws &ws, hipStream_t st)
#else
hipError_t launch_gemm_q4k_dsc(const uint8_t *W, const float *fw, const float *fm, const int8_t *q,
                               const float *d, const float *s, int M, int N, int K, float *out,
                               const Ws &ws, hipStream_t st)
#endif
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int nsplit = ws.ptr ? nsplit_for(M, N, K) : 1;
    return run_split_k(nsplit, (int64_t)M * N, out, ws, st, [&](float *dst) {
        launch(gemm_q4k_kernel<false, true>, dim3((unsigned)(tiles * nsplit)), dim3(NTHR), 0, st, 
            W, nullptr, Dsc{fw, fm}, q, d, s, M, N, K, tiles_m, nsplit, dst, nullptr, nullptr, nullptr);
        return hipGetLastError();
    });
}
#endif

#if !defined(MQ_Q4K_SMALL) && !MQ_Q5K
hipError_t launch_gemm_q4k_ffn(const uint8_t *Wg, const uint8_t *Wu, const int8_t *q, const float *d,
                               const float *s, int M, int N, int K, int8_t *qo, float *do_, float *so,
                               float *y, hipStream_t st)
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN / 2 - 1) / (BN / 2);
    launch(gemm_q4k_kernel<true, false>, dim3((unsigned)(tiles_m * tiles_n)), dim3(NTHR), 0, st, 
        Wg, Wu, Dsc{nullptr, nullptr}, q, d, s, M, N, K, tiles_m, 1, y, qo, do_, so);
    return hipGetLastError();
}
#endif

} // namespace mq
