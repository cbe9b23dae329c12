// Prefill GEMM for Q4_K weights on the fp8 matrix cores (gfx950).
//
// The pages' prefill multiplies the raw 4-bit quants with the int8
// activation plane on the tensor cores and applies the block scales after
// each integer sub-block product (minfer Features, "GPU — CUDA": raw-nibble
// int8 GEMMs for q4_K and q6_K). The result per token t and row n is
//     out[t,n] = sum_j  d_x[t,j] * (d*sc_j)[n] * I_j  -  s_x[t,j] * (dmin*m_j)[n],
//     I_j = sum over the 32 values i of sub-block j of  q4[n,i] * q[t,i]   (exact integer).
// On gfx950 the int8 matrix cores return I_j as an int32, and the f32
// epilogue then converts it, forms the scale product and adds: three VALU
// operations per token, row and sub-block, which bound that design. This
// kernel takes the same exact products through the scaled fp8 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4), which returns I_j as an f32, so the
// epilogue is the scale product and one fused multiply-add.
//
// Exact fp8 operands. The e4m3 codes 0..15 are the values 0..15 * 2^-9
// (the subnormals and the first binade share the step 2^-9), so a 4-bit
// quant zero-extended to a byte is its own e4m3 operand, and a per-block
// E8M0 scale of 2^9 restores the integer. The int8 activation q is biased
// to u = q + 128 in 0..255 and split into two base-16 digits,
// u = 16*uh + ul. One MFMA of K = 64 takes, for each of the sub-block's 32
// positions, the digit uh in the first 32-value K block (E8M0 scale 2^13:
// 16 * 2^9) and ul in the second (2^9), against the same quants in both
// blocks: its f32 result is sum_i q4*u = I_j + 128*W_j exactly (every
// partial sum is an integer below 2^24), W_j = sum_i q4 the row's quant sum
// over the sub-block. The bias 128*W_j*d_x*fw is removed with the min term.
//
// Terms.
//   * sub-block product: acc += (I_j + 128 W_j) * (d_x[t,j] * fw[n,j]):
//     a product and a fused multiply-add per output (VALU);
//   * min term and bias: -sum_j s_x[t,j]*fm[n,j] + d_x[t,j]*(128 fw W)[n,j],
//     a rank-4 contraction per step on the bf16 matrix cores, from
//     three-limb splits of every factor (f32 accuracy; two MFMAs per tile).
//
// Tiling. A 256-thread workgroup computes 128 tokens x 128 rows; wavefront
// w owns tokens 32w..32w+31 and all 128 rows (four 32x32 tiles). K moves in
// steps of 64 (two sub-blocks, one 32-byte run of a block's quant bytes).
// Activations arrive by global->LDS DMA; each row's 32 quant bytes pass
// through registers, where they are unpacked to one byte per quant (once
// per workgroup, not per wavefront) and summed, then stored to LDS with the
// step's scale factors and min-term records. The LDS holds three stages:
// the loads of step s + 2 are in flight while step s is computed (a step's
// compute alone does not cover a load from HBM), with one barrier per step.
//
// MFMA layouts (32x32 outputs): lane l holds output column l%32 (a weight
// row) and rows 8(v/4) + 4(l/32) + v%4 (tokens). fp8 32x32x64: lane l
// supplies row / column l%32 and, in bytes 0..15, positions 16(l/32)..+15
// of K block 0, in bytes 16..31 the same positions of K block 1; the E8M0
// scale of a row's K block b is taken from lane row + 32b. bf16 32x32x16:
// lane l supplies K slots 8(l/32)..+7.
#include "mq_device.h"
#include "mq_launch.h"

namespace mq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int NTHR = 256;
constexpr int NSTAGE = 3;
constexpr int BLK = 144;                      // Q4_K super-block bytes
constexpr int A_CHUNKS = BM * BK / 16;        // 16-byte activation chunks per step
constexpr int VM_PER_STEP = A_CHUNKS / NTHR + 4;   // vector-memory ops a thread issues per step
// int8-equivalent ops per second of one resident workgroup, for the split-K
// choice (about 600 TOPS over 512 resident workgroups)
constexpr double SLOT_OPS = 1.2e12;
// E8M0 scales 2^(e - 127) of the fp8 operands (codes 0..15 = 0..15 * 2^-9)
constexpr int SCALE_HI = 127 + 13;            // activation high digit: 16 * 2^9
constexpr int SCALE_LO = 127 + 9;             // activation low digit
constexpr int SCALE_W = 127 + 9;              // quants

// One step's tiles. Activation chunk c (values 16c..16c+15 of the step) of
// token r sits in 16-byte slot a_slot(r, c). Quants of sub-block jj (0: low
// nibbles, 1: high nibbles of the step's 32 bytes) as bytes: row n,
// positions 16g..16g+15 in slot g*BN + n (16 consecutive rows of one half
// are 256 consecutive bytes: no bank conflicts). The min-term records hold
// bf16 limbs (bf16_limbs3) of the contraction over the terms
//     0, 1: s_x(j0), s_x(j1)  x  -fm(j0), -fm(j1)
//     2, 3: d_x(j0), d_x(j1)  x  -128 fw W(j0), -128 fw W(j1)
// as mt0 / mr0 = {x1 t0t1, x1 t2t3, x2 t0t1, x2 t2t3} and mt1 / mr1 =
// {x3 t0t1, x3 t2t3} per token / row. dx, fw: the f32 factors of the
// sub-block products.
struct alignas(16) Stage {
    int8_t a[A_CHUNKS * 16];
    uint8_t w[2][BN * 32];
    uint4 mt0[BM];
    uint4 mr0[BN];
    uint2 mt1[BM];
    uint2 mr1[BN];
    float dx[2][BM];
    float fw[2][BN];
};
static_assert(2 * NSTAGE * sizeof(Stage) <= 160 * 1024, "two workgroups per CU");

// 16 consecutive tokens reading the same chunk hit 16 different 16-byte
// bank groups (a row is 64 bytes: rows r and r + 4 start on the same banks,
// so the chunk is permuted by bits 2..3 of the row).
__device__ __forceinline__ int a_slot(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// DMA of step st's activations (token rows past M read the last token).
__device__ __forceinline__ void issue_act(Stage &s, const int8_t *__restrict__ q, int M, int K, int t0, int st,
                                          int wave, int lane)
{
#pragma unroll
    for (int ii = 0; ii < A_CHUNKS / NTHR; ++ii) {
        const int i = wave * (A_CHUNKS / NTHR) + ii;
        const int p = 64 * i + lane;
        const int r = p >> 2;
        const int c = (p & 3) ^ ((r >> 2) & 3);
        const int t = min(t0 + r, M - 1);
        dma16(q + (int64_t)t * K + (int64_t)st * BK + 16 * c, s.a + 1024 * i);
    }
}

// What a thread loads for a step: thread tid covers weight row n0 + tid/2
// (half tid&1 of its 32 quant bytes, and the block header) and token
// t0 + tid/2 (the step's two activation scales and sums). Rows past N and
// tokens past M read the last valid one; their factors are zeroed.
struct Side {
    uint4 raw, hdr;
    float2 sx, dx;
};

__device__ __forceinline__ void load_side(Side &p, const uint8_t *__restrict__ W, const float *__restrict__ dx,
                                          const float *__restrict__ sx, int M, int N, int K, int t0, int n0,
                                          int st)
{
    const int tid = threadIdx.x, rl = tid >> 1, hh = tid & 1;
    const uint8_t *blk = W + (int64_t)min(n0 + rl, N - 1) * ((K >> 8) * BLK) + (int64_t)(st >> 2) * BLK;
    p.hdr = *reinterpret_cast<const uint4 *>(blk);
    p.raw = *reinterpret_cast<const uint4 *>(blk + 16 + 32 * (st & 3) + 16 * hh);
    const int64_t ti = (int64_t)min(t0 + rl, M - 1) * (K >> 5) + 2 * st;
    p.sx = *reinterpret_cast<const float2 *>(sx + ti);
    p.dx = *reinterpret_cast<const float2 *>(dx + ti);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// Each thread writes half of its row's and of its token's data: thread
// hh = tid & 1 takes the terms 2hh, 2hh + 1 of the min-term records and the
// factors of sub-block hh.
__device__ __forceinline__ void store_side(Stage &s, const Side &p, int M, int N, int t0, int n0, int st)
{
    const int tid = threadIdx.x, rl = tid >> 1, hh = tid & 1;
    const bool rok = n0 + rl < N, tok = t0 + rl < M;
    // quants as bytes, and their sums over the thread's 16 positions of
    // each sub-block, then over the row (the partner thread tid ^ 1)
    const uint32_t m4 = 0x0f0f0f0fu;
    const uint4 lo = make_uint4(p.raw.x & m4, p.raw.y & m4, p.raw.z & m4, p.raw.w & m4);
    const uint4 hi = make_uint4((p.raw.x >> 4) & m4, (p.raw.y >> 4) & m4, (p.raw.z >> 4) & m4, (p.raw.w >> 4) & m4);
    *reinterpret_cast<uint4 *>(s.w[0] + 16 * (BN * hh + rl)) = lo;
    *reinterpret_cast<uint4 *>(s.w[1] + 16 * (BN * hh + rl)) = hi;
    const int ones = 0x01010101;
    int w0 = dot4((int)lo.x, ones, dot4((int)lo.y, ones, dot4((int)lo.z, ones, dot4((int)lo.w, ones, 0))));
    int w1 = dot4((int)hi.x, ones, dot4((int)hi.y, ones, dot4((int)hi.z, ones, dot4((int)hi.w, ones, 0))));
    w0 += __builtin_amdgcn_mov_dpp(w0, 0xb1, 0xf, 0xf, false);      // quad_perm [1,0,3,2]: lane ^ 1
    w1 += __builtin_amdgcn_mov_dpp(w1, 0xb1, 0xf, 0xf, false);

    // block header: f16 d, f16 dmin, 6-bit codes; sub-blocks j0 = 2c, j1 = 2c + 1
    // of the super-block, c = st & 3 (codes 0..3 are the low 6 bits of bytes
    // 0..3 / 4..7; codes 4..7 take their low 4 bits from bytes 8..11 and
    // their high 2 bits from the top of bytes 0..3 / 4..7)
    const uint4 h = p.hdr;
    const int c = st & 3;
    const float dd = f16_bits_to_f32(h.x), dm = f16_bits_to_f32(h.x >> 16);
    const uint32_t scw = c < 2 ? (h.y & 0x3f3f3f3fu) : ((h.w & 0x0f0f0f0fu) | ((h.y >> 2) & 0x30303030u));
    const uint32_t mw = c < 2 ? (h.z & 0x3f3f3f3fu) : (((h.w >> 4) & 0x0f0f0f0fu) | ((h.z >> 2) & 0x30303030u));
    const int sh = 16 * (c & 1);
    const float fw0 = dd * (float)((scw >> sh) & 0xffu), fw1 = dd * (float)((scw >> (sh + 8)) & 0xffu);
    const float fm0 = dm * (float)((mw >> sh) & 0xffu), fm1 = dm * (float)((mw >> (sh + 8)) & 0xffu);

    uint32_t a1, a2, a3, b1, b2, b3;
    {   // min-term row record: terms 0, 1 (hh = 0) or 2, 3 (hh = 1)
        const float v0 = hh ? -128.0f * (fw0 * (float)w0) : -fm0;
        const float v1 = hh ? -128.0f * (fw1 * (float)w1) : -fm1;
        bf16_limbs3(rok ? v0 : 0.0f, a1, a2, a3);
        bf16_limbs3(rok ? v1 : 0.0f, b1, b2, b3);
        uint32_t *r0 = reinterpret_cast<uint32_t *>(&s.mr0[rl]);
        r0[hh] = pack2(a1, b1);
        r0[2 + hh] = pack2(a2, b2);
        reinterpret_cast<uint32_t *>(&s.mr1[rl])[hh] = pack2(a3, b3);
        s.fw[hh][rl] = rok ? (hh ? fw1 : fw0) : 0.0f;
    }
    {   // min-term token record: s_x (hh = 0) or d_x (hh = 1) of the two sub-blocks
        const float2 v = hh ? p.dx : p.sx;
        bf16_limbs3(tok ? v.x : 0.0f, a1, a2, a3);
        bf16_limbs3(tok ? v.y : 0.0f, b1, b2, b3);
        uint32_t *r0 = reinterpret_cast<uint32_t *>(&s.mt0[rl]);
        r0[hh] = pack2(a1, b1);
        r0[2 + hh] = pack2(a2, b2);
        reinterpret_cast<uint32_t *>(&s.mt1[rl])[hh] = pack2(a3, b3);
        s.dx[hh][rl] = tok ? (hh ? p.dx.y : p.dx.x) : 0.0f;
    }
}

// One step (two sub-blocks) of wavefront wm's 32 tokens x 128 rows: eight
// tile products k = 4*jj + b (sub-block jj, row tile b), software-pipelined:
// the MFMA of product k + 1 is issued and the LDS operands of product k + 2
// read before the epilogue of product k, so that the matrix cores work
// while the VALU does. Each stage is pinned by a scheduling barrier. wz is
// an opaque zero (see the kernel): the second read of each quant chunk, at
// wz + the same address, cannot be merged with the first, so the chunk
// lands in both halves of the fp8 operand without register copies.
struct Ops {
    v4i w0, w1;
    float fw;
};

__device__ __forceinline__ void compute_step(const Stage &s, v16f (&acc)[4], int wm, int lr, int lh, int wz)
{
    const int tr = wm * 32 + lr;
    const int sa = lh ? SCALE_LO : SCALE_HI;
    const uint8_t *wbase = reinterpret_cast<const uint8_t *>(&s.w[0][0]) + 16 * (BN * lh + lr);
    auto read_ops = [&](int k, Ops &o) {
        const int jj = k >> 2, b = k & 3;
        const uint8_t *pw = wbase + jj * (BN * 32) + b * 512;
        o.w0 = *reinterpret_cast<const v4i *>(pw);
        o.w1 = *reinterpret_cast<const v4i *>(pw + wz);
        o.fw = s.fw[jj][b * 32 + lr];
    };
    auto act = [&](int jj, v8i &A) {
        const v4i qa = *reinterpret_cast<const v4i *>(s.a + 16 * a_slot(tr, 2 * jj + lh));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            A[e] = ((qa[e] >> 4) & 0x0f0f0f0f) ^ 0x08080808;   // high digit of q + 128
            A[4 + e] = qa[e] & 0x0f0f0f0f;                      // low digit
        }
    };
    // the 16 token scales of the lane's outputs (tokens wm*32 + 8(v/4) +
    // 4 lh + v%4) of each sub-block
    float dv[2][16];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const float4 d4 = *reinterpret_cast<const float4 *>(&s.dx[jj][wm * 32 + 8 * g4 + 4 * lh]);
            dv[jj][4 * g4] = d4.x;
            dv[jj][4 * g4 + 1] = d4.y;
            dv[jj][4 * g4 + 2] = d4.z;
            dv[jj][4 * g4 + 3] = d4.w;
        }
    v8i A[2];
    Ops ops[2];
    v16f I[2];
    float fwk[2];
    auto mfma = [&](int k) {
        const Ops &o = ops[k & 1];
        const v8i B = {o.w0.x, o.w0.y, o.w0.z, o.w0.w, o.w1.x, o.w1.y, o.w1.z, o.w1.w};
        I[k & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[k >> 2], B, v16f{}, 0, 0, 0, sa, 0, SCALE_W);
        fwk[k & 1] = o.fw;                    // o is refilled before product k's epilogue
    };
    act(0, A[0]);
    read_ops(0, ops[0]);
    read_ops(1, ops[1]);
    mfma(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_barrier(0);
        if (k + 1 < 8)
            mfma(k + 1);
        if (k + 2 < 8) {
            if (k + 2 == 4)
                act(1, A[1]);
            read_ops(k + 2, ops[k & 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int b = k & 3;
        const float f = fwk[k & 1];
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[b][v] = fmaf(I[k & 1][v], dv[k >> 2][v] * f, acc[b][v]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // min term and bias: two bf16 MFMAs per tile. K slot 8*lh + e pairs
    // element e of the A and B operands; lane half 0 carries x1*y1, x1*y2
    // (first MFMA) and x2*y2, x3*y1 (second), lane half 1 x2*y1, x1*y3 and
    // x2*y3, x3*y2, for the four terms each.
    const uint4 r0 = s.mt0[tr];
    const uint2 r1 = s.mt1[tr];
    const v4i A0 = v4i{(int)(lh ? r0.z : r0.x), (int)(lh ? r0.w : r0.y), (int)r0.x, (int)r0.y};
    const v4i A1 = v4i{(int)r0.z, (int)r0.w, (int)r1.x, (int)r1.y};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int n = b * 32 + lr;
        const uint4 q0 = s.mr0[n];
        const uint2 q1 = s.mr1[n];
        const uint32_t y2a = lh ? q1.x : q0.z, y2b = lh ? q1.y : q0.w;   // y2 | y3
        const v4i B0 = {(int)q0.x, (int)q0.y, (int)y2a, (int)y2b};
        const v4i B1 = {(int)y2a, (int)y2b, (int)(lh ? q0.z : q0.x), (int)(lh ? q0.w : q0.y)};
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, A0), __builtin_bit_cast(v8bf, B0),
                                                         acc[b], 0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, A1), __builtin_bit_cast(v8bf, B1),
                                                         acc[b], 0, 0, 0);
    }
}

__global__ __launch_bounds__(NTHR, 2) void gemm_q4k_f8_kernel(const uint8_t *__restrict__ W,
                                                             const int8_t *__restrict__ q,
                                                             const float *__restrict__ dx,
                                                             const float *__restrict__ sx, int M, int N, int K,
                                                             int tiles_m, int nsplit, float *__restrict__ out)
{
    __shared__ Stage S[NSTAGE];
    // blockIdx = split * tiles + tile; split s of nsplit covers the
    // super-blocks [s*P/nsplit, (s+1)*P/nsplit) of P = K/256 and, when
    // nsplit > 1, writes its partial sums to out + s*M*N.
    const int tiles = gridDim.x / nsplit;
    const int split = blockIdx.x / tiles;
    const int tile = blockIdx.x - split * tiles;
    int tile_m, tile_n;
    tile_order(tile, tiles_m, tiles / tiles_m, tile_m, tile_n);
    const int nsb = K >> 8;
    const int st_begin = 4 * (int)((int64_t)split * nsb / nsplit);
    const int st_end = 4 * (int)((int64_t)(split + 1) * nsb / nsplit);
    float *dst = out + (int64_t)split * M * N;
    const int t0 = tile_m * BM, n0 = tile_n * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    int wz;                                   // 0, opaque to the compiler
    asm volatile("s_mov_b32 %0, 0" : "=s"(wz));

    v16f acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[b][v] = 0.0f;

    // Step st lives in stage st % NSTAGE. The loads of step st + 2 are
    // issued before step st is computed (into the stage step st - 1 used,
    // which the previous barrier freed); after the compute, the loads of
    // step st + 1 (all but the VM_PER_STEP most recent operations) are
    // complete and it is stored, and one barrier publishes it. The step
    // range holds at least 4 steps (one super-block).
    Side pa, pb;                              // side loads of the even and the odd steps
    issue_act(S[st_begin % NSTAGE], q, M, K, t0, st_begin, wave, lane);
    load_side(pa, W, dx, sx, M, N, K, t0, n0, st_begin);
    issue_act(S[(st_begin + 1) % NSTAGE], q, M, K, t0, st_begin + 1, wave, lane);
    load_side(pb, W, dx, sx, M, N, K, t0, n0, st_begin + 1);
    wait_vm<VM_PER_STEP>();
    store_side(S[st_begin % NSTAGE], pa, M, N, t0, n0, st_begin);
    __syncthreads();
    // step st: mine = the side loads of st's parity (refilled with st + 2),
    // next = those of st + 1
    auto step = [&](int st, Side &mine, Side &next) {
        const bool pre = st + 2 < st_end;
        if (pre) {
            issue_act(S[(st + 2) % NSTAGE], q, M, K, t0, st + 2, wave, lane);
            load_side(mine, W, dx, sx, M, N, K, t0, n0, st + 2);
        }
        compute_step(S[st % NSTAGE], acc, wave, lr, lh, wz);
        if (st + 1 < st_end) {
            if (pre)
                wait_vm<VM_PER_STEP>();
            else
                wait_vm<0>();
            store_side(S[(st + 1) % NSTAGE], next, M, N, t0, n0, st + 1);
        }
        __syncthreads();
    };
    for (int st = st_begin; st < st_end; st += 2) {   // st_begin is even, the range a multiple of 4
        step(st, pa, pb);
        step(st + 1, pb, pa);
    }

#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int n = n0 + b * 32 + lr;
        if (n < N) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = t0 + wave * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                if (t < M)
                    dst[(int64_t)t * N + n] = acc[b][v];
            }
        }
    }
}

int nsplit_for(int M, int N, int K)
{
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return gemm_splits(tiles, BM * BN, K >> 8, M, N, K, SLOT_OPS);
}

} // namespace

int splits_gemm_q4k_f8(int M, int N, int K) { return nsplit_for(M, N, K); }

hipError_t launch_gemm_q4k_f8(const uint8_t *W, const int8_t *q, const float *d, const float *s, int M, int N,
                              int K, float *out, const Ws &ws, hipStream_t st)
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int nsplit = ws.ptr ? nsplit_for(M, N, K) : 1;
    return run_split_k(nsplit, (int64_t)M * N, out, ws, st, [&](float *dst) {
        launch(gemm_q4k_f8_kernel, dim3((unsigned)(tiles * nsplit)), dim3(NTHR), 0, st, W, q, d, s, M, N, K,
               tiles_m, nsplit, dst);
        return hipGetLastError();
    });
}

} // namespace mq
