// Device-side helpers shared by the gfx950 kernels of libmq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// IEEE binary16 bits -> f32 (exact, subnormals included: f16 denormals are
// kept on gfx9).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

// 16 bytes read once (streamed): a nontemporal load, which on MI355X keeps a
// cold sweep of HBM from allocating in the caches. Measured on a 47.5 MB
// activation plane read cold: 12.5 us with this hint, about twice that with
// plain loads.
__device__ __forceinline__ float4 ld_stream_f4(const float *p)
{
    const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}

// Signed 4-way int8 dot product with int32 accumulate (v_dot4_i32_i8).
__device__ __forceinline__ int dot4(int a, int b, int c)
{
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// v from another lane, moved by a DPP pattern (lanes the pattern leaves
// without a source, or whose row is masked off, receive 0).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_move(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, true));
}

// Sum over the 64 lanes of a wavefront with DPP moves (no LDS crossbar);
// every lane receives the total. Pairs, quads, half-rows and rows of 16 are
// folded within each row, then rows 0+1 and 2+3 and finally all four rows
// are combined through the row broadcasts, leaving the sum in lane 63.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_move<0xb1>(v);          // quad_perm [1,0,3,2]
    v += dpp_move<0x4e>(v);          // quad_perm [2,3,0,1]
    v += dpp_move<0x141>(v);         // row_half_mirror
    v += dpp_move<0x140>(v);         // row_mirror
    v += dpp_move<0x142, 0xa>(v);    // row_bcast:15 into rows 1 and 3
    v += dpp_move<0x143, 0xc>(v);    // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// bf16 bits (round to nearest even) of x.
__device__ __forceinline__ uint32_t bf16_bits(float x)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// Three bf16 limbs of x: x = x1 + x2 + x3 up to 2^-27 relative, each limb
// the nearest bf16 of what the previous ones left. Products of limbs are
// exact in the f32 accumulation of the bf16 matrix cores, so a sum of the
// limb products other than the smallest ones carries an f32 product's
// accuracy.
__device__ __forceinline__ void bf16_limbs3(float x, uint32_t &x1, uint32_t &x2, uint32_t &x3)
{
    x1 = bf16_bits(x);
    const float r = x - __builtin_bit_cast(float, x1 << 16);
    x2 = bf16_bits(r);
    x3 = bf16_bits(r - __builtin_bit_cast(float, x2 << 16));
}

// The 4*n bytes at a 2-byte aligned address p, as n dwords, using only
// aligned dword loads. When p is 2 mod 4 the loads also cover the 2 bytes
// before p and the 2 bytes after p + 4n: callers keep [p - 2, p + 4n + 2)
// inside one allocation.
template <int n>
__device__ __forceinline__ void load_dwords_a2(const uint8_t *p, uint32_t (&out)[n])
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t *base = reinterpret_cast<const uint32_t *>(a & ~uintptr_t(3));
    const uint32_t sh = (uint32_t)(a & 3u);   // 0 or 2
    uint32_t w[n + 1];
#pragma unroll
    for (int i = 0; i < n; ++i)
        w[i] = base[i];
    w[n] = sh ? base[n] : 0u;
#pragma unroll
    for (int i = 0; i < n; ++i)
        out[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
}

// One 16-byte global->LDS DMA per lane (global_load_lds_dwordx4): lane L's
// 16 bytes land at LDS byte address lds_dst + 16 * L, where lds_dst must be
// wave-uniform and 16-byte aligned, src 16-byte aligned. Issued as inline asm
// so that the compiler neither waits for it at the next LDS access nor
// reorders LDS accesses around it; completion is awaited with wait_vm(). The
// instruction takes its LDS address from M0, which the compiler may hold a
// value in: the asm saves it and puts it back.
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

// One 4-byte global->LDS DMA per lane (global_load_lds_dword): lane L's
// dword lands at LDS byte address lds_dst + 4 * L (lds_dst wave-uniform and
// 4-byte aligned, src 4-byte aligned). As dma16 otherwise.
__device__ __forceinline__ void dma4(const void *src, const void *lds_dst)
{
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds_dst);
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %2\n\t"
                 "global_load_lds_dword %1, off\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(src), "s"(base)
                 : "memory");
}

// Tile order of the GEMMs. Workgroups are handed to the 8 XCDs in turn
// (workgroup b to XCD b % 8), and each XCD has its own L2. b is renumbered
// so that each XCD walks one contiguous range of the tile sequence, and the
// sequence runs in bands of MQ_TILE_GROUP token tiles: within a band
// consecutive tiles step through its token tiles first, then through the
// weight panels. The workgroups an XCD holds at once then share one band of
// activation rows (4 x 128 tokens of K int8) in its L2 while the weight
// panels stream past, instead of every XCD streaming the whole activation
// plane for each panel. Measured on MI355X (rocprofv3 FETCH_SIZE, bytes
// fetched past L2, at 3314 x 18944 x 3584): 570 MiB per launch in the plain
// order, 302 with bands of 8 token tiles, 251 with 4, 277 with bands of 8
// weight panels instead; the time moved by under 2%, since the kernel is
// bound by its VALU. A bijection of [0, tiles_m * tiles_n); MQ_TILE_GROUP = 0
// keeps the plain order (token tile fastest).
#ifndef MQ_TILE_GROUP
#define MQ_TILE_GROUP 4
#endif
__device__ __forceinline__ void tile_order(int b, int tiles_m, int tiles_n, int &tile_m, int &tile_n)
{
    if (MQ_TILE_GROUP <= 0) {
        tile_m = b % tiles_m;
        tile_n = b / tiles_m;
        return;
    }
    constexpr int X = 8;                          // XCDs
    const int T = tiles_m * tiles_n;
    const int per = T / X, extra = T % X;
    const int x = b % X, l = b / X;
    const int g = x * per + min(x, extra) + l;     // XCD x: [x per + min(x, extra), + per + (x < extra))
    const int first = g / (MQ_TILE_GROUP * tiles_n) * MQ_TILE_GROUP;
    const int gm = min(tiles_m - first, MQ_TILE_GROUP);
    const int r = g - first * tiles_n;             // in [0, gm * tiles_n)
    tile_n = r / gm;
    tile_m = first + r % gm;
}

// Wait until at most N vector memory operations of this wavefront are
// outstanding. Loads complete in issue order, so with N = the number of
// loads issued after some load L, L has completed (any stores in between
// only make the wait longer).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

} // namespace mq
