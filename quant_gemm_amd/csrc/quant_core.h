// Per-32 int8 quantization of values already in registers, shared by the
// activation quantizer and the producer-fused kernels of libmq.
//
// Rule (mq.h, mq_quantize_act): for each 32-value block, amax = max |v|,
// d = amax / 127 (IEEE f32 division), q = d == 0 ? 0 : clamp(roundf(v / d),
// -127, 127) with roundf rounding halves away from zero, s = d * (float)sum(q).
//
// Layout: lane li (0..7) of an 8-lane group holds values 4 li .. 4 li + 3 of
// a block, one float4 per chunk; groups are aligned (lanes 8 g .. 8 g + 7 of
// a wavefront) and all 8 lanes of a group are active. A lane may hold NC
// chunks (NC blocks, each with its own group). The chunks are processed
// stage by stage (all amax exchanges, then all scales, ...) so that their
// latencies overlap.
//
// Group exchanges use DPP moves inside the 8 lanes (quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], then row_half_mirror, which pairs lane i of the group
// with lane 7 - i of the other quad), so max and sum reach all 8 lanes
// without a trip through the LDS crossbar.
//
// The scale. With R = f32(1/127), q0 = f32(amax * R) and
// d = fma(fma(-q0, 127, amax), R, q0) (the remainder of q0 against amax,
// exact in the inner fma, corrects q0 once): d equals the IEEE quotient
// amax / 127 for every non-negative finite f32 amax, subnormals included
// (checked by enumerating all of them on the host). Non-finite inputs are
// outside the rule (their output is unspecified).
//
// The quotient. rdb = 1/d from the hardware reciprocal refined by one
// Newton step, within 2^-23 relative of 1/d. With |v| <= 127.0001 d (v lies
// in d's block), t = f32(v * rdb) is within 127.0001 * (2^-23 + 2^-24) <
// 2.3e-5 of v / d and f32(v / d) within 127.0001 * 2^-24 < 7.6e-6 of it, so
// t and the IEEE quotient are less than 3.1e-5 apart: unless t is within
// 6e-5 of a half-integer (the only rounding boundaries of roundf), both round
// to the same integer, and there round-to-nearest-even (rint) agrees with
// roundf. Those rare values, and blocks with d < 2^-100 (where rdb could
// overflow or d lose relative precision), take the IEEE division and roundf
// in a separate, wave-uniform pass.
//
// sum(q): the codes are integers of magnitude at most 127, so the per-lane
// sums and the group total (at most 32 * 127) are exact in f32.
#pragma once

#include "mq_device.h"

#pragma clang fp contract(off)

namespace mq {

__device__ __forceinline__ float q_clamp_round(float t)
{
    float r = __builtin_roundf(t);
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    return r;
}

// Max / sum over the aligned 8-lane group of the calling lane. The max is
// taken on the bits of non-negative floats, whose unsigned order is the
// numeric order.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
}

__device__ __forceinline__ uint32_t group8_umax(uint32_t a)
{
    a = max(a, dpp_u32<0xb1>(a));          // quad_perm [1,0,3,2]
    a = max(a, dpp_u32<0x4e>(a));          // quad_perm [2,3,0,1]
    return max(a, dpp_u32<0x141>(a));      // row_half_mirror
}

__device__ __forceinline__ float group8_sum(float a)
{
    a += dpp_move<0xb1>(a);
    a += dpp_move<0x4e>(a);
    return a + dpp_move<0x141>(a);
}

// Distance of t from its nearest integer r beyond which t may round
// differently from the IEEE quotient it approximates.
constexpr float Q_NEAR_HALF = 0.5f - 6e-5f;

// True when t = f32(v * rdb) may round differently from the IEEE quotient
// v / d it approximates (r = rint(t); t - r is exact: |t| < 2^7 and r is the
// nearest integer).
__device__ __forceinline__ bool q_near_half(float t, float r)
{
    return fabsf(t - r) > Q_NEAR_HALF;
}

// d = amax / 127 as the IEEE quotient (see above), for finite amax >= 0.
__device__ __forceinline__ float q_scale(float amax)
{
    constexpr float R = 1.0f / 127.0f;
    const float q0 = amax * R;
    return __builtin_fmaf(__builtin_fmaf(-q0, 127.0f, amax), R, q0);
}

// rdb for the fast quotient: 1/d within 2^-23 relative (0 when d == 0).
__device__ __forceinline__ float q_recip(float d)
{
    const float r0 = __builtin_amdgcn_rcpf(d);
    return d == 0.0f ? 0.0f : __builtin_fmaf(__builtin_fmaf(-d, r0, 1.0f), r0, r0);
}

// v[c]: this lane's 4 values of chunk c. Outputs per chunk: qp = the 4 int8
// codes packed little-endian; d and s of the chunk's block (the same in all
// 8 lanes of its group).
//
// Fast path: q = rint(t) with no clamp (|t| <= 127.00003, so |q| <= 127).
// Whether any value of the wavefront needs the IEEE pass is decided once,
// from the largest |t - rint(t)| (a block with d < 2^-100 counts as 1; a
// block with d == 0 has t == 0).
template <int NC>
__device__ __forceinline__ void quant_chunks(const float4 (&v)[NC], uint32_t (&qp)[NC], float (&d)[NC],
                                             float (&s)[NC])
{
    float rdb[NC];
    float qf[NC][4];
    float dev = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const float a = fmaxf(fmaxf(fabsf(v[c].x), fabsf(v[c].y)), fmaxf(fabsf(v[c].z), fabsf(v[c].w)));
        const uint32_t am = group8_umax(__builtin_bit_cast(uint32_t, a));
        d[c] = q_scale(__builtin_bit_cast(float, am));
        rdb[c] = q_recip(d[c]);
        const float e[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float t = e[i] * rdb[c];
            qf[c][i] = __builtin_rintf(t);
            m = fmaxf(m, fabsf(t - qf[c][i]));
        }
        const bool tiny = d[c] < 0x1p-100f && d[c] != 0.0f;
        dev = fmaxf(dev, tiny ? 1.0f : m);
    }
    if (__any(dev > Q_NEAR_HALF)) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const bool zero = d[c] == 0.0f;
            const float e[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float t = e[i] * rdb[c];
                if (!zero && (d[c] < 0x1p-100f || q_near_half(t, __builtin_rintf(t))))
                    qf[c][i] = q_clamp_round(e[i] / d[c]);
            }
        }
    }
    float sum[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int q0 = (int)qf[c][0], q1 = (int)qf[c][1], q2 = (int)qf[c][2], q3 = (int)qf[c][3];
        qp[c] = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) | ((uint32_t)(q2 & 0xff) << 16) |
                ((uint32_t)(q3 & 0xff) << 24);
        sum[c] = group8_sum((qf[c][0] + qf[c][1]) + (qf[c][2] + qf[c][3]));
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
        s[c] = d[c] * sum[c];
}

} // namespace mq
