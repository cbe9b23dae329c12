// Per-32 int8 quantization of values already in registers, shared by the
// activation quantizer and the producer-fused kernels of libmq.
//
// Rule (mq.h, mq_quantize_act): for each 32-value block, amax = max |v|,
// d = amax / 127 (IEEE f32 division), q = d == 0 ? 0 : clamp(roundf(v / d),
// -127, 127) with roundf rounding halves away from zero, s = d * (float)sum(q).
//
// Layout: lane li (0..7) of an 8-lane group holds values 4 li .. 4 li + 3 of
// a block, one float4 per chunk; a lane may hold NC chunks (NC blocks, each
// with its own group). The chunks are processed stage by stage (all amax
// shuffles, then all scales, ...) so that their latencies overlap.
//
// The quotient. With rdb = f32(1 / d) and |v| <= 127.0001 d (v lies in d's
// block), t = f32(v * rdb) is within 127.0001 * (2^-23 + 2^-48) < 1.52e-5 of
// v / d and f32(v / d) within 127.0001 * 2^-24 < 7.6e-6 of it, so t and the
// IEEE quotient are less than 2.3e-5 apart: unless t is within 3e-5 of a
// half-integer (the only rounding boundaries of roundf), both round to the
// same integer. Those rare values, and blocks with d < 2^-100 (where rdb
// could overflow), take the IEEE division in a separate, wave-uniform pass.
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

// True when t may round differently from the IEEE quotient it approximates.
__device__ __forceinline__ bool q_near_half(float t)
{
    const float a = fabsf(t);
    return fabsf((a - floorf(a)) - 0.5f) < 3e-5f;
}

// v[c]: this lane's 4 values of chunk c. Outputs per chunk: qp = the 4 int8
// codes packed little-endian; d and s of the chunk's block (the same in all
// 8 lanes of its group).
template <int NC>
__device__ __forceinline__ void quant_chunks(const float4 (&v)[NC], uint32_t (&qp)[NC], float (&d)[NC],
                                             float (&s)[NC])
{
    float amax[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        amax[c] = fmaxf(fmaxf(fabsf(v[c].x), fabsf(v[c].y)), fmaxf(fabsf(v[c].z), fabsf(v[c].w)));
#pragma unroll
    for (int m = 1; m < 8; m <<= 1)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            amax[c] = fmaxf(amax[c], __shfl_xor(amax[c], m, 8));
    float rdb[NC];
    float qf[NC][4];
    bool slow = false;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        d[c] = amax[c] / 127.0f;
        const bool zero = d[c] == 0.0f;
        rdb[c] = zero ? 0.0f : 1.0f / d[c];
        const float e[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float t = e[i] * rdb[c];
            slow |= !zero && (d[c] < 0x1p-100f || q_near_half(t));
            qf[c][i] = q_clamp_round(t);
        }
    }
    if (__any(slow)) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const bool zero = d[c] == 0.0f;
            const float e[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float t = e[i] * rdb[c];
                if (!zero && (d[c] < 0x1p-100f || q_near_half(t)))
                    qf[c][i] = q_clamp_round(e[i] / d[c]);
            }
        }
    }
    int sum[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int q0 = (int)qf[c][0], q1 = (int)qf[c][1], q2 = (int)qf[c][2], q3 = (int)qf[c][3];
        qp[c] = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) | ((uint32_t)(q2 & 0xff) << 16) |
                ((uint32_t)(q3 & 0xff) << 24);
        sum[c] = q0 + q1 + q2 + q3;
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            sum[c] += __shfl_xor(sum[c], m, 8);
#pragma unroll
    for (int c = 0; c < NC; ++c)
        s[c] = d[c] * (float)sum[c];
}

} // namespace mq
