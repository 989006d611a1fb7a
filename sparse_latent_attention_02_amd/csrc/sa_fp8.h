// sa_fp8.h -- fp8 (OCP e4m3) round trip of bf16 values on the device.
//
// "Module attn" rustdoc (DeepSeek-V4.1 reference), act_quant_inplace and
// pow2_ceil: per block of 32 contiguous values, scale = power-of-two ceiling of
// amax / 448 with amax floored at 1e-4, values rounded to e4m3 (nearest, ties
// to even, clamped) at that scale, dequantised and stored back as bf16.  The
// "Precision" paragraph of the same page: the result is bf16-exact.
//
// Layout: four lanes per 32-value block, each lane one 16-byte chunk (8 bf16),
// so a wavefront covers 1 KiB of a row; the block amax is a two-step lane
// reduction.
#pragma once

#include "sa_device.h"

namespace sa {

// 2^ceil(log2 v) for a positive normal f32 from its IEEE fields: exact powers of
// two are kept, otherwise the exponent goes up by one and the mantissa clears.
__device__ __forceinline__ float pow2_ceil_ieee(float v) {
    uint32_t u = __float_as_uint(v);
    if (u & 0x007fffffu) u = ((u >> 23) + 1u) << 23;
    return __uint_as_float(u);
}

// Nearest OCP e4m3fn value (3 mantissa bits, bias 7, subnormal spacing 2^-9,
// largest finite 448), ties to even, clamped to +-448.  Below 2^-6 the grid is
// uniform (k * 2^-9): scale up by 2^9 (exact), round to an integer with
// round-half-even, scale back.  From 2^-6 up the f32 mantissa is cut to its top 3
// bits with round-half-even on the 20 dropped bits (a carry moves into the
// exponent, which is the right neighbour).
__device__ __forceinline__ float e4m3_round(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = u & 0x80000000u;
    uint32_t a = u & 0x7fffffffu;
    float r;
    if (__uint_as_float(a) < 0.015625f) {
        r = rintf(__uint_as_float(a) * 512.0f) * (1.0f / 512.0f);
    } else {
        a = (a + 0x7ffffu + ((a >> 20) & 1u)) & 0xfff00000u;
        r = fminf(__uint_as_float(a), 448.0f);
    }
    return __uint_as_float(__float_as_uint(r) | sign);
}

// fp8 round trip of one 16-byte chunk (8 bf16) whose 32-value block is spread
// over lanes 4k..4k+3 of the wavefront; every lane of the wavefront must call
// it (the block amax is reduced across the four lanes).
__device__ __forceinline__ u32x4_t fp8_round_trip_chunk(u32x4_t w) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, 1e-4f);
    const float scale = pow2_ceil_ieee(amax / 448.0f);
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2(e4m3_round(v[2 * i] / scale) * scale, e4m3_round(v[2 * i + 1] / scale) * scale);
    return o;
}

}  // namespace sa
