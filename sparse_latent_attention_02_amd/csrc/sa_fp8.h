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

// Block rounding of one 16-byte chunk (8 bf16) whose 32-value block is spread
// over lanes 4k..4k+3 of the wavefront; every lane of the wavefront must call it
// (the block amax is reduced across the four lanes).  e[] receives the chunk's
// values on the e4m3fn grid (before the scale), the return value is the scale.
__device__ __forceinline__ float fp8_block_round(u32x4_t w, float e[8]) {
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
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = e4m3_round(v[i] / scale);
    return scale;
}

// fp8 round trip of one chunk: the rounded values times the scale, back in bf16
// (exact: an e4m3fn value times a power of two)
__device__ __forceinline__ u32x4_t fp8_round_trip_chunk(u32x4_t w) {
    float e[8];
    const float scale = fp8_block_round(w, e);
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(e[2 * i] * scale, e[2 * i + 1] * scale);
    return o;
}

// ---- fp8-resident KV rows: e4m3fn codes plus one E8M0 scale byte per block ----

// OCP e4m3fn code of a value already on the e4m3fn grid (|q| <= 448), from its
// f32 fields: sign, exponent rebiased from 127 to 7, the top 3 mantissa bits;
// below 2^-6 the code is the subnormal count q / 2^-9 (exact).
__device__ __forceinline__ uint32_t e4m3_code(float q) {
    const uint32_t u = __float_as_uint(q);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a < 0x3c800000u) return sign | (uint32_t)(__uint_as_float(a) * 512.0f);
    return sign | (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);
}

// Codes of one chunk (8 bytes, value i in byte i) and its block's scale byte
// (the f32 biased exponent of the power-of-two scale, which is its E8M0 code).
// Same lane contract as fp8_block_round.
__device__ __forceinline__ u32x2_t fp8_pack_chunk(u32x4_t w, uint32_t &scale_byte) {
    float e[8];
    const float scale = fp8_block_round(w, e);
    scale_byte = __float_as_uint(scale) >> 23;
    u32x2_t c;
#pragma unroll
    for (int j = 0; j < 2; ++j)
        c[j] = e4m3_code(e[4 * j]) | (e4m3_code(e[4 * j + 1]) << 8) | (e4m3_code(e[4 * j + 2]) << 16) |
               (e4m3_code(e[4 * j + 3]) << 24);
    return c;
}

// 8 codes of one block (byte i = value i) at scale 2^(scale_byte - 127) -> 8 bf16,
// with the gfx950 scaled conversion (exact: each value is an e4m3fn value times a
// power of two well inside the bf16 range).  scale_byte must lie in [1, 254].
__device__ __forceinline__ u32x4_t kv8_expand(u32x2_t c, uint32_t scale_byte) {
    const float sc = __uint_as_float(scale_byte << 23);
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        o[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j], sc, false));
        o[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j], sc, true));
    }
    return o;
}

}  // namespace sa
