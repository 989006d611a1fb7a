// sa_quant.hip -- fp8 (OCP e4m3) round trip of bf16 KV rows, in place.
//
// "Module attn" rustdoc (DeepSeek-V4.1 reference), act_quant_inplace and
// pow2_ceil: per block of 32 contiguous values, scale = power-of-two ceiling of
// amax / 448 with amax floored at 1e-4, values rounded to e4m3 (nearest, ties
// to even, clamped) at that scale, dequantised and stored back as bf16.  The
// "Precision" paragraph of the same page: the result is bf16-exact.
//
// Layout: four lanes per 32-value block, each lane one 16-byte chunk (8 bf16),
// so a wavefront reads and writes 1 KiB contiguous; the block amax is a
// two-step lane reduction.  HBM bound: 2 bytes read + 2 written per value.
#include "sa_device.h"
#include "../../include/sparse_attn.h"

namespace {

using namespace sa;

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

__global__ void __launch_bounds__(256) act_quant_kernel(uint16_t *__restrict__ x, int64_t n_chunks) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // every lane takes part in the block reduction; lanes past the end idle on a zero chunk
    const bool live = t < n_chunks;
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (live) w = *reinterpret_cast<const u32x4_t *>(x + t * 8);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // the four chunks of a block sit in lanes 4k..4k+3
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, 1e-4f);
    const float scale = pow2_ceil_ieee(amax / 448.0f);
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = e4m3_round(v[2 * i] / scale) * scale;
        const float b = e4m3_round(v[2 * i + 1] / scale) * scale;
        o[i] = pack_bf16x2(a, b);
    }
    if (live) *reinterpret_cast<u32x4_t *>(x + t * 8) = o;
}

}  // namespace

extern "C" sa_status sa_act_quant_fp8_inplace(uint16_t *x, int64_t n_rows, int32_t row_len,
                                              void *stream) {
    if (n_rows < 0 || row_len <= 0 || row_len % 32 != 0) return SA_ERR_SHAPE;
    if (n_rows == 0) return SA_OK;
    if (!x) return SA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return SA_ERR_SHAPE;
    const int64_t n_chunks = n_rows * (row_len / 8);
    const int threads = 256;  // multiple of 4: a block never straddles two workgroups
    const int64_t blocks = (n_chunks + threads - 1) / threads;
    if (blocks > 0x7fffffff) return SA_ERR_SHAPE;
    hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                       (hipStream_t)stream, x, n_chunks);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}
