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

__global__ void __launch_bounds__(256) act_quant_kernel(uint16_t *__restrict__ x, int64_t n_chunks) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // lanes past the end take part in the block reduction on a zero chunk
    const bool live = t < n_chunks;
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (live) w = *reinterpret_cast<const u32x4_t *>(x + t * 8);
    const u32x4_t o = fp8_round_trip_chunk(w);
    if (live) *reinterpret_cast<u32x4_t *>(x + t * 8) = o;
}

// Fused fp8 round trip + ring-cache write of a chunk of new KV rows.  Row t of
// the chunk (position start_pos + t) is rounded through fp8 in place and, when it
// is among the chunk's last `window` rows, also copied to ring slot
// (start_pos + t) % window -- the layout the "Module attn" rustdoc ring-cache
// worked example fixes (12 tokens into 8 slots leave slots 4..7 = tokens 4..7,
// slots 0..3 = tokens 8..11; decode step 12 writes slot 4).
__global__ void __launch_bounds__(256) window_kv_update_kernel(uint16_t *__restrict__ ring,
                                                               uint16_t *__restrict__ rows,
                                                               int64_t n_chunks, int32_t chunks_per_row,
                                                               int32_t seqlen, int32_t window,
                                                               int64_t ring_stride, int64_t start_pos) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = t < n_chunks;
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (live) w = *reinterpret_cast<const u32x4_t *>(rows + t * 8);
    const u32x4_t o = fp8_round_trip_chunk(w);
    if (!live) return;
    *reinterpret_cast<u32x4_t *>(rows + t * 8) = o;
    const int64_t row = t / chunks_per_row;        // (batch, chunk row)
    const int32_t c = (int32_t)(t % chunks_per_row);
    const int32_t tr = (int32_t)(row % seqlen);     // row within the chunk
    const int64_t bi = row / seqlen;
    if (tr < seqlen - window) return;               // overwritten later in the same chunk
    const int64_t slot = (start_pos + tr) % window;
    *reinterpret_cast<u32x4_t *>(ring + ((bi * ring_stride + slot) * chunks_per_row + c) * 8) = o;
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

extern "C" sa_status sa_window_kv_update(uint16_t *ring, int64_t ring_stride, uint16_t *rows, int32_t bsz,
                                         int32_t window, int32_t d, int64_t start_pos, int32_t seqlen,
                                         void *stream) {
    if (bsz < 0 || window <= 0 || d <= 0 || d % 32 != 0 || seqlen < 0 || start_pos < 0 || ring_stride < window)
        return SA_ERR_SHAPE;
    if (start_pos > 0 && seqlen != 1) return SA_ERR_UNSUPPORTED;
    const int64_t n_chunks = (int64_t)bsz * seqlen * (d / 8);
    if (n_chunks == 0) return SA_OK;
    if (!ring || !rows) return SA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(ring) | reinterpret_cast<uintptr_t>(rows)) % 16 != 0) return SA_ERR_SHAPE;
    const int threads = 256;
    const int64_t blocks = (n_chunks + threads - 1) / threads;
    if (blocks > 0x7fffffff) return SA_ERR_SHAPE;
    hipLaunchKernelGGL(window_kv_update_kernel, dim3((unsigned)blocks), dim3(threads), 0, (hipStream_t)stream,
                       ring, rows, n_chunks, d / 8, seqlen, window, ring_stride, start_pos);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}
