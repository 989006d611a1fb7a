// sa_rope.hip -- rotary embedding of the last rope_dim values of bf16 rows.
//
// "Module attn" rustdoc (DeepSeek-V4.1 reference), apply_rotary, and
// apply_rotary_emb on the "attention / query-latent" page: adjacent pairs of the
// rotated part are complex numbers, multiplied in f32 by the position's table
// entry (its conjugate for the inverse rotation the attention output gets) and
// written back as bf16.  Elementwise and HBM bound: one thread per pair.
#include "sa_device.h"
#include "../../include/sparse_attn.h"

namespace {

using namespace sa;

__global__ void __launch_bounds__(256) rotary_kernel(uint16_t *__restrict__ x, const float *__restrict__ table,
                                                     int64_t n_pairs, int32_t half, int32_t row_len, int32_t h,
                                                     int64_t s, int64_t start_pos, bool inverse) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_pairs) return;
    const int32_t j = (int32_t)(t % half);
    const int64_t row = t / half;                 // (b, s, h) row
    const int64_t pos = start_pos + (row / h) % s;
    uint32_t *pr = reinterpret_cast<uint32_t *>(x + row * row_len + (row_len - 2 * half) + 2 * j);
    const float2 cs = *reinterpret_cast<const float2 *>(table + (pos * half + j) * 2);
    *pr = rope_pair(*pr, cs.x, cs.y, inverse);
}

}  // namespace

extern "C" sa_status sa_apply_rotary(uint16_t *x, int64_t b, int64_t s, int32_t h, int32_t row_len,
                                     int32_t rope_dim, const float *table, int64_t n_pos, int64_t start_pos,
                                     int32_t inverse, void *stream) {
    if (b < 0 || s < 0 || h < 0 || row_len < 0 || rope_dim < 0 || n_pos < 0 || start_pos < 0) return SA_ERR_SHAPE;
    if (rope_dim % 2 != 0 || rope_dim > row_len || row_len % 2 != 0) return SA_ERR_SHAPE;
    if (!mul_le(b, s, 0x7fffffffLL) || !mul_le(b * s, (int64_t)h * (rope_dim / 2), 0x7fffffffLL * 256))
        return SA_ERR_SHAPE;
    const int64_t n_pairs = b * s * h * (rope_dim / 2);
    if (n_pairs == 0) return SA_OK;
    if (!x || !table) return SA_ERR_NULL;
    if (start_pos + s > n_pos) return SA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(x) % 4) || (reinterpret_cast<uintptr_t>(table) % 8)) return SA_ERR_SHAPE;
    const int threads = 256;
    const int64_t blocks = (n_pairs + threads - 1) / threads;
    if (blocks > 0x7fffffff) return SA_ERR_SHAPE;
    hipLaunchKernelGGL(rotary_kernel, dim3((unsigned)blocks), dim3(threads), 0, (hipStream_t)stream, x, table,
                       n_pairs, rope_dim / 2, row_len, h, s, start_pos, inverse != 0);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}
