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
#include "sa_fp8.h"
#include "../../include/sparse_attn.h"

namespace {

using namespace sa;

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

// fp8-resident KV rows: thread per 16-byte chunk (8 values); the 8 codes go to
// codes[t * 8 ..], the first lane of each block writes its scale byte into the
// row's 16-byte scale record (unused record bytes are set to 127, scale 2^0).
__global__ void __launch_bounds__(256) kv8_pack_kernel(const uint16_t *__restrict__ x, uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales, int64_t n_chunks,
                                                       int32_t chunks_per_row) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = t < n_chunks;
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (live) w = *reinterpret_cast<const u32x4_t *>(x + t * 8);
    uint32_t sb;
    const u32x2_t c = fp8_pack_chunk(w, sb);
    if (!live) return;
    *reinterpret_cast<u32x2_t *>(codes + t * 8) = c;
    const int64_t row = t / chunks_per_row;
    const int32_t k = (int32_t)(t % chunks_per_row);
    if ((k & 3) == 0) scales[row * SA_KV8_SCALE_BYTES + k / 4] = (uint8_t)sb;
    if (k == 0)
        for (int j = chunks_per_row / 4; j < SA_KV8_SCALE_BYTES; ++j) scales[row * SA_KV8_SCALE_BYTES + j] = 127;
}

__global__ void __launch_bounds__(256) kv8_unpack_kernel(const uint8_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales,
                                                         uint16_t *__restrict__ x, int64_t n_chunks,
                                                         int32_t chunks_per_row) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_chunks) return;
    const int64_t row = t / chunks_per_row;
    const int32_t k = (int32_t)(t % chunks_per_row);
    const u32x2_t c = *reinterpret_cast<const u32x2_t *>(codes + t * 8);
    *reinterpret_cast<u32x4_t *>(x + t * 8) = kv8_expand(c, scales[row * SA_KV8_SCALE_BYTES + k / 4]);
}

}  // namespace

extern "C" sa_status sa_act_quant_fp8_inplace(uint16_t *x, int64_t n_rows, int32_t row_len,
                                              void *stream) {
    if (n_rows < 0 || row_len <= 0 || row_len % 32 != 0 || !mul_le(n_rows, row_len / 8, 0x7fffffffLL * 256))
        return SA_ERR_SHAPE;
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

static sa_status kv8_args(int64_t n_rows, int32_t row_len) {
    if (n_rows < 0 || row_len <= 0 || row_len % 32 != 0 || !mul_le(n_rows, row_len / 8, 0x7fffffffLL * 256))
        return SA_ERR_SHAPE;
    if (row_len > 32 * SA_KV8_SCALE_BYTES) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

extern "C" sa_status sa_kv8_pack(const uint16_t *x, uint8_t *codes, uint8_t *scales, int64_t n_rows,
                                 int32_t row_len, void *stream) {
    sa_status st = kv8_args(n_rows, row_len);
    if (st != SA_OK || n_rows == 0) return st;
    if (!x || !codes || !scales) return SA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(codes) | reinterpret_cast<uintptr_t>(scales)) %
        16)
        return SA_ERR_SHAPE;
    const int64_t n_chunks = n_rows * (row_len / 8);
    const int64_t blocks = (n_chunks + 255) / 256;
    if (blocks > 0x7fffffff) return SA_ERR_SHAPE;
    hipLaunchKernelGGL(kv8_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, x, codes, scales,
                       n_chunks, row_len / 8);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

extern "C" sa_status sa_kv8_unpack(const uint8_t *codes, const uint8_t *scales, uint16_t *x, int64_t n_rows,
                                   int32_t row_len, void *stream) {
    sa_status st = kv8_args(n_rows, row_len);
    if (st != SA_OK || n_rows == 0) return st;
    if (!x || !codes || !scales) return SA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(codes) | reinterpret_cast<uintptr_t>(scales)) %
        16)
        return SA_ERR_SHAPE;
    const int64_t n_chunks = n_rows * (row_len / 8);
    const int64_t blocks = (n_chunks + 255) / 256;
    if (blocks > 0x7fffffff) return SA_ERR_SHAPE;
    hipLaunchKernelGGL(kv8_unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, codes, scales,
                       x, n_chunks, row_len / 8);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}
