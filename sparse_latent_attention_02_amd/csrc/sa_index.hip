// sa_index.hip -- index-list builders of the sparse attention path.
//
//  * window slot lists: "DeepSeek V4.1 ... attention / attend", get_window_topk_idxs
//    (prefill: one causal window per query into the chunk; decode: the ring oldest
//    first, -1 for slots not yet written);
//  * compressed-index append: "DeepSeek V4.1 ... attention / query-latent",
//    Attention.forward (window and compressed lists concatenated along topk) and
//    the Indexer tail (reachable positions shifted by the window-row count,
//    unreachable ones -1).
// Integer fills, one thread per output entry; memory bound and negligible next to
// the attention itself.
#include "sa_device.h"
#include "../../include/sparse_attn.h"

namespace {

__global__ void window_idx_kernel(int32_t *__restrict__ out, int64_t n_out, int32_t nrows,
                                  int32_t cols, int64_t row_stride, int32_t window,
                                  int64_t start_pos) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_out) return;
    const int32_t j = (int32_t)(t % cols);
    const int64_t row = t / cols;                 // (batch, query row) flattened
    const int32_t r = (int32_t)(row % nrows);     // query row within the chunk
    int64_t slot, newest;
    if (start_pos == 0) {
        // causal window of the chunk ending at query r
        const int64_t first = r - window + 1 > 0 ? (int64_t)r - window + 1 : 0;
        slot = first + j;
        newest = r;
    } else {
        // ring listed oldest first: one past the newest slot, wrapping around
        slot = (start_pos % window + 1 + j) % window;
        newest = start_pos;
    }
    out[row * row_stride + j] = slot > newest ? -1 : (int32_t)slot;
}

__global__ void append_idx_kernel(int32_t *__restrict__ out, int64_t row_stride, int32_t col0,
                                  const int32_t *__restrict__ cidx, int64_t n_out, int32_t kc,
                                  int32_t offset) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_out) return;
    const int64_t r = t / kc;
    const int32_t j = (int32_t)(t % kc);
    const int32_t c = cidx[t];
    out[r * row_stride + col0 + j] = c < 0 ? -1 : c + offset;
}

}  // namespace

extern "C" sa_status sa_window_topk_idxs_shape(int32_t window, int32_t seqlen, int64_t start_pos,
                                               int32_t *rows, int32_t *cols) {
    if (!rows || !cols) return SA_ERR_NULL;
    if (window <= 0 || seqlen < 0 || start_pos < 0) return SA_ERR_SHAPE;
    if (start_pos == 0) {
        *rows = seqlen;
        *cols = seqlen < window ? seqlen : window;
        return SA_OK;
    }
    if (seqlen != 1) return SA_ERR_UNSUPPORTED;
    *rows = 1;
    *cols = window;
    return SA_OK;
}

extern "C" sa_status sa_window_topk_idxs(int32_t window, int32_t bsz, int32_t seqlen,
                                         int64_t start_pos, int32_t *idx, int64_t row_stride,
                                         void *stream) {
    int32_t nrows = 0, cols = 0;
    sa_status st = sa_window_topk_idxs_shape(window, seqlen, start_pos, &nrows, &cols);
    if (st != SA_OK) return st;
    if (bsz < 0 || row_stride < cols) return SA_ERR_SHAPE;
    const int64_t n_out = (int64_t)bsz * nrows * cols;
    if (n_out == 0) return SA_OK;
    if (!idx) return SA_ERR_NULL;
    const int threads = 256;
    const int64_t blocks = (n_out + threads - 1) / threads;
    if (blocks > 0x7fffffff) return SA_ERR_SHAPE;
    hipLaunchKernelGGL(window_idx_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                       (hipStream_t)stream, idx, n_out, nrows, cols, row_stride, window, start_pos);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

extern "C" sa_status sa_append_compressed_idxs(int32_t *idx, int64_t row_stride, int32_t col0,
                                               const int32_t *cidx, int64_t n_rows, int32_t kc,
                                               int32_t offset, void *stream) {
    if (n_rows < 0 || kc < 0 || col0 < 0 || offset < 0 || row_stride < (int64_t)col0 + kc)
        return SA_ERR_SHAPE;
    const int64_t n_out = n_rows * kc;
    if (n_out == 0) return SA_OK;
    if (!idx || !cidx) return SA_ERR_NULL;
    const int threads = 256;
    const int64_t blocks = (n_out + threads - 1) / threads;
    if (blocks > 0x7fffffff) return SA_ERR_SHAPE;
    hipLaunchKernelGGL(append_idx_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                       (hipStream_t)stream, idx, row_stride, col0, cidx, n_out, kc, offset);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

extern "C" const char *sa_status_string(sa_status status) {
    switch (status) {
        case SA_OK: return "SA_OK";
        case SA_ERR_NULL: return "SA_ERR_NULL";
        case SA_ERR_SHAPE: return "SA_ERR_SHAPE";
        case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
        case SA_ERR_HIP: return "SA_ERR_HIP";
    }
    return "SA_ERR_UNKNOWN";
}
