// sa_index.hip -- index-list builders of the sparse attention path.
//
//  * window slot lists: "DeepSeek V4.1 ... attention / attend", get_window_topk_idxs
//    (prefill: one causal window per query into the chunk; decode: the ring oldest
//    first, -1 for slots not yet written);
//  * compressed-index append: "DeepSeek V4.1 ... attention / query-latent",
//    Attention.forward (window and compressed lists concatenated along topk) and
//    the Indexer tail (reachable positions shifted by the window-row count,
//    unreachable ones -1).
// Integer fills: a grid of (column chunks) x (rows), four consecutive entries
// per thread, written as one 16-byte store when the row layout allows it;
// memory bound and small next to the attention itself.
#include "sa_device.h"
#include "../../include/sparse_attn.h"

#include <algorithm>

namespace {

using namespace sa;

// entries j0 .. j0 + 3 (those < cols) of row `row` at out_row, vectorised when `vec`
__device__ __forceinline__ void store4(int32_t *out_row, int32_t j0, int32_t cols, bool vec, i32x4_t v) {
    if (vec) {
        *reinterpret_cast<i32x4_t *>(out_row + j0) = v;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (j0 + i < cols) out_row[j0 + i] = v[i];
    }
}

// grid: x = chunks of 4 columns, y = query rows (strided), z = batch (strided)
__global__ void window_idx_kernel(int32_t *__restrict__ out, int32_t bsz, int32_t nrows, int32_t cols,
                                  int64_t row_stride, int32_t window, int64_t start_pos, bool vec) {
    const int32_t j0 = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (j0 >= cols) return;
    // decode: the ring listed oldest first, starting one past the newest slot
    const int32_t oldest = start_pos > 0 ? (int32_t)(start_pos % window + 1) : 0;
    for (int32_t b = blockIdx.z; b < bsz; b += gridDim.z) {
        for (int32_t r = blockIdx.y; r < nrows; r += gridDim.y) {
            i32x4_t v;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t j = j0 + i;
                int64_t slot, newest;
                if (start_pos == 0) {
                    // causal window of the chunk ending at query r
                    slot = (r - window + 1 > 0 ? r - window + 1 : 0) + j;
                    newest = r;
                } else {
                    const int32_t s = oldest + j;   // < 2 window
                    slot = s >= window ? s - window : s;
                    newest = start_pos;
                }
                v[i] = slot > newest ? -1 : (int32_t)slot;
            }
            store4(out + ((int64_t)b * nrows + r) * row_stride, j0, cols, vec, v);
        }
    }
}

// grid: x = chunks of 4 compressed columns, y = rows (strided)
__global__ void append_idx_kernel(int32_t *__restrict__ out, int64_t row_stride, int32_t col0,
                                  const int32_t *__restrict__ cidx, int64_t n_rows, int32_t kc,
                                  int32_t offset, bool vec) {
    const int32_t j0 = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (j0 >= kc) return;
    for (int64_t r = blockIdx.y; r < n_rows; r += gridDim.y) {
        const int32_t *crow = cidx + r * kc;
        i32x4_t c;
        if (vec) {
            c = *reinterpret_cast<const i32x4_t *>(crow + j0);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) c[i] = j0 + i < kc ? crow[j0 + i] : -1;
        }
        i32x4_t v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = c[i] < 0 ? -1 : c[i] + offset;
        store4(out + r * row_stride + col0, j0, kc, vec, v);
    }
}

constexpr int kIdxThreads = 256;
constexpr int64_t kMaxGridYZ = 65535;

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
    if (bsz < 0 || row_stride < cols || !mul_le((int64_t)bsz * nrows, cols, 0x7fffffffLL * 256)) return SA_ERR_SHAPE;
    const int64_t n_out = (int64_t)bsz * nrows * cols;
    if (n_out == 0) return SA_OK;
    if (!idx) return SA_ERR_NULL;
    const bool vec = row_stride % 4 == 0 && cols % 4 == 0 && reinterpret_cast<uintptr_t>(idx) % 16 == 0;
    const unsigned gx = (unsigned)((((int64_t)cols + 3) / 4 + kIdxThreads - 1) / kIdxThreads);
    const dim3 grid(gx, (unsigned)std::min<int64_t>(nrows, kMaxGridYZ), (unsigned)std::min<int64_t>(bsz, kMaxGridYZ));
    hipLaunchKernelGGL(window_idx_kernel, grid, dim3(kIdxThreads), 0, (hipStream_t)stream, idx, bsz, nrows, cols,
                       row_stride, window, start_pos, vec);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

extern "C" sa_status sa_append_compressed_idxs(int32_t *idx, int64_t row_stride, int32_t col0,
                                               const int32_t *cidx, int64_t n_rows, int32_t kc,
                                               int32_t offset, void *stream) {
    if (n_rows < 0 || kc < 0 || col0 < 0 || offset < 0 || row_stride < (int64_t)col0 + kc ||
        !mul_le(n_rows, kc, 0x7fffffffLL * 256))
        return SA_ERR_SHAPE;
    const int64_t n_out = n_rows * kc;
    if (n_out == 0) return SA_OK;
    if (!idx || !cidx) return SA_ERR_NULL;
    const bool vec = row_stride % 4 == 0 && col0 % 4 == 0 && kc % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(idx) % 16 == 0 && reinterpret_cast<uintptr_t>(cidx) % 16 == 0;
    const unsigned gx = (unsigned)((((int64_t)kc + 3) / 4 + kIdxThreads - 1) / kIdxThreads);
    const dim3 grid(gx, (unsigned)std::min<int64_t>(n_rows, kMaxGridYZ));
    hipLaunchKernelGGL(append_idx_kernel, grid, dim3(kIdxThreads), 0, (hipStream_t)stream, idx, row_stride, col0,
                       cidx, n_rows, kc, offset, vec);
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
