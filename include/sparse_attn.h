/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) sparse latent attention library
 * (libsparse_attn.so).
 *
 * The operations are those of DeepSeek-V4.1's sparse latent attention as the
 * following web pages describe them (cited by page title and section):
 *   [ATTEND]  "DeepSeek V4.1 ... attention / attend" -- get_window_topk_idxs,
 *             the sparse_attn kernel and its wrapper.
 *   [QLAT]    "DeepSeek V4.1 ... attention / query-latent" -- Attention.forward
 *             (concatenation of window and compressed indices), Indexer tail.
 *   [ATTN-RS] "Module attn" rustdoc (DeepSeek-V4.1 reference, ratio-0
 *             attention) -- precision contract, ring-cache worked example,
 *             act_quant_inplace, pow2_ceil, sparse_attn, window_topk_idxs,
 *             apply_rotary.
 *   [ROPE]    "DeepSeek V4.1 ... attention / query-latent" -- apply_rotary_emb
 *             and the inverse rotation of the attention output.
 *   [INDEXER] same page, Indexer.forward -- the selection tail.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as uint16_t bit patterns; f32 as float.
 *   - Every tensor pointer is a DEVICE pointer (HIP device memory or memory the
 *     device can address), tensors are dense row-major (C order).  The caller
 *     owns all memory; the library allocates nothing, keeps no pointer after
 *     return and holds no mutable global state, so calls from several host
 *     threads are safe.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously on it; buffers must stay alive until the stream
 *     reaches that point.  Faults during execution surface at the caller's next
 *     synchronisation, not in the return code.
 *   - Return codes are synchronous argument checks plus the launch status:
 *       SA_OK, SA_ERR_NULL (null pointer where the sizes need data),
 *       SA_ERR_SHAPE (negative size, bad stride or block multiple, workspace
 *       too small), SA_ERR_UNSUPPORTED (a case the pages do not define or a
 *       head dim outside {64, 128, 256, 512}), SA_ERR_HIP (a HIP launch
 *       failed).  Nothing is enqueued when a check fails.
 *   - Sizes that make a call empty (zero rows/queries) return SA_OK and enqueue
 *     nothing.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SA_OK = 0,
    SA_ERR_NULL = 1,
    SA_ERR_SHAPE = 2,
    SA_ERR_UNSUPPORTED = 3,
    SA_ERR_HIP = 4
} sa_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *sa_status_string(sa_status status);

/* ------------------------------------------------------------------------
 * Window slot selection -- [ATTEND] get_window_topk_idxs, [ATTN-RS]
 * window_topk_idxs ("([queries][cols], cols)").
 *
 * Host-only shape query.  start_pos == 0 (prefill): rows = seqlen,
 * cols = min(seqlen, window).  start_pos > 0 (decode): rows = 1, cols = window,
 * and seqlen must be 1 (a chunk starting after position 0 is not defined on the
 * pages: SA_ERR_UNSUPPORTED).
 */
sa_status sa_window_topk_idxs_shape(int32_t window, int32_t seqlen, int64_t start_pos,
                                    int32_t *rows, int32_t *cols);

/* Writes the window slot lists into idx (device, int32) laid out
 * [bsz][rows][row_stride]; only the first `cols` entries of each row are
 * written, so the lists can go straight into the leading columns of a wider
 * index buffer (row_stride >= cols, else SA_ERR_SHAPE).
 *   Prefill: query p lists the chunk positions max(0, p-window+1) + j,
 *            j < cols, with -1 where that position is past p.
 *   Decode:  the ring listed oldest first -- slots (start_pos % window + 1 + j)
 *            % window -- with -1 for slots above start_pos (ring still
 *            filling).  The newest token's slot comes last.
 * The same rows are written for every batch element. */
sa_status sa_window_topk_idxs(int32_t window, int32_t bsz, int32_t seqlen, int64_t start_pos,
                              int32_t *idx, int64_t row_stride, void *stream);

/* ------------------------------------------------------------------------
 * Compressed-index concatenation -- [QLAT] Attention.forward concatenates the
 * compressed indices after the window ones; the Indexer tail shifts reachable
 * positions by the window-row count and leaves unreachable ones at -1.
 *
 * For r < n_rows, j < kc:  idx[r*row_stride + col0 + j] =
 *     cidx[r*kc + j] < 0 ? -1 : cidx[r*kc + j] + offset.
 * idx, cidx: device int32.  row_stride >= col0 + kc and offset >= 0, else
 * SA_ERR_SHAPE.  Other columns of idx are left untouched. */
sa_status sa_append_compressed_idxs(int32_t *idx, int64_t row_stride, int32_t col0,
                                    const int32_t *cidx, int64_t n_rows, int32_t kc,
                                    int32_t offset, void *stream);

/* ------------------------------------------------------------------------
 * fp8 round trip -- [ATTN-RS] act_quant_inplace, pow2_ceil, "Precision".
 *
 * x: device bf16 [n_rows][row_len], modified in place.  For every block of 32
 * contiguous values along a row: amax = max|x| floored at 1e-4,
 * scale = 2^ceil(log2(amax / 448)) (f32 quotient, power-of-two ceiling from
 * the IEEE fields), each value rounded to OCP e4m3 (nearest, ties to even,
 * clamped to +-448) at that scale, multiplied back and stored as bf16 (exact:
 * e4m3 times a power of two).  row_len must be a positive multiple of 32 (else
 * SA_ERR_SHAPE).  Bit-exact; idempotent. */
sa_status sa_act_quant_fp8_inplace(uint16_t *x, int64_t n_rows, int32_t row_len, void *stream);

/* ------------------------------------------------------------------------
 * fp8-resident KV rows ("kv8") -- [ATTN-RS] act_quant_inplace and "Precision":
 * after the fp8 round trip each block of 32 values is an e4m3fn value times a
 * power of two, so a row can be held as one e4m3fn byte per value plus one
 * scale byte per block and expanded to exactly the same bf16 values.  Holding
 * the cache this way halves the bytes (and, in the attention kernels, the copy
 * instructions) of every gathered row; the attention results are identical.
 *
 *   codes  [n_rows][row_len]            uint8  OCP e4m3fn codes (sign, 4
 *                                               exponent bits bias 7, 3
 *                                               mantissa bits)
 *   scales [n_rows][SA_KV8_SCALE_BYTES] uint8  E8M0 scale of block j (byte b:
 *                                               scale 2^(b - 127)) in byte j <
 *                                               row_len / 32; the remaining
 *                                               bytes of the record are 127
 *
 * sa_kv8_pack: bf16 rows -> codes + scales, rounding as sa_act_quant_fp8_inplace
 * (the input need not be rounded already).  sa_kv8_unpack: the inverse
 * expansion, bit-identical to the fp8 round trip of the packed input.
 * row_len a multiple of 32 (else SA_ERR_SHAPE) and at most 512
 * (SA_ERR_UNSUPPORTED); every pointer 16-byte aligned (else SA_ERR_SHAPE). */
#define SA_KV8_SCALE_BYTES 16

sa_status sa_kv8_pack(const uint16_t *x, uint8_t *codes, uint8_t *scales, int64_t n_rows, int32_t row_len,
                      void *stream);

sa_status sa_kv8_unpack(const uint8_t *codes, const uint8_t *scales, uint16_t *x, int64_t n_rows,
                        int32_t row_len, void *stream);

/* ------------------------------------------------------------------------
 * Ring-cache update -- [ATTN-RS] ring-cache worked example (12 prefill tokens
 * into 8 slots leave slots 4..7 = tokens 4..7 and slots 0..3 = tokens 8..11;
 * decode step 12 writes slot 4, step 13 slot 5) and "the KV row rounded
 * through fp8 in place" of the module description; [QLAT] Attention.__init__
 * (zero-initialised ring of window_size slots per batch element).
 *
 * rows: device bf16 [bsz][seqlen][d], the new KV rows for positions
 * start_pos .. start_pos+seqlen-1; rounded through fp8 in place exactly as
 * sa_act_quant_fp8_inplace does (prefill attends to the chunk itself).
 * ring: device bf16, batch element b's ring is rows [b*ring_stride, b*ring_stride
 * + window) of a [bsz][ring_stride][d] buffer (ring_stride >= window, so the ring
 * can head a longer per-sequence KV buffer that also holds compressed rows);
 * the chunk's last min(seqlen, window) rows are written to slots
 * (position % window); other slots are untouched.
 * d % 32 == 0 and ring_stride >= window (else SA_ERR_SHAPE); a chunk starting after position 0 must hold
 * one row (else SA_ERR_UNSUPPORTED, as for the window lists).  Decode order: call
 * this before building the window lists and attending, so the ring holds the
 * new token. */
sa_status sa_window_kv_update(uint16_t *ring, int64_t ring_stride, uint16_t *rows, int32_t bsz,
                              int32_t window, int32_t d, int64_t start_pos, int32_t seqlen, void *stream);

/* ------------------------------------------------------------------------
 * Sparse latent attention -- [ATTEND] sparse_attn_kernel / sparse_attn,
 * [ATTN-RS] sparse_attn ("per query and head, softmax over the gathered rows
 * plus the sink (denominator only), all in f32; output bf16").
 *
 *   q    [b][s][h][d]  bf16   queries (already rotated by the caller)
 *   kv   [b][rows][d]  bf16   latent rows, each serving as key and value for
 *                             every head (one row per token, shared by heads)
 *   sink [h]           f32    per-head sink logit
 *   idx  [b][s][topk]  int32  rows of kv[b] that query (b, s) attends to;
 *                             -1 = skip.  A row listed twice counts twice and
 *                             the order within a list does not matter.
 *   out  [b][s][h][d]  bf16   result
 * For each (b, s, head i), with the valid entries t of the query's list:
 *   out = sum_t e^(x_t) kv[idx_t] / (sum_t e^(x_t) + e^(sink_i)),
 *   x_t = scale * <q_i, kv[idx_t]>;
 * a query with no valid entry outputs zeros.  Arithmetic: bf16 products with
 * f32 accumulation, f32 softmax; the attention weights are rounded to bf16 for
 * the weighted sum of rows (the pages' kernel does the same), result rounded to
 * nearest-even bf16.  Agreement with the exact f32 definition: within
 * max(2 bf16 ulp of the result, 1e-2) per element.
 *
 * Index entries outside {-1} U [0, rows) are a caller error; the kernels treat
 * them as -1 (one unsigned compare), so no out-of-bounds access results.
 * scale is always explicit (the pages' default is d^-0.5).
 * d must be one of {64, 128, 256, 512} (SA_ERR_UNSUPPORTED otherwise); h >= 1.
 * topk = 0 is allowed (zeros out).  rows = 0 is allowed only with topk
 * entries all -1.
 *
 * workspace: device scratch of at least sa_sparse_attn_workspace_bytes(b, s, h,
 * d, topk) bytes (may be NULL when that is 0).  The library picks the kernel
 * variant deterministically from (b*s, h, d, topk) and the device's compute-unit
 * count; the workspace holds the f32 partial results of the split-topk decode
 * variant.  Results are deterministic: the same inputs give bitwise identical
 * outputs. */
size_t sa_sparse_attn_workspace_bytes(int64_t b, int64_t s, int32_t h, int32_t d, int32_t topk);

sa_status sa_sparse_attn(const uint16_t *q, const uint16_t *kv, const float *sink,
                         const int32_t *idx, int64_t b, int64_t s, int32_t h, int32_t d,
                         int64_t rows, int32_t topk, float scale, uint16_t *out,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Kernel variants of sa_sparse_attn_ex. */
typedef enum {
    SA_KERNEL_AUTO = 0,
    /* one workgroup of four wavefronts per (query, 64 heads); each wavefront
     * holds 32 heads over the whole head dim and half of every 64-row stage;
     * the list is compacted (-1 entries dropped) first; two stage buffers */
    SA_KERNEL_WIDE = 1,
    /* one workgroup of four wavefronts per (query, 16 heads); 64-row stages,
     * two buffers deep, whose rows the wavefronts split for the scores and
     * whose head dim they split for the weighted sum (decode-sized batches) */
    SA_KERNEL_DECODE = 2,
    /* one workgroup of two wavefronts per (query, 64 heads); each wavefront
     * holds 32 heads over the whole head dim and walks every row of the list in
     * 32-row stages (no merge between wavefronts); under 80 KiB of LDS, so two
     * workgroups share a CU (grids of many workgroups: prefill) */
    SA_KERNEL_PAIR = 3
} sa_kernel;

/* Same operation with the variant forced (for tests and measurement):
 *   kernel in sa_kernel (SA_KERNEL_AUTO = the automatic choice);
 *   splits >= 1: the index list is cut into that many contiguous pieces, each
 *   handled by its own workgroup, and the f32 partial results (running max,
 *   running sum, unnormalised output) are combined by a second kernel through
 *   the workspace; 0 = automatic.  Unknown kernels or negative splits give
 *   SA_ERR_UNSUPPORTED.  The workspace must hold
 *   sa_sparse_attn_workspace_bytes_ex() bytes (16-byte aligned). */
size_t sa_sparse_attn_workspace_bytes_ex(int64_t b, int64_t s, int32_t h, int32_t d, int32_t topk,
                                         int32_t kernel, int32_t splits);

sa_status sa_sparse_attn_ex(const uint16_t *q, const uint16_t *kv, const float *sink,
                            const int32_t *idx, int64_t b, int64_t s, int32_t h, int32_t d,
                            int64_t rows, int32_t topk, float scale, uint16_t *out,
                            void *workspace, size_t workspace_bytes, void *stream,
                            int32_t kernel, int32_t splits);

/* ------------------------------------------------------------------------
 * sa_sparse_attn_ex with no workspace argument and no allocation -- for callers
 * that cannot allocate device memory at the call (code under HIP graph capture,
 * tight serving loops, harnesses that forbid it).
 *
 * Same arguments, variant choice and result (bit for bit) as sa_sparse_attn_ex
 * with kernel and splits as given.  When the variant splits the index list, its
 * f32 partials go to a scratch array of the library's own in device memory,
 * sa_sparse_attn_noalloc_scratch_bytes() (32 MiB) on each device the library
 * runs on, held until the process ends.  A call whose partials need more
 * (sa_sparse_attn_workspace_bytes_ex(b, s, h, d, topk, kernel, splits) above
 * that) returns SA_ERR_SHAPE with nothing enqueued; a call that needs none
 * does not touch the array.  The call makes no hipMalloc, hipFree or other
 * allocating call; the first call on a device looks up the array's address
 * there (SA_ERR_HIP if that fails).
 *
 * Every call on one device shares that device's array, and the kernels of a
 * call use it until they finish: calls whose work overlaps on one device
 * (different streams, or host threads without ordering between their streams)
 * race on it and must be serialised by the caller.  Nothing in the array needs
 * to start at zero; each call writes every partial it reads. */
size_t sa_sparse_attn_noalloc_scratch_bytes(void);

sa_status sa_sparse_attn_noalloc(const uint16_t *q, const uint16_t *kv, const float *sink,
                                 const int32_t *idx, int64_t b, int64_t s, int32_t h, int32_t d,
                                 int64_t rows, int32_t topk, float scale, uint16_t *out, void *stream,
                                 int32_t kernel, int32_t splits);

/* ------------------------------------------------------------------------
 * One decode step in one launch -- [QLAT] Attention.forward at a decode step
 * (the new KV row rounded through fp8 and written into the ring, the window
 * list, the compressed indices concatenated after it, sparse_attn), [ATTEND]
 * get_window_topk_idxs (decode branch), [ATTN-RS] ring-cache worked example.
 *
 * Same result as this sequence of calls, with seqlen = 1 and s = 1:
 *   sa_window_kv_update(kv, rows, kv_new', b, window, d, start_pos, 1)
 *   sa_window_topk_idxs(window, b, 1, start_pos, idx, window + kc)
 *   sa_append_compressed_idxs(idx, window + kc, window, cidx, b, kc, window)
 *   sa_sparse_attn(q, kv, sink, idx, b, 1, h, d, rows, window + kc, scale, out)
 * except that kv_new is read only (kv_new' is a copy that gets rounded): the
 * rounded row goes to ring slot start_pos % window of kv.  The list is built
 * inside the attention kernel, the new row is rounded there and enters the
 * attention from registers, so nothing of the list or the new row makes an
 * extra trip through memory.
 *
 *   q       [b][h][d]      bf16  one query per sequence, at position start_pos
 *   kv      [b][rows][d]   bf16  per sequence: rows [0, window) the ring, rows
 *                                [window, rows) the compressed cache; slot
 *                                start_pos % window is overwritten
 *   kv_new  [b][d]         bf16  this step's latent row before the fp8 round trip
 *   sink    [h]            f32
 *   cidx    [b][kc]        int32 compressed positions (-1 = none); may be NULL
 *                                when kc == 0; entry c addresses kv row window + c
 *   idx_out [b][window+kc] int32 NULL, or receives the concatenated list (what
 *                                the calls above would leave in idx)
 *   out     [b][h][d]      bf16
 * start_pos >= 1 (position 0 is a prefill: SA_ERR_UNSUPPORTED); window >= 1;
 * rows >= window; d in {64, 128, 256, 512}; kc >= 0.  Pointers of bf16 data
 * 16-byte aligned (else SA_ERR_SHAPE).  Tolerance, determinism and the index
 * rules are those of sa_sparse_attn.  Of kv, only row start_pos % window of
 * each sequence is written.
 *
 * kernel, splits: as for sa_sparse_attn_ex (0, 0 = automatic).  workspace: at
 * least sa_sparse_attn_decode_step_workspace_bytes(b, h, d, window, kc, kernel,
 * splits) bytes, 16-byte aligned (may be NULL when that is 0). */
size_t sa_sparse_attn_decode_step_workspace_bytes(int64_t b, int32_t h, int32_t d, int32_t window, int32_t kc,
                                                  int32_t kernel, int32_t splits);

sa_status sa_sparse_attn_decode_step(const uint16_t *q, uint16_t *kv, const uint16_t *kv_new,
                                     const float *sink, const int32_t *cidx, int32_t *idx_out,
                                     int64_t b, int32_t h, int32_t d, int64_t rows, int32_t window,
                                     int32_t kc, int64_t start_pos, float scale, uint16_t *out,
                                     void *workspace, size_t workspace_bytes, void *stream,
                                     int32_t kernel, int32_t splits);

/* ------------------------------------------------------------------------
 * Prefill with the list built in the attention kernel -- [QLAT]
 * Attention.forward at position 0 (the window list of the chunk, the
 * compressed indices concatenated after it, sparse_attn), [ATTEND]
 * get_window_topk_idxs (prefill branch).
 *
 * Same result as these calls, with wcols = min(s, window):
 *   sa_window_topk_idxs(window, b, s, 0, idx, wcols + kc)
 *   sa_append_compressed_idxs(idx, wcols + kc, wcols, cidx, b * s, kc, s)
 *   sa_sparse_attn(q, kv, sink, idx, b, s, h, d, rows, wcols + kc, scale, out)
 * without the list's trip through memory: each workgroup of the pair kernel
 * builds its query's list in LDS (query t takes chunk rows max(0, t - window +
 * 1) + j while <= t, then cidx entries + s).  The chunk's rows must already hold their fp8 round
 * trip (sa_window_kv_update on the chunk, or sa_act_quant_fp8_inplace).
 *
 *   q       [b][s][h][d]     bf16  the chunk's queries, positions 0 .. s-1
 *   kv      [b][rows][d]     bf16  per sequence: rows [0, s) the chunk, rows
 *                                  [s, rows) the compressed cache
 *   sink    [h]              f32
 *   cidx    [b][s][kc]       int32 compressed positions (-1 = none); may be NULL
 *                                  when kc == 0; entry c addresses kv row s + c
 *   idx_out [b][s][wcols+kc] int32 NULL, or receives the concatenated list (what
 *                                  the calls above would leave in idx)
 *   out     [b][s][h][d]     bf16
 * window >= 1; rows >= s; d in {64, 128, 256, 512}; kc >= 0.  Pointers of
 * bf16 data 16-byte aligned (else SA_ERR_SHAPE).  Tolerance, determinism and
 * the index rules are those of sa_sparse_attn; entries outside [0, rows) are
 * skipped like -1.
 *
 * kernel: 0 or SA_KERNEL_PAIR (the pair kernel builds this list; any other
 * value: SA_ERR_UNSUPPORTED); splits: as for sa_sparse_attn_ex (0 = automatic).
 * workspace: at least sa_sparse_attn_prefill_step_workspace_bytes(b, s, h, d,
 * window, kc, kernel, splits) bytes, 16-byte aligned (may be NULL when that is
 * 0). */
size_t sa_sparse_attn_prefill_step_workspace_bytes(int64_t b, int64_t s, int32_t h, int32_t d, int32_t window,
                                                   int32_t kc, int32_t kernel, int32_t splits);

sa_status sa_sparse_attn_prefill_step(const uint16_t *q, const uint16_t *kv, const float *sink,
                                      const int32_t *cidx, int32_t *idx_out, int64_t b, int64_t s, int32_t h,
                                      int32_t d, int64_t rows, int32_t window, int32_t kc, float scale,
                                      uint16_t *out, void *workspace, size_t workspace_bytes, void *stream,
                                      int32_t kernel, int32_t splits);

/* ------------------------------------------------------------------------
 * Sparse latent attention over fp8-resident rows -- the operation of
 * sa_sparse_attn and sa_sparse_attn_decode_step with the latent rows held as
 * kv8 codes + scale records (layout as for sa_kv8_pack) instead of bf16:
 *
 *   kv_codes  [b][rows][d]                  uint8
 *   kv_scales [b][rows][SA_KV8_SCALE_BYTES] uint8
 *
 * Each gathered row is expanded in LDS to exactly the bf16 values
 * sa_kv8_unpack gives, so the output is bitwise that of sa_sparse_attn_ex
 * (kernel SA_KERNEL_DECODE, same splits) on the unpacked rows.  The rows are
 * read by the decode kernel only (it walks lists of any length; splits as for
 * sa_sparse_attn_ex, 0 = automatic).  The decode step writes the new row's
 * codes and scale record into ring slot start_pos % window of kv_codes /
 * kv_scales: exactly what sa_kv8_pack stores for kv_new, whose expansion is
 * the fp8 round trip of kv_new (the row the bf16 step writes).  (Packing that
 * rounded row again can give other codes for the same values: a block whose
 * amax rounds up onto 448 times a power of two gets half the scale.)  Nothing
 * else of kv_codes / kv_scales is written.  Codes and scale records must come
 * from sa_kv8_pack or an earlier decode step: a scale byte of 0 or 255 is a
 * caller error (its rows expand to unspecified values, no out-of-bounds access
 * results).  Every pointer of bf16 or kv8 data 16-byte aligned (else
 * SA_ERR_SHAPE); the other rules are those of the bf16 entry points.
 * workspace: sa_sparse_attn_kv8_workspace_bytes(b, s, h, d, topk, splits)
 * bytes (for the decode step s = 1, topk = window + kc). */
size_t sa_sparse_attn_kv8_workspace_bytes(int64_t b, int64_t s, int32_t h, int32_t d, int32_t topk,
                                          int32_t splits);

sa_status sa_sparse_attn_kv8(const uint16_t *q, const uint8_t *kv_codes, const uint8_t *kv_scales,
                             const float *sink, const int32_t *idx, int64_t b, int64_t s, int32_t h,
                             int32_t d, int64_t rows, int32_t topk, float scale, uint16_t *out,
                             void *workspace, size_t workspace_bytes, void *stream, int32_t splits);

sa_status sa_sparse_attn_decode_step_kv8(const uint16_t *q, uint8_t *kv_codes, uint8_t *kv_scales,
                                         const uint16_t *kv_new, const float *sink, const int32_t *cidx,
                                         int32_t *idx_out, int64_t b, int32_t h, int32_t d, int64_t rows,
                                         int32_t window, int32_t kc, int64_t start_pos, float scale,
                                         uint16_t *out, void *workspace, size_t workspace_bytes,
                                         void *stream, int32_t splits);

/* ------------------------------------------------------------------------
 * Rotary embedding -- [ATTN-RS] apply_rotary, [ROPE] apply_rotary_emb.
 *
 *   x     [b][s][h][row_len] bf16, modified in place (h = 1 for [b][s][row_len])
 *   table [n_pos][rope_dim / 2][2] f32: (cos, sin) of position p, pair j
 * The last rope_dim values of every row are rotated; row (bi, si, hi) sits at
 * position start_pos + si.  Pair j of the rotated part, (a, b) = (x[2j],
 * x[2j+1]), is the complex number a + i b, multiplied in f32 by cos + i sin
 * (inverse != 0: by cos - i sin, which removes a rotation) -- each real product
 * rounded, then the sum, no fused multiply-add -- and stored as bf16 (round to
 * nearest even):
 *   forward: (a cos - b sin, a sin + b cos)   inverse: (a cos + b sin, b cos - a sin)
 * Bit-exact against that definition.  rope_dim even and <= row_len, row_len
 * even, start_pos + s <= n_pos (else SA_ERR_SHAPE); x 4-byte and table 8-byte
 * aligned (else SA_ERR_SHAPE). */
sa_status sa_apply_rotary(uint16_t *x, int64_t b, int64_t s, int32_t h, int32_t row_len, int32_t rope_dim,
                          const float *table, int64_t n_pos, int64_t start_pos, int32_t inverse, void *stream);

/* ------------------------------------------------------------------------
 * Sparse latent attention with the output's inverse rotation fused into its
 * epilogue -- [ROPE] Attention.forward: after sparse_attn the last rope_dim
 * values of the output are un-rotated at the query's position
 * (apply_rotary_emb(o[..., -rd:], freqs_cis, inverse=True)).
 *
 * Same result, bit for bit, as the unfused pair of calls
 *   sa_sparse_attn_ex(..., kernel, splits)   (resp. sa_sparse_attn_decode_step,
 *                                             sa_sparse_attn_prefill_step)
 *   sa_apply_rotary(out, b, s, h, d, rope_dim, rope_table, n_pos, start_pos, 1)
 * (the rounded bf16 output is rotated, as the pages round before rotating),
 * without the second pass over the output.  Query si of a sequence sits at
 * position start_pos + si (the decode step: start_pos; the prefill step: si).  rope_table as for
 * sa_apply_rotary, 16-byte aligned; rope_dim a multiple of 8 in [8, d];
 * positions within [0, n_pos) (else SA_ERR_SHAPE); NULL rope_table:
 * SA_ERR_NULL.  Other arguments, workspace and errors as for the unfused
 * entry points. */
sa_status sa_sparse_attn_rope(const uint16_t *q, const uint16_t *kv, const float *sink, const int32_t *idx,
                              int64_t b, int64_t s, int32_t h, int32_t d, int64_t rows, int32_t topk, float scale,
                              uint16_t *out, void *workspace, size_t workspace_bytes, void *stream,
                              int32_t kernel, int32_t splits, const float *rope_table, int64_t n_pos,
                              int32_t rope_dim, int64_t start_pos);

sa_status sa_sparse_attn_decode_step_rope(const uint16_t *q, uint16_t *kv, const uint16_t *kv_new,
                                          const float *sink, const int32_t *cidx, int32_t *idx_out, int64_t b,
                                          int32_t h, int32_t d, int64_t rows, int32_t window, int32_t kc,
                                          int64_t start_pos, float scale, uint16_t *out, void *workspace,
                                          size_t workspace_bytes, void *stream, int32_t kernel, int32_t splits,
                                          const float *rope_table, int64_t n_pos, int32_t rope_dim);

sa_status sa_sparse_attn_prefill_step_rope(const uint16_t *q, const uint16_t *kv, const float *sink,
                                           const int32_t *cidx, int32_t *idx_out, int64_t b, int64_t s, int32_t h,
                                           int32_t d, int64_t rows, int32_t window, int32_t kc, float scale,
                                           uint16_t *out, void *workspace, size_t workspace_bytes, void *stream,
                                           int32_t kernel, int32_t splits, const float *rope_table, int64_t n_pos,
                                           int32_t rope_dim);

/* ------------------------------------------------------------------------
 * The indexer's selection tail -- [INDEXER] Indexer.forward after the scores
 * (the compressed half of the index list).
 *
 *   scores [b][s][n_cols] f32   index scores of the n_cols = (start_pos + s) /
 *                               ratio compressed positions (else SA_ERR_SHAPE);
 *                               not NaN (a NaN ranks above +inf, undefined by
 *                               the pages)
 *   idx    int32, rows of row_stride entries, one per (b, s) query; the
 *          selection goes to columns [col0, col0 + topk) and nothing else is
 *          written (row_stride >= col0 + topk, else SA_ERR_SHAPE)
 * For query (bi, si): compress_lens = (si + 1) / ratio when start_pos == 0
 * (positions past it are masked to -inf), else (start_pos + s) / ratio;
 * topk = min(index_topk, n_cols) positions with the largest scores (equal
 * scores: the lower position first -- the pages leave the choice open) are
 * listed in position order as position + offset, or -1 where the position is
 * >= compress_lens.  Deterministic; bit-exact against that definition.
 * ratio >= 1, offset >= 0, col0 >= 0 (else SA_ERR_SHAPE). */
sa_status sa_indexer_topk(const float *scores, int64_t b, int64_t s, int32_t n_cols, int64_t start_pos,
                          int32_t ratio, int32_t index_topk, int32_t offset, int32_t *idx, int64_t row_stride,
                          int32_t col0, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
