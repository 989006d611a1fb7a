/*
 * sa_oracle.c -- plain, slow, obviously-correct CPU oracle for sparse latent
 * attention (DeepSeek-V4.1) and the helpers on its data path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library shares
 * no code, header, table or constant generator with this file, and this file
 * includes nothing from it.
 *
 * Sources (web pages, cited by title and section):
 *   [ATTEND]  "DeepSeek V4.1 ... attention / attend": get_window_topk_idxs and
 *             the sparse_attn kernel + wrapper.
 *   [QLAT]    "DeepSeek V4.1 ... attention / query-latent": Attention.forward
 *             (window/compressed concatenation), Indexer tail (offset, -1).
 *   [ATTN-RS] "Module attn" (deepseek_v41_ref attn rustdoc): precision
 *             contract, ring-cache worked example, act_quant_inplace,
 *             pow2_ceil, sparse_attn, window_topk_idxs, apply_rotary contracts.
 *   [ROPE]    "DeepSeek V4.1 ... attention / query-latent": apply_rotary_emb
 *             and its use on the attention output (inverse rotation).
 *   [INDEXER] same page, Indexer.forward: the selection tail (causal
 *             compress_lens mask, top-k, position order, offset / -1).
 *
 * Arithmetic: sparse_attn in f32 as [ATTN-RS] "Precision" fixes it (f32
 * softmax, bf16 result).  It is written as the plain two-pass softmax
 * definition, not as the pages' blocked online kernel (which reaches the same
 * value up to rounding order).  bf16 values travel as uint16 bit patterns.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define SAO_OK 0
#define SAO_ERR_NULL 1
#define SAO_ERR_SHAPE 2
#define SAO_ERR_UNSUPPORTED 3
#define SAO_ERR_INDEX 5

/* ---------------------------------------------------------------- bf16 --- */

static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round-to-nearest-even f32 -> bf16 (torch's .to(torch.bfloat16)), NaN kept
 * quiet. */
static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------- window slot selection --- */

/* Shape of the window selection ([ATTN-RS] window_topk_idxs: "([queries][cols],
 * cols)").  Prefill (start_pos == 0): one row per query, min(seqlen, window)
 * columns.  Decode: a single query, the whole ring ([ATTEND]
 * get_window_topk_idxs).  A chunk that starts after position 0 with more than
 * one token is not defined on the pages and is rejected. */
int sao_window_topk_idxs_shape(int32_t window, int32_t seqlen, int64_t start_pos,
                               int32_t *rows, int32_t *cols) {
    if (!rows || !cols) return SAO_ERR_NULL;
    if (window <= 0 || seqlen < 0 || start_pos < 0) return SAO_ERR_SHAPE;
    if (start_pos == 0) {
        *rows = seqlen;
        *cols = seqlen < window ? seqlen : window;
        return SAO_OK;
    }
    if (seqlen != 1) return SAO_ERR_UNSUPPORTED;
    *rows = 1;
    *cols = window;
    return SAO_OK;
}

/* [ATTEND] get_window_topk_idxs.
 * Prefill: query p sees the causal window of the chunk ending at p, i.e. slots
 *   first(p) + j for j < cols, first(p) = max(0, p - window + 1); a slot past p
 *   (the sequence has not reached it) is -1.
 * Decode: the ring listed oldest first.  The newest token sits in slot
 *   start_pos % window, so the listing starts one past it and wraps; a slot
 *   whose index exceeds start_pos has never been written (ring still filling)
 *   and is -1.
 * The same rows are written for every batch element; row r of batch b starts at
 * out + (b * nrows + r) * row_stride, and only the first cols entries of a row
 * are written. */
int sao_window_topk_idxs(int32_t window, int32_t bsz, int32_t seqlen, int64_t start_pos,
                         int32_t *out, int64_t row_stride) {
    int32_t nrows, cols;
    int st = sao_window_topk_idxs_shape(window, seqlen, start_pos, &nrows, &cols);
    if (st != SAO_OK) return st;
    if (bsz < 0 || row_stride < cols) return SAO_ERR_SHAPE;
    if ((int64_t)bsz * nrows * cols == 0) return SAO_OK;
    if (!out) return SAO_ERR_NULL;
    for (int32_t b = 0; b < bsz; ++b) {
        for (int32_t r = 0; r < nrows; ++r) {
            int32_t *row = out + ((int64_t)b * nrows + r) * row_stride;
            for (int32_t j = 0; j < cols; ++j) {
                int64_t slot;
                int64_t last; /* the newest position this query may see */
                if (start_pos == 0) {
                    int64_t first = (int64_t)r - window + 1;
                    if (first < 0) first = 0;
                    slot = first + j;
                    last = r;
                } else {
                    int64_t oldest = start_pos % window + 1;
                    slot = (oldest + j) % window;
                    last = start_pos;
                }
                row[j] = slot > last ? -1 : (int32_t)slot;
            }
        }
    }
    return SAO_OK;
}

/* ------------------------------------------------------- ring cache write --- */

/* Writes a chunk of `seqlen` new KV rows (positions start_pos .. start_pos +
 * seqlen - 1) into a ring of `window` slots: position t lands in slot
 * t % window.  Only the last `window` positions of the chunk survive, so
 * earlier ones are skipped.  Behaviour fixed by the [ATTN-RS] ring-cache worked
 * example (12 prefill tokens into 8 slots leave slots 4..7 = tokens 4..7 and
 * slots 0..3 = tokens 8..11; decode step 12 writes slot 4, step 13 slot 5) and
 * the zero-initialised ring buffer of [QLAT] Attention.__init__.
 * ring: [bsz][window][d], rows: [bsz][seqlen][d], both bf16 bits. */
int sao_ring_write(uint16_t *ring, const uint16_t *rows, int32_t bsz, int32_t window,
                   int32_t d, int64_t start_pos, int32_t seqlen) {
    if (bsz < 0 || window <= 0 || d <= 0 || seqlen < 0 || start_pos < 0) return SAO_ERR_SHAPE;
    if ((int64_t)bsz * seqlen == 0) return SAO_OK;
    if (!ring || !rows) return SAO_ERR_NULL;
    int64_t end = start_pos + seqlen;
    int64_t from = end - window > start_pos ? end - window : start_pos;
    for (int32_t b = 0; b < bsz; ++b)
        for (int64_t t = from; t < end; ++t)
            memcpy(ring + ((int64_t)b * window + t % window) * d,
                   rows + ((int64_t)b * seqlen + (t - start_pos)) * d, (size_t)d * 2);
    return SAO_OK;
}

/* ------------------------------------------------ fp8 (e4m3) round trip --- */

/* [ATTN-RS] pow2_ceil: 2 ** ceil(log2 v) for a positive normal f32, taken from
 * the IEEE fields: an exact power of two (zero mantissa) is returned as is,
 * otherwise the exponent is raised by one and the mantissa cleared. */
float sao_pow2_ceil(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    if ((u & 0x007fffffu) != 0) u = ((u >> 23) + 1u) << 23;
    float r;
    memcpy(&r, &u, 4);
    return r;
}

/* Nearest OCP e4m3fn value to y (ties to even mantissa), clamped to +-448.
 * e4m3fn: 3 mantissa bits, exponent bias 7, normals from 2^-6, subnormals
 * spaced 2^-9, largest finite 448, no infinity.  The spacing of the grid at |y|
 * is 2^(e-3) for 2^e <= |y| < 2^(e+1) (e >= -6) and 2^-9 below 2^-6; |y| is
 * divided by that spacing (an exact power-of-two scaling), rounded to an
 * integer with ties to even, and scaled back. */
static float e4m3_rne(float y) {
    float a = fabsf(y);
    if (a == 0.0f) return y; /* keeps the sign of zero */
    int e;
    (void)frexpf(a, &e); /* a = f * 2^e, f in [0.5, 1) -> 2^(e-1) <= a < 2^e */
    int exp_floor = e - 1;
    if (exp_floor < -6) exp_floor = -6;
    float quantum = ldexpf(1.0f, exp_floor - 3);
    float r = a / quantum; /* exact */
    float fl = floorf(r);
    float frac = r - fl; /* exact */
    float n = fl;
    if (frac > 0.5f || (frac == 0.5f && fmodf(fl, 2.0f) != 0.0f)) n = fl + 1.0f;
    float q = n * quantum;
    if (q > 448.0f) q = 448.0f;
    return y < 0 ? -q : q;
}

/* [ATTN-RS] act_quant_inplace: per block of FP8_BLOCK (= 32) contiguous values
 * along a row, scale = pow2_ceil(amax / 448) with amax floored at 1e-4; each
 * value goes to e4m3 (RNE, clamped) at that scale and is dequantised and
 * rounded back to bf16, in place.  "The fp8 round trip is bf16-exact"
 * ([ATTN-RS] Precision): e4m3 times a power of two, so the final bf16
 * conversion is exact for in-range values.  row_len must be a multiple of
 * 32. */
int sao_act_quant_fp8_inplace(uint16_t *x, int64_t n_rows, int32_t row_len) {
    if (n_rows < 0 || row_len <= 0 || row_len % 32 != 0) return SAO_ERR_SHAPE;
    if (n_rows == 0) return SAO_OK;
    if (!x) return SAO_ERR_NULL;
    int64_t nblocks = n_rows * (row_len / 32);
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < nblocks; ++blk) {
        uint16_t *v = x + blk * 32;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(bf16_to_f32(v[i]));
            if (a > amax) amax = a;
        }
        if (amax < 1e-4f) amax = 1e-4f;
        float scale = sao_pow2_ceil(amax / 448.0f);
        for (int i = 0; i < 32; ++i) {
            float y = bf16_to_f32(v[i]) / scale;
            float e = e4m3_rne(y);
            v[i] = f32_to_bf16(e * scale);
        }
    }
    return SAO_OK;
}

/* ----------------------------------------- fp8-resident KV rows (kv8) --- */

/* The fp8 round trip above keeps, per block of 32 values, an e4m3fn value times
 * a power-of-two scale; a KV row can therefore be held as those e4m3fn codes
 * (one byte per value) plus one scale byte per block, and expanded to exactly
 * the bf16 values the round trip gives ([ATTN-RS] "Precision": bf16-exact).
 * Scale bytes use the E8M0 encoding: byte b stands for 2^(b - 127). */

/* OCP e4m3fn code of a value on the e4m3fn grid (|q| <= 448): sign bit, four
 * exponent bits with bias 7, three mantissa bits; exponent field 0 holds the
 * subnormals m * 2^-9 (and zero). */
static uint8_t e4m3_code(float q) {
    uint8_t sign = signbit(q) ? 0x80u : 0u;
    float a = fabsf(q);
    if (a < 0.015625f) return (uint8_t)(sign | (uint8_t)(a * 512.0f)); /* exact: a = m 2^-9 */
    int e;
    (void)frexpf(a, &e);                                   /* 2^(e-1) <= a < 2^e */
    int ef = e - 1;                                         /* unbiased exponent */
    int m = (int)((ldexpf(a, -ef) - 1.0f) * 8.0f);          /* exact: 3 mantissa bits */
    return (uint8_t)(sign | (uint8_t)((ef + 7) << 3) | (uint8_t)m);
}

/* value of an e4m3fn code (0x7f and 0xff are NaN) */
static float e4m3_value(uint8_t c) {
    int ef = (c >> 3) & 15, m = c & 7;
    if (ef == 15 && m == 7) return NAN;
    float a = ef == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, ef - 7);
    return (c & 0x80u) ? -a : a;
}

/* bf16 rows [n_rows][row_len] -> codes [n_rows][row_len] and scale bytes
 * [n_rows][row_len / 32], with the rounding of sao_act_quant_fp8_inplace. */
int sao_kv8_pack(const uint16_t *x, uint8_t *codes, uint8_t *scales, int64_t n_rows, int32_t row_len) {
    if (n_rows < 0 || row_len <= 0 || row_len % 32 != 0) return SAO_ERR_SHAPE;
    if (n_rows == 0) return SAO_OK;
    if (!x || !codes || !scales) return SAO_ERR_NULL;
    int64_t nblocks = n_rows * (row_len / 32);
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < nblocks; ++blk) {
        const uint16_t *v = x + blk * 32;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(bf16_to_f32(v[i]));
            if (a > amax) amax = a;
        }
        if (amax < 1e-4f) amax = 1e-4f;
        float scale = sao_pow2_ceil(amax / 448.0f);
        int e;
        (void)frexpf(scale, &e); /* scale = 2^(e-1) exactly */
        scales[blk] = (uint8_t)(e - 1 + 127);
        for (int i = 0; i < 32; ++i) codes[blk * 32 + i] = e4m3_code(e4m3_rne(bf16_to_f32(v[i]) / scale));
    }
    return SAO_OK;
}

/* codes + scale bytes -> bf16 rows: e4m3fn value times 2^(scale byte - 127) */
int sao_kv8_unpack(const uint8_t *codes, const uint8_t *scales, uint16_t *x, int64_t n_rows, int32_t row_len) {
    if (n_rows < 0 || row_len <= 0 || row_len % 32 != 0) return SAO_ERR_SHAPE;
    if (n_rows == 0) return SAO_OK;
    if (!x || !codes || !scales) return SAO_ERR_NULL;
    int64_t n = n_rows * row_len;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        x[i] = f32_to_bf16(ldexpf(e4m3_value(codes[i]), (int)scales[i / 32] - 127));
    return SAO_OK;
}

/* -------------------------------------- compressed-index concatenation --- */

/* [QLAT] Attention.forward concatenates the window indices with the
 * compressed ones along the topk axis, the compressed ones addressing rows
 * after the window rows; the Indexer tail shifts reachable positions by that
 * offset and leaves unreachable ones at -1.  Here: out[r][col0 + j] =
 * cidx[r][j] + offset, or -1 where cidx[r][j] < 0, for n_rows rows of kc
 * entries; out rows are row_stride apart. */
int sao_append_compressed_idxs(int32_t *out, int64_t row_stride, int32_t col0,
                               const int32_t *cidx, int64_t n_rows, int32_t kc,
                               int32_t offset) {
    if (n_rows < 0 || kc < 0 || col0 < 0 || offset < 0 || row_stride < (int64_t)col0 + kc)
        return SAO_ERR_SHAPE;
    if (n_rows * kc == 0) return SAO_OK;
    if (!out || !cidx) return SAO_ERR_NULL;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int32_t j = 0; j < kc; ++j) {
            int32_t c = cidx[r * kc + j];
            out[r * row_stride + col0 + j] = c < 0 ? -1 : c + offset;
        }
    return SAO_OK;
}

/* ------------------------------------------------------------ sparse_attn --- */

/* [ATTN-RS] sparse_attn / [ATTEND] sparse_attn_kernel: for each batch element,
 * query and head i, a softmax over the KV rows that the query's index list
 * selects (entries of -1 are skipped; a row listed twice counts twice), with
 * the per-head sink logit sink[i] added to the denominator only, in f32;
 * output rounded to bf16.  The same latent row serves as key and value.  A
 * query with no valid entry outputs zeros ([ATTEND] kernel: the finite
 * running-max start makes an all -1 row give zero).
 *   q   [b][s][h][d] bf16      kv  [b][rows][d] bf16     sink [h] f32
 *   idx [b][s][topk] int32     out [b][s][h][d] bf16     out_f32 optional, same
 *   shape, the value before the bf16 rounding.
 * Plain definition (two passes):
 *   s_t = scale * sum_c q[i][c] * kv[idx_t][c]          (f32, c in order)
 *   M   = max(max_t s_t, sink[i])
 *   L   = sum_t exp(s_t - M) + exp(sink[i] - M)
 *   o_c = sum_t exp(s_t - M) * kv[idx_t][c] / L
 * Including the sink in M only rescales numerator and denominator by the same
 * factor, so this equals the pages' form in which the sink is left out of the
 * running max.  Entries outside {-1} U [0, rows) are a caller error: the
 * oracle checks all of them first and returns SAO_ERR_INDEX. */
int sao_sparse_attn(const uint16_t *q, const uint16_t *kv, const float *sink,
                    const int32_t *idx, int64_t b, int64_t s, int32_t h, int32_t d,
                    int64_t rows, int32_t topk, float scale, uint16_t *out, float *out_f32) {
    if (b < 0 || s < 0 || h < 0 || d < 0 || rows < 0 || topk < 0) return SAO_ERR_SHAPE;
    int64_t nq = b * s;
    if (nq * h * d == 0) return SAO_OK;
    if (!q || !sink || !out || (topk > 0 && !idx) || (rows > 0 && !kv)) return SAO_ERR_NULL;
    for (int64_t e = 0; e < nq * topk; ++e)
        if (idx[e] < -1 || idx[e] >= rows) return SAO_ERR_INDEX;

    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t qi = 0; qi < nq; ++qi) {
        int64_t bi = qi / s;
        const int32_t *ix = idx ? idx + qi * topk : NULL;
        const uint16_t *kvb = kv ? kv + bi * rows * d : NULL;
        /* scratch on the stack is bounded by topk and d; heap-free on purpose */
        float sc_buf[16384];
        float acc_buf[1024];
        if (topk > 16384 || d > 1024) { bad = 1; continue; }
        for (int32_t i = 0; i < h; ++i) {
            const uint16_t *qv = q + (qi * h + i) * (int64_t)d;
            uint16_t *ov = out + (qi * h + i) * (int64_t)d;
            float *of = out_f32 ? out_f32 + (qi * h + i) * (int64_t)d : NULL;
            int nvalid = 0;
            float m = sink[i];
            for (int32_t t = 0; t < topk; ++t) {
                if (ix[t] == -1) continue;
                const uint16_t *kr = kvb + (int64_t)ix[t] * d;
                float dot = 0.0f;
                for (int32_t c = 0; c < d; ++c) dot += bf16_to_f32(qv[c]) * bf16_to_f32(kr[c]);
                float st = scale * dot;
                sc_buf[t] = st;
                if (st > m) m = st; /* m starts at sink[i] */
                ++nvalid;
            }
            if (nvalid == 0) {
                for (int32_t c = 0; c < d; ++c) {
                    ov[c] = 0;
                    if (of) of[c] = 0.0f;
                }
                continue;
            }
            float l = expf(sink[i] - m);
            for (int32_t c = 0; c < d; ++c) acc_buf[c] = 0.0f;
            for (int32_t t = 0; t < topk; ++t) {
                if (ix[t] == -1) continue;
                float p = expf(sc_buf[t] - m);
                l += p;
                const uint16_t *kr = kvb + (int64_t)ix[t] * d;
                for (int32_t c = 0; c < d; ++c) acc_buf[c] += p * bf16_to_f32(kr[c]);
            }
            for (int32_t c = 0; c < d; ++c) {
                float o = acc_buf[c] / l;
                ov[c] = f32_to_bf16(o);
                if (of) of[c] = o;
            }
        }
    }
    return bad ? SAO_ERR_UNSUPPORTED : SAO_OK;
}

/* ------------------------------------------------------ rotary embedding --- */

/* [ATTN-RS] apply_rotary, [ROPE] apply_rotary_emb: rotate the last rope_dim
 * values of every row_len-wide row of x [b][s][h][row_len] in place; row
 * (bi, si, hi) sits at position start_pos + si.  Adjacent pairs (x[2j],
 * x[2j+1]) of the rotated part are the complex number a + i b, multiplied in
 * f32 by the table entry (c, sn) of that position and pair -- by its conjugate
 * c - i sn when inverse (the output's un-rotation after sparse_attn) -- and
 * written back as bf16 (round to nearest even).  The f32 complex product rounds
 * each real product, then the sum:
 *   forward: re = a c - b sn,   im = a sn + b c
 *   inverse: re = a c + b sn,   im = b c - a sn
 *   table [n_pos][rope_dim / 2][2] f32 (cos, sin) of position p, pair j.
 * rope_dim must be even and at most row_len (else SAO_ERR_SHAPE); every
 * position start_pos + si must lie in [0, n_pos) (else SAO_ERR_INDEX). */
int sao_apply_rotary(uint16_t *x, int64_t b, int64_t s, int32_t h, int32_t row_len, int32_t rope_dim,
                     const float *table, int64_t n_pos, int64_t start_pos, int inverse) {
    if (b < 0 || s < 0 || h < 0 || row_len < 0 || rope_dim < 0 || n_pos < 0) return SAO_ERR_SHAPE;
    if (rope_dim % 2 != 0 || rope_dim > row_len) return SAO_ERR_SHAPE;
    if (b * s * h == 0 || rope_dim == 0) return SAO_OK;
    if (!x || !table) return SAO_ERR_NULL;
    if (start_pos < 0 || start_pos + s > n_pos) return SAO_ERR_INDEX;
    const int32_t half = rope_dim / 2;
    for (int64_t bi = 0; bi < b; ++bi)
        for (int64_t si = 0; si < s; ++si) {
            const float *tp = table + (start_pos + si) * (int64_t)half * 2;
            for (int32_t hi = 0; hi < h; ++hi) {
                uint16_t *row = x + ((bi * s + si) * h + hi) * (int64_t)row_len + (row_len - rope_dim);
                for (int32_t j = 0; j < half; ++j) {
                    const float a = bf16_to_f32(row[2 * j]), bb = bf16_to_f32(row[2 * j + 1]);
                    const float c = tp[2 * j], sn = tp[2 * j + 1];
                    const float ac = a * c, bs = bb * sn, as = a * sn, bc = bb * c;
                    float re, im;
                    if (inverse) {
                        re = ac + bs;
                        im = bc - as;
                    } else {
                        re = ac - bs;
                        im = as + bc;
                    }
                    row[2 * j] = f32_to_bf16(re);
                    row[2 * j + 1] = f32_to_bf16(im);
                }
            }
        }
    return SAO_OK;
}

/* ------------------------------------------------ indexer selection tail --- */

typedef struct {
    float score;
    int32_t t;
} sao_cand;

/* best first: larger score, then the lower position */
static int cand_order(const void *pa, const void *pb) {
    const sao_cand *a = (const sao_cand *)pa, *b = (const sao_cand *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->t > b->t) - (a->t < b->t);
}

static int int_order(const void *pa, const void *pb) {
    const int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* [INDEXER] Indexer.forward, after the scores: with end_pos = start_pos + s and
 * T = end_pos / ratio compressed positions scored per query (scores
 * [b][s][T] f32, not NaN):
 *   compress_lens: prefill (start_pos == 0) query si sees (si + 1) / ratio
 *     positions and the rest of its row is masked to -inf; otherwise every query
 *     sees end_pos / ratio (= T) and nothing is masked;
 *   topk = min(index_topk, T) positions with the largest scores (equal scores:
 *     the lower position first -- the pages leave the choice open), re-sorted
 *     into position order;
 *   out[bi][si][j] = position + offset if position < compress_lens, else -1.
 * out rows are row_stride apart, entries from column col0 (row_stride >=
 * col0 + topk).  Integer division is floor division (all operands >= 0). */
int sao_indexer_topk(const float *scores, int64_t b, int64_t s, int32_t T, int64_t start_pos, int32_t ratio,
                     int32_t index_topk, int32_t offset, int32_t *out, int64_t row_stride, int32_t col0) {
    if (b < 0 || s < 0 || T < 0 || start_pos < 0 || ratio <= 0 || index_topk < 0 || offset < 0 || col0 < 0)
        return SAO_ERR_SHAPE;
    if ((int64_t)T != (start_pos + s) / ratio) return SAO_ERR_SHAPE;
    const int32_t topk = index_topk < T ? index_topk : T;
    if (row_stride < (int64_t)col0 + topk) return SAO_ERR_SHAPE;
    if (b * s == 0 || topk == 0) return SAO_OK;
    if (!scores || !out) return SAO_ERR_NULL;
    for (int64_t e = 0; e < b * s * T; ++e)
        if (isnan(scores[e])) return SAO_ERR_INDEX;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < b * s; ++r) {
        const int64_t si = r % s;
        const int64_t cl = start_pos == 0 ? (si + 1) / ratio : (start_pos + s) / ratio;
        sao_cand *c = (sao_cand *)malloc(sizeof(sao_cand) * (size_t)T);
        int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)topk);
        if (!c || !sel) {
            free(c);
            free(sel);
            bad = 1;
            continue;
        }
        for (int32_t t = 0; t < T; ++t) {
            c[t].score = t >= cl ? -INFINITY : scores[r * T + t];
            c[t].t = t;
        }
        qsort(c, (size_t)T, sizeof(sao_cand), cand_order);
        for (int32_t j = 0; j < topk; ++j) sel[j] = c[j].t;
        qsort(sel, (size_t)topk, sizeof(int32_t), int_order);
        for (int32_t j = 0; j < topk; ++j) out[r * row_stride + col0 + j] = sel[j] < cl ? sel[j] + offset : -1;
        free(c);
        free(sel);
    }
    return bad ? SAO_ERR_UNSUPPORTED : SAO_OK;
}

/* Thread count of the OpenMP loops above: n > 0 sets it; returns the count a
 * parallel loop will use from now on (timing support, no arithmetic). */
int sao_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
}
