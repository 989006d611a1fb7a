// sa_attn.hip -- sparse latent attention for CDNA4 (gfx950): the pair, wide
// and decode kernels, the split combine and the dispatcher.
//
// Operation ("DeepSeek V4.1 ... attention / attend": sparse_attn_kernel and its
// wrapper; "Module attn" rustdoc: sparse_attn): for every query and head, a
// softmax over the latent KV rows its index list selects (-1 skipped), the
// per-head sink adding to the denominator only, f32 arithmetic, bf16 result.
// One latent row is both key and value and is shared by every head, so a
// workgroup gathers each selected row into LDS once and all its heads use it.
//
// Three kernels share the operation; the dispatcher picks one from the shape.
//  * pair kernel (prefill-sized grids): one workgroup of two wavefronts per
//    (query, 64 heads[, index split]); each wavefront holds a 32-head tile over
//    the whole head dim and walks every row of the list in 32-row stages, so no
//    merge between wavefronts; under 80 KiB of LDS, two workgroups per CU.
//  * wide kernel (long lists in decode-sized grids): four wavefronts per
//    (query, 64 heads[, split]) as 2 head tiles x 2 halves of every 64-row
//    stage; the halves are merged once at the end.
//  * decode kernel (short lists, decode-sized grids): four wavefronts per
//    (query, 16 heads[, split]), see its own header below.
// The wide and pair kernels:
//  1. compaction: the query's index entries are scanned and the valid ones
//     (0 <= idx < rows) packed into an LDS list, so -1 entries cost no MFMA work
//     and no traffic;
//  2. gather: stages of rows copied HBM -> LDS with the direct global->LDS path
//     (16 B per lane, one 1 KiB row per wave instruction at d = 512), two
//     buffers, so the copy of stage t+1 overlaps the maths of stage t.  A row
//     takes 2 d + 64 bytes of LDS with its 16-byte chunks swizzled in groups of
//     four rows (RowLayout below), which keeps both operand read patterns free
//     of bank conflicts and makes every operand address a per-lane base plus an
//     immediate;
//  3. scores S^T[32 rows][32 heads] = K[rows][:] . Q[heads][:]^T on MFMA
//     32x32x16 bf16 (A = gathered rows from LDS, B = the wave's Q held in
//     registers for the whole list), f32 accumulation;
//  4. softmax in the base-2 domain (scale * log2 e folded once) against a fixed
//     reference max: the first stage max a wavefront sees.  A later stage max may
//     exceed it by up to 2^32 (weights stay far inside bf16 and f32 range), so O
//     is never rescaled inside the loop; should one outrun it further, the
//     workgroup replays the list against the larger max.  The reference starts
//     at the finite -1e30 of the pages' kernel, so a list with no valid entry
//     yields zeros rather than NaN;
//  5. O^T[d][head] += V^T[d][rows] . P^T[rows][head] on the same MFMA: P is
//     rounded to bf16 straight from the score registers (its lane layout is the
//     B operand's, up to a permutation of the contraction index that the V^T
//     reads follow), V^T comes from LDS through the gfx950 transposing read
//     ds_read_b64_tr_b16;
//  6. sink fold, normalisation, bf16 staged through LDS and stored one row per
//     wave instruction -- or, for split variants, f32 partials (running max,
//     sum, unnormalised O) combined by a second pass.
#include "sa_fp8.h"
#include "../../include/sparse_attn.h"

#include <algorithm>
#include <mutex>
#include <type_traits>

namespace {

using namespace sa;

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kListCap = 4096;        // compacted entries held in LDS at once
constexpr float kRescaleSlack = 8.0f; // log2 units the reference max may lag behind
constexpr int kPfvEarly = 1;          // weighted-sum operand reads issued ahead of the weights (0..2 measured alike)

struct AttnParams {
    const uint16_t *q;
    const uint16_t *kv;
    const float *sink;
    const int32_t *idx;
    uint16_t *out;
    float *part_o;   // [nq][n_sp][h][d] f32 (split variant only)
    float *part_ml;  // [nq][n_sp][h][2] f32: running max (log2 units), running sum
    int64_t rows;    // kv rows per sequence
    int32_t nq;      // b * s
    int32_t s;       // queries per sequence
    int32_t total_wg;
    int32_t h;
    int32_t topk;
    int32_t n_hg;       // head groups
    int32_t n_sp;       // index splits
    int32_t split_len;  // index entries per split
    float scale_log2;   // softmax scale * log2(e)
    int32_t stagger_cu; // pair kernel: workgroups [stagger_cu, 2 stagger_cu) start late (0: none)
    int32_t qchunk;     // wide and pair kernels: consecutive queries per XCD run (see wide_unit)
    // fused decode step only: the list is built in the kernel and the step's
    // new latent row is rounded through fp8 and written into its ring slot
    const uint16_t *kv_new;  // [nq][d] this step's raw latent rows
    uint16_t *kv_ring;       // == kv, writable: ring slot new_slot receives the rounded row
    const int32_t *cidx;     // [nq][kc] compressed positions (-1 = none)
    int32_t *idx_out;        // [nq][topk] concatenated list written out, or null
    int64_t pos;             // position of the step's token (start_pos >= 1); -1 for the
                             // pair kernel's prefill list
    int32_t window;          // ring slots = window-list columns (prefill list: min(s, window))
    int32_t kc;              // compressed columns
    int32_t wbase;           // (pos + 1) % window: slot of the oldest entry
    int32_t new_slot;        // pos % window: slot of the new row (list entry window - 1)
    // inverse rotation of the output's last rope_dim values (null rope: none):
    // query (b, s) at position rope_pos0 + s, table [positions][rope_dim / 2] of
    // (cos, sin) f32
    const float *rope;
    int32_t rope_dim;
    int64_t rope_pos0;
    // fp8-resident rows (kv8): e4m3fn codes [..][rows][d] and 16-byte scale
    // records [..][rows][16] in place of kv; the fused step writes the new
    // row's codes and scale record into its ring slot.  (Last: the bf16 kernels
    // never read them, so their arguments stay within three 64-byte lines,
    // all loaded at kernel start.)
    const uint8_t *kv8c;
    const uint8_t *kv8s;
    uint8_t *kv8c_ring;
    uint8_t *kv8s_ring;
};

// The window part of a list built in the kernel, for one query, in one form
// for both cases: entry e is row (first + e), less wrap once it reaches wrap,
// valid while <= last; compressed position c becomes entry c + coff.
//  * decode step: the ring listed oldest first (first = (pos + 1) % W, wrap =
//    W), -1 for slots past pos (not yet written); compressed rows follow the
//    ring's W rows;
//  * prefill (PREFILL, the pair kernel's own instance): the query at chunk
//    position t takes chunk rows max(0, t - W + 1) + e, -1 past t (window =
//    min(s, W) columns; for s < W the first row is 0 either way); compressed
//    rows follow the chunk's s rows.
// ("DeepSeek V4.1 ... attention / attend", get_window_topk_idxs; "... /
// query-latent", Attention.forward and the Indexer tail.)
struct ListForm {
    int first, wrap, coff;
    int64_t last;
};
template <bool PREFILL>
__device__ __forceinline__ ListForm list_form(const AttnParams &p, uint32_t qi) {
    ListForm f;
    if constexpr (PREFILL) {
        const int t = (int)(qi % (uint32_t)p.s);
        f.first = max(0, t - p.window + 1);
        f.wrap = 0x7fffffff;
        f.last = t;
        f.coff = p.s;
    } else {
        f.first = p.wbase;
        f.wrap = p.window;
        f.last = p.pos;
        f.coff = p.window;
    }
    return f;
}
__device__ __forceinline__ int window_entry(const ListForm &f, int e) {
    int r = f.first + e;
    if (r >= f.wrap) r -= f.wrap;
    return (int64_t)r <= f.last ? r : -1;
}
__device__ __forceinline__ int compressed_entry(const ListForm &f, int c) {
    return c < 0 ? -1 : (int)((uint32_t)c + (uint32_t)f.coff);
}
// Entry e of the concatenated list: the window entries, then the compressed ones.
__device__ __forceinline__ int step_entry(const AttnParams &p, const ListForm &f, uint32_t qi, int e) {
    if (e < p.window) return window_entry(f, e);
    return compressed_entry(f, p.cidx[(int64_t)qi * p.kc + (e - p.window)]);
}

__device__ __forceinline__ bf16x8_t lds_read_b128(const SA_LDS char *p) {
    return *reinterpret_cast<const SA_LDS bf16x8_t *>(p);
}

__device__ __forceinline__ i16x4_t lds_read_tr16(const SA_LDS char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<SA_LDS i16x4_t *>(const_cast<SA_LDS char *>(p)));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Score product step S^T += K Q^T on MFMA 32x32x16 bf16 with the accumulator
// in VGPRs.  The compiler picks one register class for the accumulators of all
// MFMAs of a kernel; with O in the accumulator registers it would put the score
// tile there too and move an O tile out and back at every stage.  The wait
// states the hardware does not interlock are placed here: one before each MFMA
// (a VALU write of a source operand just before), and after the last MFMA of a
// chain 24 before any VALU reads (or overwrites) the result (8-pass XDL: 11).
// The first step takes an inline-zero accumulator; the output never shares
// registers with the operands.
__device__ __forceinline__ void mfma_s_first(f32x16_t &acc, const bf16x8_t &a, const bf16x8_t &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_next(f32x16_t &acc, const bf16x8_t &a, const bf16x8_t &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_last(f32x16_t &acc, const bf16x8_t &a, const bf16x8_t &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 7"
                 : "+v"(acc)
                 : "v"(a), "v"(b));
}

// max / sum of v over lanes l and l ^ 32 (gfx950 v_permlane32_swap: a VALU
// exchange of the wave's halves, no LDS round trip)
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until at most n (wave-uniform, 0..16) vector-memory operations of this
// wave are outstanding; the count is an immediate of the instruction, so the
// value selects one of the fixed waits.
__device__ __forceinline__ void wait_vmcnt_upto16(int n) {
#define SA_VMW(k) \
    case k: asm volatile("s_waitcnt vmcnt(" #k ")" : : : "memory"); break;
    switch (__builtin_amdgcn_readfirstlane(n)) {
        SA_VMW(1) SA_VMW(2) SA_VMW(3) SA_VMW(4) SA_VMW(5) SA_VMW(6) SA_VMW(7) SA_VMW(8)
        SA_VMW(9) SA_VMW(10) SA_VMW(11) SA_VMW(12) SA_VMW(13) SA_VMW(14) SA_VMW(15) SA_VMW(16)
        default: asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); break;
    }
#undef SA_VMW
}

// Copy of query qi's rotation table row (rope_dim floats, in 16-byte chunks,
// up to two wave instructions) into LDS at tab; called by one whole wavefront.
__device__ __forceinline__ void copy_rope_row(const AttnParams &p, uint32_t qi, int lane, uint32_t tab) {
    const float *row = p.rope + (p.rope_pos0 + (int64_t)(qi % (uint32_t)p.s)) * p.rope_dim;
    const int chunks = p.rope_dim / 4;
    if (lane < chunks) dma_16B(row + 4 * lane, tab);
    if (chunks > 64 && lane < chunks - 64) dma_16B(row + 256 + 4 * lane, tab + 1024);
}

// The inverse rotation of one 16-byte output chunk (8 rounded bf16 values from
// d0), if it lies in the last rope_dim values of the row: pair j of the rotated
// part takes (cos, sin) from tab[2 j], tab[2 j + 1] (the query's table row in
// LDS).  rope_dim is a multiple of 8, so a chunk lies wholly inside or outside.
__device__ __forceinline__ u32x4_t unrotate_chunk(u32x4_t v, int d0, int d, int rope_dim, const SA_LDS float *tab) {
    if (d0 < d - rope_dim) return v;
    const SA_LDS float *cs = tab + (d0 - (d - rope_dim));
    const f32x4_t c0 = *reinterpret_cast<const SA_LDS f32x4_t *>(cs);
    const f32x4_t c1 = *reinterpret_cast<const SA_LDS f32x4_t *>(cs + 4);
    v[0] = rope_pair(v[0], c0[0], c0[1], true);
    v[1] = rope_pair(v[1], c0[2], c0[3], true);
    v[2] = rope_pair(v[2], c1[0], c1[1], true);
    v[3] = rope_pair(v[3], c1[2], c1[3], true);
    return v;
}

// Logical workgroup id (decode kernel).  The dispatcher hands workgroups to the
// 8 XCDs round robin; the remap gives each XCD a contiguous range of logical
// ids, so the head groups and splits of one query, which gather the same rows,
// share that XCD's L2.
__device__ __forceinline__ uint32_t logical_wg(uint32_t T) {
    const uint32_t per = T >> 3, rem = T & 7, x = blockIdx.x & 7, k = blockIdx.x >> 3;
    return x < rem ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

// Wide/pair-kernel workgroup -> (query, j = head group * n_sp + split); false
// for a padding workgroup.  The dispatcher hands block b to XCD b % 8, each XCD
// taking its blocks in order.  A query's n_hg * n_sp workgroups are consecutive
// blocks of one XCD (they gather the same rows: the later ones hit that XCD's
// L2).  Queries go to the XCDs in runs of qchunk consecutive queries, eight runs
// a round in serpentine order (XCD 0..7, then 7..0), so lists whose length grows
// with the query position (a causal prefill) load every XCD alike; within an
// XCD the highest query index goes
// first (long work first leaves short work for the tail).  Runs of more than one
// query serve long prefills: neighbouring queries' windows share most of their
// rows, so an XCD's run fetches them into its L2 once instead of every XCD
// fetching every row.  The grid holds 8 * qchunk * ceil(nq / (8 * qchunk))
// queries' worth of workgroups.
__device__ __forceinline__ bool wide_unit(const AttnParams &p, uint32_t &qi, uint32_t &j) {
    const uint32_t g = (uint32_t)(p.n_hg * p.n_sp);
    const uint32_t k = blockIdx.x >> 3, m = k / g;
    j = k - m * g;
    const uint32_t C = (uint32_t)p.qchunk;
    const uint32_t runs = ((uint32_t)p.nq + 8u * C - 1u) / (8u * C);   // runs per XCD
    const uint32_t r = m / C, w = m - r * C;
    // round R of eight runs (highest first) goes to the XCDs in serpentine order,
    // so the XCDs' shares of a causal prefill's growing lists stay even
    const uint32_t R = runs - 1u - r, x = blockIdx.x & 7u;
    const uint32_t run = 8u * R + ((R & 1u) ? 7u - x : x);
    qi = run * C + (C - 1u - w);
    return qi < (uint32_t)p.nq;
}

// Stage-buffer row layout of the wide and pair kernels.  A gathered row of D
// bf16 values takes RS = 2 D + 64 bytes of LDS, and its 16-byte chunk c sits
// in slot c ^ swz(r) of row r, swz(r) = (r >> 2) & 3 (the chunks of each
// aligned group of four trade places).  The LDS serves 64 banks of 4 bytes:
//  * score operand reads (16 B a lane, 16 lanes a cycle: 16 consecutive rows,
//    one chunk): RS puts row r at bank offset 64 r mod 256 bytes, four rows
//    apart coinciding; the swizzle moves those four to four different chunks;
//  * transposing reads of the weighted-sum operand (8 B a lane, 32 lanes a
//    cycle: 4 consecutive rows sharing swz, 4 aligned chunks each): the rows'
//    64-byte spans sit 64 B apart, the swizzle only permutes chunks inside a
//    span -- conflict-free as well (the unswizzled 48-byte padding served
//    these at half rate).
// The direct copy writes a row's chunks contiguously, so the swizzle is taken
// on the global side: lane i copies chunk i ^ swz(r).
template <int D>
struct RowLayout {
    static constexpr int RS = 2 * D + 64;
    static_assert(RS % 64 == 0 && (RS / 64) % 2 == 1, "row stride: an odd multiple of 64 bytes");
    static constexpr int OUT_RS = 2 * D + 16;  // bf16 output staging rows (written 8 B a lane, read whole)
    __device__ static __forceinline__ int swz(int r) { return (r >> 2) & 3; }
    // per-lane bases of the score operand reads: lane (hf, n) reads chunk
    // 2 ks + hf of row r; k-steps alternate between the two bases, 64 B apart
    // per pair of k-steps (chunk 2 ks + hf ^ swz = 4 (ks >> 1) + ((2 (ks & 1) + hf) ^ swz))
    __device__ static __forceinline__ int kbase(int r, int hf) { return r * RS + 16 * (hf ^ swz(r)); }
    __device__ static __forceinline__ int koff(int kb_even, int ks) {
        return (ks & 1 ? kb_even ^ 32 : kb_even) + 64 * (ks >> 1);
    }
    // per-lane bases of the transposing reads: the 16-lane group reads rows
    // r0 + 4 hf + p/4 (rows of a block of 16, +8 for the upper half of the
    // contraction index) and, within each 64-byte span, chunk 2 (lane bit 4) +
    // (p bit 1), half p bit 0 (p = lane % 16)
    __device__ static __forceinline__ int vbase(int r0, int lane, bool upper) {
        const int hf = lane >> 5, p16 = lane & 15;
        const int r = r0 + 4 * hf + (p16 >> 2) + (upper ? 8 : 0);
        const int c = 2 * ((lane >> 4) & 1) + ((p16 >> 1) & 1);
        return r * RS + 16 * (c ^ swz(r)) + 8 * (p16 & 1);
    }
};

// Index-list compaction.  The entries of idx[c0, c1) (at most CAP) are
// spread over the workgroup's threads as e = c0 + k * NT + tid, k < K, and all
// K loads of a thread are issued together, so a chunk costs one memory latency.
// Valid entries (0 <= v < rows) are packed into list[0, nv) in (k, thread)
// order -- deterministic, and any order is correct (each entry is independent).
template <int NT, int CAP = kListCap>
struct Compactor {
    static constexpr int K = CAP / NT;
    static constexpr int NW = NT / 64;
    int v[K];

    // fetch(e) gives list entry e (a load, or an entry built in place)
    template <class F>
    __device__ __forceinline__ void load(F fetch, int c0, int c1) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = c0 + k * NT + (int)threadIdx.x;
            v[k] = e < c1 ? fetch(e) : -1;
        }
    }

    // the fused decode step's entries [c0, c1), built in place: ring slots by
    // formula, compressed entries from cidx.  The compressed indices are loaded
    // from clamped addresses, all of a thread's loads before any value is used:
    // a load under a per-lane condition gets a wait of its own right behind it,
    // which would put one memory latency per entry on the startup path.
    __device__ __forceinline__ void load_step(const AttnParams &p, uint32_t qi, int c0, int c1) {
        int c[K];
#pragma unroll
        for (int k = 0; k < K; ++k) c[k] = -1;
        if (p.kc > 0) {  // (uniform)
            const int32_t *crow = p.cidx + (int64_t)qi * p.kc;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int e = c0 + k * NT + (int)threadIdx.x;
                c[k] = crow[min(max(e - p.window, 0), p.kc - 1)];
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = c0 + k * NT + (int)threadIdx.x;
            int slot = p.wbase + e;
            if (slot >= p.window) slot -= p.window;
            const int ring = (int64_t)slot <= p.pos ? slot : -1;
            const int comp = c[k] < 0 ? -1 : (int)((uint32_t)c[k] + (uint32_t)p.window);
            v[k] = e >= c1 ? -1 : (e < p.window ? ring : comp);
        }
    }

    // the raw entries of [c0, c1) from list[] (placed there by direct copies:
    // entry e at list[e - c0]); read before pack() rewrites list[]
    __device__ __forceinline__ void load_lds(const int *list, int c0, int c1) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = c0 + k * NT + (int)threadIdx.x;
            v[k] = e < c1 ? list[e - c0] : -1;
        }
    }

    // prefill list from list[] (entry e at list[e - c0]): the window entries as
    // stored, the compressed positions (copied there raw) shifted past the chunk's
    // s rows, -1 kept
    __device__ __forceinline__ void load_lds_prefill(const int *list, int c0, int c1, int window, int s) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = c0 + k * NT + (int)threadIdx.x;
            const int raw = e < c1 ? list[e - c0] : -1;
            v[k] = e >= c1 ? -1 : (e < window || raw < 0 ? raw : (int)((uint32_t)raw + (uint32_t)s));
        }
    }

    // wait for the entry loads here: a compiler-placed wait for them further on
    // would also wait for every copy queued behind them
    __device__ __forceinline__ void ready() const {
#pragma unroll
        for (int k = 0; k < K; ++k) asm volatile("" : : "v"(v[k]));
    }

    // the raw entries of [c0, c1) written out (fused decode step, one head group)
    __device__ __forceinline__ void store(int32_t *out, int c0, int c1) const {
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int e = c0 + k * NT + (int)threadIdx.x;
            if (e < c1) out[e] = v[k];
        }
    }

    // every thread of the workgroup calls it; returns nv
    __device__ __forceinline__ int pack(int64_t rows, int *list, int *wcnt /* [K][NW] */) {
        const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
        uint64_t mask[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            mask[k] = __ballot(v[k] >= 0 && (int64_t)v[k] < rows);
            if (lane == 0) wcnt[k * NW + wave] = __popcll(mask[k]);
        }
        lds_barrier();
        int base = 0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            int pre = 0, tot = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int cw = wcnt[k * NW + w];
                pre += w < wave ? cw : 0;
                tot += cw;
            }
            const uint64_t m = mask[k];
            if ((m >> lane) & 1) {
                const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
                list[base + pre + pos] = v[k];
            }
            base += tot;
        }
        lds_barrier();
        return base;
    }
};

// Weights of one wavefront's 32-row slice of a stage, and its share of the
// weighted sum O^T[d][32 heads] += V^T P^T (wide and pair kernels).
//  * Score value i of lane (hf, n) is slice row 8 (i / 4) + 4 hf + i % 4,
//    head n; rows at or past the list end (entry ebase + row >= nv) weigh 0.
//  * Weights are 2^(scale log2(e) s - m_ref) against a fixed reference: the
//    first slice holding a valid row sets m_ref to its own max.  Later slices
//    take their weights at once and compare their exponents with SLACK only
//    behind the first MFMA of the weighted sum (one ballot; the cross-half max
//    is taken only when it fires): an exponent past SLACK (weights up to
//    2^SLACK stay far inside bf16 and f32 range) raises the replay flag, and
//    the workgroup replays the list against the larger max, so O is never
//    rescaled inside the loop.
//  * The running sum adds the weights as rounded to bf16, as the MFMA takes them.
//  * The first operand reads of the weighted sum go out before the weights:
//    they do not depend on them.  MFMA j = kk DT + dt reads, in 16-lane group
//    (hf, column half), rows 16 kk + 8 rd + 4 hf + p / 4 (rd = 0, 1) and
//    columns 32 dt + 16 (column half) + 4 (p % 4), p = lane % 16, through the
//    transposing read; P enters from the score registers (its lane layout is
//    the B operand's up to the matching permutation of the contraction index).
template <class C>
__device__ __forceinline__ void slice_weights_pv(const f32x16_t &sacc, int ebase, int nv, float scale_log2,
                                                 float &m_ref, float &m_seen, float &l_run, bool &have_ref,
                                                 int &replay_flag, const SA_LDS char *buf, int vlo, int vhi,
                                                 f32x16_t (&acc_o)[C::DT]) {
    const int lane = threadIdx.x & 63;
    const int hf = lane >> 5;
    auto vread = [&](int j) {
        const int dt = j % C::DT, kk = j / C::DT;
        const i16x4_t lo4 = lds_read_tr16(buf + vlo + (16 * kk) * C::RS + 64 * dt);
        const i16x4_t hi4 = lds_read_tr16(buf + vhi + (16 * kk) * C::RS + 64 * dt);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int NJ = 2 * C::DT;
    constexpr int PF = C::PFV;
    bf16x8_t vq[PF];
#pragma unroll
    for (int i = 0; i < C::PFV_EARLY; ++i) vq[i] = vread(i);
    __builtin_amdgcn_sched_barrier(0);

    // rows of a last, partial slice past the list end (partial is wave-uniform)
    const bool partial = ebase + 32 > nv;
    auto valid = [&](int i) { return ebase + 8 * (i >> 2) + 4 * hf + (i & 3) < nv; };
    const bool check = have_ref;
    if (!have_ref && ebase < nv) {
        // the first slice with a valid row: the reference is its max
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, partial && !valid(i) ? -INFINITY : sacc[i] * scale_log2);
        m_ref = m_seen = max_xor32(mx);
        have_ref = true;
    }
    // exponents t = scale log2(e) s - m_ref (-inf for rows past the list end)
    // and their max, which checks the reference behind the first MFMA below
    // (two copies of the loop, so full slices carry no masking)
    float mt = -INFINITY;
    uint32_t pk[8];
    auto weights = [&](auto PARTIAL) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float t0 = fmaf(sacc[2 * i], scale_log2, -m_ref);
            float t1 = fmaf(sacc[2 * i + 1], scale_log2, -m_ref);
            if constexpr (decltype(PARTIAL)::value) {
                t0 = valid(2 * i) ? t0 : -INFINITY;
                t1 = valid(2 * i + 1) ? t1 : -INFINITY;
            }
            mt = fmaxf(mt, fmaxf(t0, t1));
            pk[i] = pack_bf16x2(exp2_fast(t0), exp2_fast(t1));
        }
    };
    if (partial)
        weights(std::true_type{});
    else
        weights(std::false_type{});
    const bf16x8_t pb0 = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
    const bf16x8_t pb1 = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[4], pk[5], pk[6], pk[7]});
#pragma unroll
    for (int i = C::PFV_EARLY; i < PF; ++i) vq[i] = vread(i);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const bf16x8_t a = vq[j % PF];
        if (j + PF < NJ) vq[j % PF] = vread(j + PF);
        acc_o[j % C::DT] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, j >= C::DT ? pb1 : pb0, acc_o[j % C::DT], 0, 0, 0);
        if (j == 0 && check && __ballot(mt > C::SLACK)) {
            // a slice exponent past SLACK in some lane: replay against the larger
            // max.  The head's max over both row halves and the new reference are
            // taken only here: a head's earlier slices that did not trigger stayed
            // within SLACK of its reference, and the new one is never lower, so the
            // replayed pass keeps every weight within 2^SLACK as well.
            mt = max_xor32(mt);
            m_seen = fmaxf(m_seen, m_ref + mt);
            if (lane == 0) replay_flag = 1;
            m_ref = m_seen;
        }
        // the running sum over the weights behind MFMAs 1 .. NJ-1, in order
        if (j >= 1) {
#pragma unroll
            for (int k = (j - 1) * 8 / (NJ - 1); k < j * 8 / (NJ - 1); ++k) {
                const uint32_t b = pk[k];
                l_run += __uint_as_float(b << 16) + __uint_as_float(b & 0xffff0000u);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D>
struct WideCfg {
    // Four wavefronts: 2 head tiles of 32 heads x 2 row halves of every 64-row
    // stage.  A wavefront covers the whole head dim of its 32 heads (Q in
    // registers, O in accumulator registers) and keeps its own running max and
    // sum over the rows it sees; the two row halves of a head tile are merged
    // once, at the end (the algebra of the split combine).  A stage therefore
    // needs no exchange between wavefronts and a single barrier.
    static constexpr int NW = 4;
    static constexpr int THREADS = 64 * NW;
    static constexpr int HEADS = 64;
    static constexpr int ROWS = 64;               // rows per stage (32 per wavefront)
    static constexpr int RPW = ROWS / NW;         // rows each wavefront copies per stage
    using L = RowLayout<D>;
    // stage rows in the swizzled layout of RowLayout: every operand address is
    // one of a few per-lane bases plus a compile-time offset
    static constexpr int RS = L::RS;
    static constexpr int CH = D / 8;              // 16-byte chunks per row
    static constexpr int KS = D / 16;             // k-steps of the score product
    static constexpr int DT = D / 32;             // 32-wide d tiles of the output
    static constexpr int STAGE_BYTES = ROWS * RS;
    static constexpr int NBUF = 2;                // the copy of stage t+1 overlaps the maths of stage t
    // operand reads in flight ahead of the MFMAs (score / weighted-sum product); at
    // d = 512 Q and O fill the register file and the depth is kept small
    // log2 units a stage max may exceed the fixed reference of the weights
    static constexpr float SLACK = 32.0f;
    static constexpr int PFK = D > 256 ? 3 : 4;
    static constexpr int PFV = D > 256 ? 2 : 3;
    static constexpr int PFV_EARLY = kPfvEarly;
    // The next stage's copies are spread evenly over the KS MFMAs of the score
    // product: a wave's memory instructions issue only as fast as the memory
    // pipeline drains, and a wave held up issuing a block of them leaves its MFMA
    // unit idle.  copy_at(i) = first copy issued at score step i.
    static constexpr int copy_at(int i) { return (i * RPW + KS - 1) / KS; }
    // end merge: each wavefront hands half its O tiles (DT/2) to its partner in NR
    // rounds of TPR tiles, 64 B per lane per tile, next to the staged bf16 output
    static constexpr int NR = DT / 2 > 1 ? 2 : 1;
    static constexpr int TPR = DT / 2 / NR;
    static constexpr int XR_BYTES = NW * TPR * 64 * 64;
    static constexpr int OUT_BYTES = HEADS * L::OUT_RS;  // staged bf16 output of the workgroup
    static constexpr int SMEM = std::max(NBUF * STAGE_BYTES, XR_BYTES + OUT_BYTES);
    static_assert(KS >= 4 && DT >= 2 && DT % 2 == 0 && RPW == 16 && PFV_EARLY <= PFV, "tiling");
};

template <int D, bool FUSED, bool SPLIT>
__global__ void __launch_bounds__(WideCfg<D>::THREADS, 1) sa_attn_wide(const AttnParams p) {
    using C = WideCfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
    __shared__ int list[kListCap];
    __shared__ int wcnt[kListCap / 64];
    __shared__ float mlx[2][2][32][2];  // end merge: [head tile][row half][head][max, sum]
    __shared__ int replay[2];
    __shared__ __attribute__((aligned(16))) float rtab[D];  // the query's rotation table row

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave values in SGPRs
    const int lane = tid & 63;
    const int hf = lane >> 5;  // which half of a 32-wide MFMA k (or m) block this lane feeds
    const int n = lane & 31;   // head (B / C column) or row (A row) of this lane
    const int hw = wave >> 1;  // head tile of this wavefront
    const int rh = wave & 1;   // row half of every stage this wavefront computes
    const bool chunk_lane = C::CH == 64 || lane < C::CH;

    uint32_t qi, j;
    if (!wide_unit(p, qi, j)) return;  // (uniform over the workgroup, before any barrier)
    const uint32_t sp = j % (uint32_t)p.n_sp;
    const uint32_t hg = j / (uint32_t)p.n_sp;
    const uint32_t bi = qi / (uint32_t)p.s;

    const int lo = (int)sp * p.split_len;
    const int hi = min(p.topk, lo + p.split_len);
    const int32_t *idxq = FUSED ? nullptr : p.idx + (int64_t)qi * p.topk;
    const ListForm lform = list_form<false>(p, qi);
    auto fetch = [&](int e) -> int { return FUSED ? step_entry(p, lform, qi, e) : idxq[e]; };
    // fused decode step: the new row's entry (window - 1) in this workgroup's range
    const bool has_new = FUSED && p.window - 1 >= lo && p.window - 1 < hi;
    u32x4_t new_raw = {0u, 0u, 0u, 0u};
    if (has_new && wave == 0 && chunk_lane)
        new_raw = *reinterpret_cast<const u32x4_t *>(p.kv_new + (int64_t)qi * D + lane * 8);
    // the first index chunk goes in flight before anything else: it heads the critical path
    Compactor<C::THREADS> cmp;
    if constexpr (FUSED)
        cmp.load_step(p, qi, lo, min(hi, lo + kListCap));
    else
        cmp.load(fetch, lo, min(hi, lo + kListCap));

    cmp.ready();
    if (has_new && wave == 0) {
        // the new row rounded through fp8 into its ring slot.  Every workgroup
        // whose list holds it writes the same bytes and gathers the slot only
        // after its own write is complete (the wait below, then the barrier in
        // pack), so each one reads its own write whatever L2 it sits behind.
        const u32x4_t r = fp8_round_trip_chunk(new_raw);
        if (chunk_lane)
            *reinterpret_cast<u32x4_t *>(p.kv_ring + ((int64_t)bi * p.rows + p.new_slot) * D + lane * 8) = r;
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    }

    const int head = ((int)hg * 2 + hw) * 32 + n;
    const bool head_ok = head < p.h;
    const uint32_t smem_base = lds_addr((const SA_LDS void *)smem);
    // the output rotation's table row for this query, ahead of the head-row copies
    // (so the wait for those covers it)
    const bool rot = p.rope != nullptr && p.n_sp == 1;
    if (rot && wave == 0) copy_rope_row(p, qi, lane, lds_addr((const SA_LDS void *)rtab));
    const SA_LDS char *lds = (const SA_LDS char *)smem;

    // the workgroup's 64 head rows of q, copied once into stage buffer 0 (wave w
    // copies rows 16 w .. 16 w + 15; heads past h get zero rows) and read into
    // registers once the first stage's copies are out -- both wavefronts of a head
    // tile need them, and a copy through LDS fetches them once.  Stage st uses
    // buffer (st + 1) % 2, so stage 0 does not overwrite them.
#pragma unroll 1
    for (int u = 0; u < C::RPW; ++u) {
        const int hl = wave * C::RPW + u;
        const int hd = (int)hg * C::HEADS + hl;
        if (hd < p.h) {
            if (chunk_lane)
                dma_16B_nt(p.q + ((int64_t)qi * p.h + hd) * D + (lane ^ C::L::swz(hl)) * 8, smem_base + hl * C::RS);
        } else if (chunk_lane) {
            *reinterpret_cast<SA_LDS u32x4_t *>((SA_LDS char *)smem + hl * C::RS + 16 * lane) =
                u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    // Q as the B operand: lane (hf, n) holds q[head n][16 ks + 8 hf .. +8] for every ks
    bf16x8_t qreg[C::KS];

    float m_ref = -1e30f;   // fixed reference max (log2 domain) the weights are taken against
    float m_seen = -1e30f;  // largest stage max seen
    float l_run = 0.0f;     // this lane's share of the running sum
    bool have_ref = false;  // m_ref set (wave-uniform)
    f32x16_t acc_o[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc_o[dt] = f32x16_t{};
    if (tid == 0) replay[0] = replay[1] = 0;  // read only after the barriers of pack

    const uint16_t *kvb = p.kv + (int64_t)bi * p.rows * D;
    // per-lane operand bases inside a stage buffer (see the two read patterns below)
    const int kb = C::L::kbase(32 * rh + n, hf);
    const int vlo = C::L::vbase(32 * rh, lane, false);
    const int vhi = C::L::vbase(32 * rh, lane, true);


    // The weights are taken against a fixed reference: the first stage max a wave
    // sees.  A later stage max may exceed it by up to SLACK (weights <= 2^SLACK, far
    // inside bf16 and f32 range), so O is never rescaled inside the loop (with O
    // and Q filling the register file there is no room to).  Should a stage max
    // outrun the reference by more, the workgroup replays the whole list against
    // the larger max -- correct for any input, and it does not occur for attention
    // logits of any realistic spread.  replay[st & 1] is raised during stage st and
    // read after the barrier that opens stage st+1; the two slots alternate, so a
    // read never races the next stage's writes.
    bool first_pass = true;
    for (bool again = true; again; first_pass = false) {
    again = false;
    for (int c0 = lo; c0 < hi; c0 += kListCap) {
        const int c1 = min(hi, c0 + kListCap);
        if (c0 != lo || !first_pass) {
            if constexpr (FUSED)
                cmp.load_step(p, qi, c0, c1);
            else
                cmp.load(fetch, c0, c1);
        }
        if (FUSED && first_pass && hg == 0 && p.idx_out) cmp.store(p.idx_out + (int64_t)qi * p.topk, c0, c1);
        const int nv = cmp.pack(p.rows, list, wcnt);
        const int nst = (nv + C::ROWS - 1) / C::ROWS;

        // copies of stage st into buffer (st + 1) % 2: this wave's RPW rows, one wave
        // instruction (one 16-byte chunk per lane of a row) each.  Lane u (< RPW)
        // holds the row of copy u; entries past the list end repeat its last row.
        auto stage_rows = [&](int st) -> int {
            const int e = st * C::ROWS + wave * C::RPW + (lane & 15);
            return list[e < nv ? e : nv - 1];
        };
        auto copy_rows = [&](int st, int rows_reg, int u0, int u1) {
            const uint32_t buf = smem_base + (uint32_t)(((st + 1) & 1) * C::STAGE_BYTES + wave * C::RPW * C::RS);
            for (int u = u0; u < u1; ++u) {
                const int row = __builtin_amdgcn_readlane(rows_reg, u);
                if (chunk_lane) dma_16B(kvb + (int64_t)row * D + (lane ^ C::L::swz(wave * C::RPW + u)) * 8, buf + u * C::RS);
            }
        };
        if (nv > 0) {
            const int r0 = stage_rows(0);
#pragma unroll 1
            for (int u = 0; u < C::RPW; ++u) copy_rows(0, r0, u, u + 1);
        }
        if (c0 == lo && first_pass) {
            // this wave's head-row copies are done (only stage 0's RPW copies may still
            // run); after the barrier, every wave's
            if (nv > 0)
                asm volatile("s_waitcnt vmcnt(%0)" : : "n"(C::RPW) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
            lds_barrier();
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                qreg[ks] = lds_read_b128(lds + C::L::koff(C::L::kbase(hw * 32 + n, hf), ks));
        }
        if (nv == 0) continue;

        for (int st = 0; st < nst; ++st) {
            asm volatile("s_waitcnt vmcnt(0)" : : : "memory");  // this wave's copies of stage st
            lds_barrier();  // everyone's copies in place; stage st-1 consumed, its buffer free
            // the previous stage's replay flag, tested after the score product (see
            // the pair kernel)
            const int replay_prev = st > 0 ? replay[(st - 1) & 1] : 0;
            const SA_LDS char *buf = lds + ((st + 1) & 1) * C::STAGE_BYTES;
            const bool more = st + 1 < nst;
            const int rows_next = more ? stage_rows(st + 1) : 0;

            // ---- scores S^T[32 rows][32 heads]: lane (hf, n) feeds row n, d chunk 2 ks + hf.
            //      Operand reads run four MFMAs ahead; the next stage's copies go out one
            //      or a few per k-step, so the wave is not held up issuing them in a block;
            //      the scheduling barriers keep the compiler from hoisting the reads ----
            f32x16_t sacc;
            {
                constexpr int PF = C::PFK;
                bf16x8_t kq[PF];
#pragma unroll
                for (int i = 0; i < PF; ++i) kq[i] = lds_read_b128(buf + C::L::koff(kb, i));
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    const bf16x8_t a = kq[ks % PF];
                    if (ks + PF < C::KS) kq[ks % PF] = lds_read_b128(buf + C::L::koff(kb, ks + PF));
                    if (more) copy_rows(st + 1, rows_next, C::copy_at(ks), C::copy_at(ks + 1));
                    if (ks == 0)
                        mfma_s_first(sacc, a, qreg[ks]);
                    else if (ks + 1 < C::KS)
                        mfma_s_next(sacc, a, qreg[ks]);
                    else
                        mfma_s_last(sacc, a, qreg[ks]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            if (replay_prev) break;
            // ---- weights and weighted sum of this wave's half of the stage ----
            slice_weights_pv<C>(sacc, st * C::ROWS + 32 * rh, nv, p.scale_log2, m_ref, m_seen, l_run, have_ref,
                                replay[st & 1], buf, vlo, vhi, acc_o);
        }
        lds_barrier();  // the last stage's flag is raised by now
        if (replay[0] | replay[1]) {
            again = true;
            break;
        }
    }
    if (again) {
        // start over against the larger reference (replay[] read by every wave above)
        lds_barrier();
        if (tid == 0) replay[0] = replay[1] = 0;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) acc_o[dt] = f32x16_t{};
        l_run = 0.0f;
    }
    }

    // ---- merge the two row halves of each head tile: M = max, O and l rescaled
    //      to M and added.  Wave rh finalises d tiles [rh DT/2, (rh+1) DT/2) and
    //      hands the other half of its O to its partner ----
    l_run = sum_xor32(l_run);  // the head's sum over this wave's rows
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");  // (an empty list leaves the head-row copies running)
    lds_barrier();                     // stage buffers free
    if (hf == 0) {
        mlx[hw][rh][n][0] = m_ref;
        mlx[hw][rh][n][1] = l_run;
    }
    lds_barrier();
    const float m_o = mlx[hw][rh ^ 1][n][0];
    const float l_o = mlx[hw][rh ^ 1][n][1];
    const float M = fmaxf(m_ref, m_o);
    const float f_s = exp2_fast(m_ref - M);
    const float f_o = exp2_fast(m_o - M);
    const float Ls = l_run * f_s + l_o * f_o;
    constexpr int DH2 = C::DT / 2;
    constexpr bool split = SPLIT;  // (a template parameter: the split-free build keeps no partial-store code)
    // output = (own O f_s + partner's O f_o) / (Ls + sink term); split partials
    // keep O unnormalised against M
    float a_s = f_s, a_o = f_o;
    if (!split) {
        const float sink_l2 = head_ok ? p.sink[head] * kLog2e : 0.f;
        const float Lt = Ls + exp2_fast(sink_l2 - M);
        const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;  // empty list: 0 / inf, or a guarded 0 / 0
        a_s *= inv;
        a_o *= inv;
    }
    SA_LDS char *xo = (SA_LDS char *)smem;
    SA_LDS char *stg = (SA_LDS char *)smem + C::XR_BYTES;  // staged bf16 output, clear of the exchange
    // The row half R finalises d tiles [R DT/2, (R+1) DT/2) (a template parameter:
    // register arrays take compile-time indices only).  The partner's share comes
    // through LDS in NR rounds of TPR tiles; each merged tile goes straight to its
    // destination (bf16 staging rows, or the split partials).
    auto finish = [&](auto RC) {
        constexpr int R = decltype(RC)::value;
#pragma unroll
        for (int r = 0; r < C::NR; ++r) {
            if (r > 0) lds_barrier();  // the previous round's exchange has been read
#pragma unroll
            for (int t = 0; t < C::TPR; ++t) {  // the partner's tiles of this round, as they stand
                const f32x16_t &v = acc_o[(1 - R) * DH2 + r * C::TPR + t];
                // [slot][quarter][lane] x 16 B: each wave instruction is 1 KiB contiguous
                SA_LDS f32x4_t *dst = reinterpret_cast<SA_LDS f32x4_t *>(xo + (wave * C::TPR + t) * 4096) + lane;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    dst[64 * q4] = f32x4_t{v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]};
            }
            lds_barrier();
#pragma unroll
            for (int t = 0; t < C::TPR; ++t) {  // own tiles: own a_s + partner's a_o
                const int k = R * DH2 + r * C::TPR + t;  // d tile
                const SA_LDS f32x4_t *src =
                    reinterpret_cast<const SA_LDS f32x4_t *>(xo + ((wave ^ 1) * C::TPR + t) * 4096) + lane;
                const f32x16_t &w = acc_o[k];
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const f32x4_t x = src[64 * qd];
                    const f32x4_t o = {fmaf(w[4 * qd], a_s, x[0] * a_o), fmaf(w[4 * qd + 1], a_s, x[1] * a_o),
                                       fmaf(w[4 * qd + 2], a_s, x[2] * a_o), fmaf(w[4 * qd + 3], a_s, x[3] * a_o)};
                    // lane (hf, n) holds head n, d = 32 k + 8 qd + 4 hf + (0..3)
                    if (split) {
                        if (head_ok)
                            *reinterpret_cast<f32x4_t *>(p.part_o +
                                                         (((int64_t)qi * p.n_sp + sp) * p.h + head) * D +
                                                         32 * k + 8 * qd + 4 * hf) = o;
                    } else {
                        *reinterpret_cast<SA_LDS u32x2_t *>(stg + (hw * 32 + n) * C::L::OUT_RS + 64 * k + 16 * qd + 8 * hf) =
                            u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    if (rh == 0)
        finish(std::integral_constant<int, 0>{});
    else
        finish(std::integral_constant<int, 1>{});
    if (split) {
        if (head_ok && hf == 0 && rh == 0) {
            const int64_t prow = ((int64_t)qi * p.n_sp + sp) * p.h + head;
            p.part_ml[prow * 2] = M;
            p.part_ml[prow * 2 + 1] = Ls;
        }
        return;
    }
    lds_barrier();
    // one head row per wave instruction: lane l stores chunk l (16 B) of the row
#pragma unroll 4
    for (int hr = wave; hr < C::HEADS; hr += C::NW) {
        const int hglob = (int)hg * C::HEADS + hr;
        if (hglob < p.h && chunk_lane) {
            u32x4_t v = *reinterpret_cast<const SA_LDS u32x4_t *>(stg + hr * C::L::OUT_RS + 16 * lane);
            if (rot) v = unrotate_chunk(v, 8 * lane, D, p.rope_dim, (const SA_LDS float *)rtab);
            store_16B_nt(p.out + ((int64_t)qi * p.h + hglob) * D + lane * 8, v);
        }
    }
}

// ------------------------------------------------------------------- pair --
//
// Pair kernel: one workgroup of two wavefronts per (query, 64 heads[, index
// split]), for grids of many workgroups (prefill).  Each wavefront owns a
// 32-head tile over the whole head dim (Q in registers, its 32 head rows copied
// by the wavefront itself through the stage buffers; O in accumulator
// registers) and walks
// every row of the list in 32-row stages: S^T[32 rows][32 heads] = K Q^T, the
// softmax against the fixed reference of the wide kernel, O^T[d][32 heads] +=
// V^T P^T, all on MFMA 32x32x16 with the operand layouts of the wide kernel.
// A wavefront thus ends with its heads' whole result: no merge between
// wavefronts.  With 32-row stages and a list chunk of up to 2176 entries the
// workgroup needs under 80 KiB of LDS, so two workgroups share a CU and the
// prologue (list compaction, Q loads) and epilogue (normalisation, stores) of
// one overlap the stages of the other.  The chunk capacity is a template
// parameter (the compaction's work grows with it): 512 for short lists, 2176
// for long ones (a 128 + 2048-entry list in one pass).
template <int D, int LCAP>
struct PairCfg {
    static constexpr int NW = 2;
    static constexpr int THREADS = 64 * NW;
    static constexpr int HEADS = 64;
    static constexpr int ROWS = 32;             // rows per stage (all of them, for each wavefront)
    static constexpr int RPW = ROWS / NW;       // rows each wavefront copies per stage
    using L = RowLayout<D>;
    static constexpr int RS = L::RS;            // stage rows as in the wide kernel
    static constexpr int CH = D / 8;
    static constexpr int KS = D / 16;
    static constexpr int DT = D / 32;
    static constexpr int STAGE_BYTES = ROWS * RS;
    static constexpr int NBUF = 2;
    static constexpr int LIST_CAP = LCAP;       // compacted entries held at once
    static constexpr int OUT_BYTES = HEADS * L::OUT_RS;  // staged bf16 output, over the stage buffers
    static constexpr int SMEM = std::max(NBUF * STAGE_BYTES, OUT_BYTES);
    static_assert(SMEM - OUT_BYTES >= 4 * D, "room for the rotation table row past the staged output");
    static constexpr float SLACK = 32.0f;
    static constexpr int PFK = 4;   // (the pair kernel's registers allow four at d = 512; the wide kernel's do not)
    static constexpr int PFV = D > 256 ? 2 : 3;
    static constexpr int PFV_EARLY = kPfvEarly;
    // the next stage's copies go out over the first quarter of the score product
    // (so they start their flight early; spreading them over half or all of it
    // measured the same once the rows come from L2)
    static constexpr int copy_at(int i) { return std::min(RPW, (4 * i * RPW + KS - 1) / KS); }
    static_assert(KS >= 4 && DT >= 2 && RPW == 16, "tiling");
};

template <int D, int LCAP, int MODE, bool SPLIT>
__global__ void __launch_bounds__(128, 2) sa_attn_pair(const AttnParams p) {
    using C = PairCfg<D, LCAP>;
    constexpr bool FUSED = MODE == 1;    // decode step: the list built in registers, the new row
    constexpr bool PREFILL = MODE == 2;  // prefill list: compressed positions copied, window by formula
    static_assert(C::THREADS == 128, "launch bounds");
    // Two workgroups share a CU.  Started together on lists of one length, they
    // would keep entering their HBM-bound phases (index list and Q in, output
    // out) at the same moments across the whole chip.  The second round of
    // workgroups (the CUs' second residency slot) starts a few microseconds
    // late; every later workgroup takes over the slot of one that ended, so the
    // two slots of a CU stay apart in phase for the rest of the grid and one
    // streams while the other computes.  (A bounded wait: two sleeps.)
    if (p.stagger_cu > 0 && blockIdx.x >= (uint32_t)p.stagger_cu && blockIdx.x < 2u * (uint32_t)p.stagger_cu) {
        __builtin_amdgcn_s_sleep(100);
        __builtin_amdgcn_s_sleep(100);
    }
    __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
    __shared__ int list[C::LIST_CAP];
    __shared__ int wcnt[C::LIST_CAP / 64];
    __shared__ int replay[2];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // head tile
    const int lane = tid & 63;
    const int hf = lane >> 5;
    const int n = lane & 31;
    const bool chunk_lane = C::CH == 64 || lane < C::CH;

    uint32_t qi, j;
    if (!wide_unit(p, qi, j)) return;  // (uniform over the workgroup, before any barrier)
    const uint32_t sp = j % (uint32_t)p.n_sp;
    const uint32_t hg = j / (uint32_t)p.n_sp;
    const uint32_t bi = qi / (uint32_t)p.s;

    const int lo = (int)sp * p.split_len;
    const int hi = min(p.topk, lo + p.split_len);
    const int32_t *idxq = MODE == 0 ? p.idx + (int64_t)qi * p.topk : nullptr;
    const int32_t *cq = PREFILL ? p.cidx + (int64_t)qi * p.kc - p.window : nullptr;  // entry e >= window: cq[e]
    const bool has_new = FUSED && p.window - 1 >= lo && p.window - 1 < hi;
    u32x4_t new_raw = {0u, 0u, 0u, 0u};
    if (has_new && wave == 0 && chunk_lane)
        new_raw = *reinterpret_cast<const u32x4_t *>(p.kv_new + (int64_t)qi * D + lane * 8);
    // Index entries, the head of the critical path.  The fused step builds them in
    // place.  Otherwise a chunk's raw entries are copied global -> list[]
    // directly (4 bytes a lane, 64 entries a wave instruction, entry e at
    // list[e - c0]): Q's copies then go out right behind them, and the wait for
    // the entries (vmcnt counts completions in issue order) leaves Q in flight --
    // the two memory round trips overlap instead of following each other.  The
    // prefill list copies only its compressed positions that way; its window
    // entries are formed when the entries are read back.
    Compactor<C::THREADS, C::LIST_CAP> cmp;
    const uint32_t list_base = lds_addr((const SA_LDS void *)list);
    auto copy_idx = [&](int c0, int c1) {
        if constexpr (PREFILL) {
#pragma unroll 1
            for (int e0 = max(c0, p.window) + wave * 64; e0 < c1; e0 += C::THREADS)
                if (e0 + lane < c1) dma_4B(cq + e0 + lane, list_base + (uint32_t)(e0 - c0) * 4);
            // the window entries by formula, stored beside them (the barrier before
            // the read-back publishes both)
            const ListForm f = list_form<true>(p, qi);
            for (int e = c0 + tid; e < min(c1, p.window); e += C::THREADS) list[e - c0] = window_entry(f, e);
        } else {
#pragma unroll 1
            for (int e0 = c0 + wave * 64; e0 < c1; e0 += C::THREADS)
                if (e0 + lane < c1) dma_4B(idxq + e0 + lane, list_base + (uint32_t)(e0 - c0) * 4);
        }
    };
    if (FUSED)
        cmp.load_step(p, qi, lo, min(hi, lo + C::LIST_CAP));
    else
        copy_idx(lo, min(hi, lo + C::LIST_CAP));
    const int head = ((int)hg * 2 + wave) * 32 + n;
    const bool head_ok = head < p.h;
    // the head's sink, ahead of Q's copies (a load issued behind the copies waits for them)
    const float sink_any = p.sink[min(head, p.h - 1)];

    if (FUSED) cmp.ready();
    // the output's inverse rotation: the query's table row is copied in the
    // epilogue, past the staged output rows (the stage buffers hold Q and rows
    // until then; no LDS of its own, which leaves room for a 2304-entry list)
    const bool rot = p.rope != nullptr && p.n_sp == 1;
    // Q rows: wave w copies its own 32 head rows (one 1 KiB row per wave
    // instruction) into rows 32 w .. 32 w + 31 of the stage buffers, to be read
    // into registers once the list is packed; a head past h takes row 0 of the
    // query (its column of S and O is never stored)
    const uint32_t smem_base = lds_addr((const SA_LDS void *)smem);
#pragma unroll 1
    for (int u = 0; u < 32; ++u) {
        const int hd = ((int)hg * 2 + wave) * 32 + u;
        if (chunk_lane)
            dma_16B_nt(p.q + ((int64_t)qi * p.h + (hd < p.h ? hd : 0)) * D + (lane ^ C::L::swz(u)) * 8,
                    smem_base + (uint32_t)((wave * 32 + u) * C::RS));
    }
    if (has_new && wave == 0) {
        // the new row rounded through fp8 into its ring slot (as in the wide kernel)
        const u32x4_t r = fp8_round_trip_chunk(new_raw);
        if (chunk_lane)
            *reinterpret_cast<u32x4_t *>(p.kv_ring + ((int64_t)bi * p.rows + p.new_slot) * D + lane * 8) = r;
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    }
    const SA_LDS char *lds = (const SA_LDS char *)smem;

    float m_ref = -1e30f;
    float m_seen = -1e30f;
    float l_run = 0.0f;
    bool have_ref = false;
    f32x16_t acc_o[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc_o[dt] = f32x16_t{};
    if (tid == 0) replay[0] = replay[1] = 0;  // read only after the barriers of pack
    // Q as the B operand: lane (hf, n) holds q[head n][16 ks + 8 hf .. +8] for every ks
    bf16x8_t qreg[C::KS];

    const uint16_t *kvb = p.kv + (int64_t)bi * p.rows * D;
    const int kb = C::L::kbase(n, hf);
    const int vlo = C::L::vbase(0, lane, false);
    const int vhi = C::L::vbase(0, lane, true);

    // weights against a fixed reference max, with a whole-list replay should a
    // stage max outrun it by more than SLACK (see the wide kernel)
    bool first_pass = true;
    for (bool again = true; again; first_pass = false) {
    again = false;
    for (int c0 = lo; c0 < hi; c0 += C::LIST_CAP) {
        const int c1 = min(hi, c0 + C::LIST_CAP);
        if (c0 != lo || !first_pass) {
            if (FUSED)
                cmp.load_step(p, qi, c0, c1);
            else
                copy_idx(c0, c1);
        }
        if (!FUSED) {
            // this wave's entry copies are in (on the first chunk Q's 32 copies,
            // issued behind them, may still fly); then everyone's
            if (c0 == lo && first_pass)
                asm volatile("s_waitcnt vmcnt(32)" : : : "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
            lds_barrier();
            if constexpr (PREFILL)
                cmp.load_lds_prefill(list, c0, c1, p.window, p.s);
            else
                cmp.load_lds(list, c0, c1);
        }
        if ((FUSED || PREFILL) && first_pass && hg == 0 && p.idx_out)
            cmp.store(p.idx_out + (int64_t)qi * p.topk, c0, c1);
        const int nv = cmp.pack(p.rows, list, wcnt);
        const int nst = (nv + C::ROWS - 1) / C::ROWS;
        if (c0 == lo && first_pass) {
            // this wave's head rows have landed: into registers, then free the buffers
            asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                qreg[ks] = lds_read_b128(lds + C::L::koff(C::L::kbase(wave * 32 + n, hf), ks));
            lds_barrier();
        }
        if (nv == 0) continue;

        // copies of stage st into buffer st % 2: this wave's RPW rows, one wave
        // instruction each; lane u (< RPW) holds the row of copy u, entries past
        // the list end repeat its last row
        auto stage_rows = [&](int st) -> int {
            const int e = st * C::ROWS + wave * C::RPW + (lane & 15);
            return list[e < nv ? e : nv - 1];
        };
        auto copy_rows = [&](int st, int rows_reg, int u0, int u1) {
            const uint32_t buf = smem_base + (uint32_t)((st & 1) * C::STAGE_BYTES + wave * C::RPW * C::RS);
            for (int u = u0; u < u1; ++u) {
                const int row = __builtin_amdgcn_readlane(rows_reg, u);
                if (chunk_lane) dma_16B(kvb + (int64_t)row * D + (lane ^ C::L::swz(wave * C::RPW + u)) * 8, buf + u * C::RS);
            }
        };
        {
            const int r0 = stage_rows(0);
#pragma unroll 1
            for (int u = 0; u < C::RPW; ++u) copy_rows(0, r0, u, u + 1);
        }

        for (int st = 0; st < nst; ++st) {
            asm volatile("s_waitcnt vmcnt(0)" : : : "memory");  // this wave's copies of stage st
            lds_barrier();  // both waves' copies in place; stage st-1 consumed, its buffer free
            // the previous stage's replay flag: read here, tested after the score
            // product, so the LDS round trip overlaps it.  Copies of the next stage
            // issued before a break land before any buffer is reused: the list
            // chunk that restarts the pass waits for all of this wave's copies.
            const int replay_prev = st > 0 ? replay[(st - 1) & 1] : 0;
            const SA_LDS char *buf = lds + (st & 1) * C::STAGE_BYTES;
            const bool more = st + 1 < nst;
            const int rows_next = more ? stage_rows(st + 1) : 0;

            // ---- scores S^T[32 rows][32 heads]; the next stage's copies spread over them ----
            f32x16_t sacc;
            {
                constexpr int PF = C::PFK;
                bf16x8_t kq[PF];
#pragma unroll
                for (int i = 0; i < PF; ++i) kq[i] = lds_read_b128(buf + C::L::koff(kb, i));
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    const bf16x8_t a = kq[ks % PF];
                    if (ks + PF < C::KS) kq[ks % PF] = lds_read_b128(buf + C::L::koff(kb, ks + PF));
                    if (more) copy_rows(st + 1, rows_next, C::copy_at(ks), C::copy_at(ks + 1));
                    if (ks == 0)
                        mfma_s_first(sacc, a, qreg[ks]);
                    else if (ks + 1 < C::KS)
                        mfma_s_next(sacc, a, qreg[ks]);
                    else
                        mfma_s_last(sacc, a, qreg[ks]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            if (replay_prev) break;
            // ---- weights and weighted sum of the stage ----
            slice_weights_pv<C>(sacc, st * C::ROWS, nv, p.scale_log2, m_ref, m_seen, l_run, have_ref, replay[st & 1],
                                buf, vlo, vhi, acc_o);
        }
        lds_barrier();  // the last stage's flag is raised by now
        if (replay[0] | replay[1]) {
            again = true;
            break;
        }
    }
    if (again) {
        lds_barrier();
        if (tid == 0) replay[0] = replay[1] = 0;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) acc_o[dt] = f32x16_t{};
        l_run = 0.0f;
    }
    }

    // ---- sink fold + normalise (or f32 partials), stage bf16 rows, store a row per instruction ----
    l_run = sum_xor32(l_run);  // the head's sum over all rows
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    constexpr bool split = SPLIT;  // (a template parameter: the split-free build keeps no partial-store code)
    if (split) {
        if (head_ok) {
            const int64_t prow = ((int64_t)qi * p.n_sp + sp) * p.h + head;
#pragma unroll
            for (int k = 0; k < C::DT; ++k) {
#pragma unroll
                for (int qd = 0; qd < 4; ++qd)
                    *reinterpret_cast<f32x4_t *>(p.part_o + prow * D + 32 * k + 8 * qd + 4 * hf) =
                        f32x4_t{acc_o[k][4 * qd], acc_o[k][4 * qd + 1], acc_o[k][4 * qd + 2], acc_o[k][4 * qd + 3]};
                __builtin_amdgcn_sched_barrier(0);  // one tile out of the accumulators at a time
            }
            if (hf == 0) {
                p.part_ml[prow * 2] = m_ref;
                p.part_ml[prow * 2 + 1] = l_run;
            }
        }
        return;
    }
    const float sink_l2 = head_ok ? sink_any * kLog2e : 0.f;
    const float Lt = l_run + exp2_fast(sink_l2 - m_ref);
    const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;
    lds_barrier();  // stage buffers free
    SA_LDS char *stg = (SA_LDS char *)smem;
    const SA_LDS float *rtab = (const SA_LDS float *)(stg + C::OUT_BYTES);
    if (rot && wave == 0) copy_rope_row(p, qi, lane, smem_base + (uint32_t)C::OUT_BYTES);
#pragma unroll
    for (int k = 0; k < C::DT; ++k) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            // lane (hf, n) holds head n, d = 32 k + 8 qd + 4 hf + (0..3)
            const f32x16_t &w = acc_o[k];
            *reinterpret_cast<SA_LDS u32x2_t *>(stg + (wave * 32 + n) * C::L::OUT_RS + 64 * k + 16 * qd + 8 * hf) =
                u32x2_t{pack_bf16x2(w[4 * qd] * inv, w[4 * qd + 1] * inv),
                        pack_bf16x2(w[4 * qd + 2] * inv, w[4 * qd + 3] * inv)};
        }
        // one tile out of the accumulators at a time: reads of all of them hoisted
        // ahead would need as many vector registers again and spill
        __builtin_amdgcn_sched_barrier(0);
    }
    if (rot && wave == 0) asm volatile("s_waitcnt vmcnt(0)" : : : "memory");  // the table row is in
    lds_barrier();
    // one head row per wave instruction (lane l: chunk l), in batches of 8 rows
    // whose LDS reads all go out before their stores
#pragma unroll 1
    for (int r0 = wave; r0 < C::HEADS; r0 += 8 * C::NW) {
        u32x4_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = *reinterpret_cast<const SA_LDS u32x4_t *>(stg + (r0 + i * C::NW) * C::L::OUT_RS + 16 * lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int hr = r0 + i * C::NW;
            const int hglob = (int)hg * C::HEADS + hr;
            if (hglob < p.h && chunk_lane) {
                u32x4_t w = v[i];
                if (rot) w = unrotate_chunk(w, 8 * lane, D, p.rope_dim, rtab);
                store_16B_nt(p.out + ((int64_t)qi * p.h + hglob) * D + lane * 8, w);
            }
        }
    }
}

// ------------------------------------------------------------------ decode --
//
// Decode kernel: one workgroup of four wavefronts per (query, group of 16
// heads), for decode-sized batches.  The query's 16 head rows are copied into
// LDS once per workgroup (every wavefront needs all of them), and the index
// list is walked in 64-entry stages two buffers deep, so the rows of stage t+1
// arrive while stage t is computed.  Each wavefront copies the rows of its 16
// entries of a stage straight from its index registers (a zero row for a -1
// entry, which then contributes nothing), so no list compaction sits on the
// latency path.  The wavefronts split the rows for the scores (S^T[16 rows][16
// heads] each, MFMA 16x16x32), exchange the per-head maxima and the bf16
// weights P through LDS, then split the head dim for O^T[d/4][16 heads] =
// V^T P^T over all the stage's rows.  Every gathered row is read from LDS once
// as K and once as V, and no partial result leaves the workgroup.
template <int D>
struct DecodeCfg {
    static constexpr int NW = 4;
    static constexpr int THREADS = 64 * NW;
    static constexpr int HEADS = 16;
    static constexpr int ROWS = 64;               // index entries per stage
    static constexpr int RPW = ROWS / NW;         // entries (rows) each wavefront copies per stage
    static constexpr int ROW_BYTES = 2 * D;
    static constexpr int RS = ROW_BYTES + 48;     // padded LDS row stride (bank position 3 r + c)
    static constexpr int CH = D / 8;              // 16-byte chunks per row
    static constexpr int KS = D / 32;             // k-steps of the score product (16x16x32)
    static constexpr int DQ = D / NW;             // head-dim share of one wavefront in the weighted sum
    static constexpr int DT = DQ / 16;            // its 16-wide d tiles
    static constexpr int PRS = 2 * ROWS + 16;     // padded row stride of the weight buffer P[head][row]
    static constexpr int STAGE_BYTES = ROWS * RS;
    static constexpr int Q_BYTES = HEADS * RS;
    // kv8: a row's codes are D bytes, CPR8 16-byte chunks, RPI8 rows per copy
    // instruction; a stage lands in an fp8 staging buffer (codes, then the rows'
    // 16-byte scale records) and is expanded into the one bf16 stage buffer
    static constexpr int CPR8 = D / 16;
    static constexpr int RPI8 = 64 / CPR8;
    static constexpr int NCI8 = RPW / RPI8;       // code copies per wave per stage (+1 for the scales)
    static constexpr int STG8 = ROWS * D + ROWS * 16;
    static constexpr int RPR = 64 / (D / 8);     // rows a wavefront expands per round (one chunk per lane)
    static constexpr int XPW = RPW / RPR;         // expansion rounds per wavefront and stage (its own rows)
    static_assert(KS >= 2 && KS % 2 == 0 && DT >= 1 && RPW == 16, "tiling");
    static_assert(NCI8 >= 1 && (D / 8) <= 64 && XPW >= 1 && XPW * RPR == RPW, "kv8 tiling");
};

template <int D, bool FUSED, bool KV8>
__global__ void __launch_bounds__(256, 1) sa_attn_decode(const AttnParams p) {
    using C = DecodeCfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem[(KV8 ? 1 : 2) * C::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) char stg8[KV8 ? 2 * C::STG8 : 16];
    __shared__ __attribute__((aligned(16))) char qbuf[C::Q_BYTES];
    __shared__ __attribute__((aligned(16))) char pbuf[C::HEADS * C::PRS];
    __shared__ float smax[C::NW][16];
    __shared__ float ssum[C::NW][16];
    __shared__ __attribute__((aligned(16))) float rtab[D];  // the query's rotation table row
    __shared__ __attribute__((aligned(16))) char newbuf[KV8 && FUSED ? 2 * D : 16];  // kv8 step: the raw new row

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave values in SGPRs
    const int lane = tid & 63;
    const int g = lane >> 4;  // 16-lane group: k (or m) block of a 16x16x32 operand
    const int n = lane & 15;  // head (B / C column) or row (A row)
    const bool chunk_lane = C::CH == 64 || lane < C::CH;  // lanes that carry a 16-byte chunk of a row

    const uint32_t L = logical_wg((uint32_t)p.total_wg);
    const uint32_t sp = L % (uint32_t)p.n_sp;
    const uint32_t t2 = L / (uint32_t)p.n_sp;
    const uint32_t hg = t2 % (uint32_t)p.n_hg;
    const uint32_t qi = t2 / (uint32_t)p.n_hg;
    const uint32_t bi = qi / (uint32_t)p.s;

    const int lo = (int)sp * p.split_len;
    const int hi = min(p.topk, lo + p.split_len);
    const int nst = hi > lo ? (hi - lo + C::ROWS - 1) / C::ROWS : 0;
    const int32_t *idxq = FUSED ? nullptr : p.idx + (int64_t)qi * p.topk;

    // this wave's 16 entries of a stage sit in lanes 0..15 (mirrored in the other
    // lane groups); the first three stages' go in flight before anything else
    const int head = (int)hg * C::HEADS + n;
    const bool head_ok = head < p.h;
    // the head's sink, loaded before any copy goes out (a load issued after them
    // would wait behind them at the end), unconditionally from a clamped address
    // with the value masked afterwards: under a per-lane condition the compiler
    // put the scaling of the value right behind the load in the same branch, so
    // the load's whole round trip stood before the first copy (fp8-resident step
    // 2.3% slower, the bf16 one 1.1%)
    const float sink_any = p.sink[min(head, p.h - 1)];
    const float sink_h = (head_ok && p.n_sp == 1) ? sink_any : 0.0f;
    const bool rot = p.rope != nullptr && p.n_sp == 1 && nst > 0;
    const int eoff = C::RPW * wave + (lane & 15);
    // (a readable dummy for a load whose value is not needed: the sink)
    const int32_t *dummy = reinterpret_cast<const int32_t *>(p.sink);
    const ListForm lform = list_form<false>(p, qi);
    auto fetch_stage = [&](int j) -> int {
        const int e = lo + j * C::ROWS + eoff;
        return e < hi ? step_entry(p, lform, qi, e) : -1;
    };
    // An index-list entry fetched ahead inside the stage loop is split into its
    // load (load_entry, from a clamped address so that the load is unconditional)
    // and its range check (finish_entry), done only at a later stage, after that
    // stage's wait: a use right behind the load would make the compiler wait for
    // it there, and that wait would also cover the row copies issued after it.
    // (The fused step fetches its entries whole: its window entries are computed,
    // not loaded, and splitting them measured slower there.)
    auto load_entry = [&](int j) -> int {
        if (FUSED) return fetch_stage(j);
        const int e = lo + j * C::ROWS + eoff;
        return *(hi > lo ? idxq + min(e, hi - 1) : dummy);
    };
    auto finish_entry = [&](int j, int v) -> int {
        if (FUSED) return v;
        return lo + j * C::ROWS + eoff < hi ? v : -1;
    };
    // The first three stages' entries (stage 2's loaded, not yet checked).  Index
    // lists: the loads go out together inside one uniform branch, so one memory
    // latency covers them.
    int v0, v_up, v_after;  // entries of stages 0, 1 (the next to copy), 2
    if (FUSED) {
        v0 = fetch_stage(0);
        v_up = fetch_stage(1);
        v_after = fetch_stage(2);
    } else {
        const int e0 = lo + eoff, e1 = e0 + C::ROWS, e2 = e0 + 2 * C::ROWS;
        int a0 = -1, a1 = -1, a2 = -1;
        if (hi > lo) {
            a0 = idxq[min(e0, hi - 1)];
            a1 = idxq[min(e1, hi - 1)];
            a2 = idxq[min(e2, hi - 1)];
        }
        v0 = e0 < hi ? a0 : -1;
        v_up = e1 < hi ? a1 : -1;
        v_after = a2;
    }
    // the entries are in registers before any copy goes out: a compiler-placed wait
    // for them after the copies would also wait for the copies
    asm volatile("" : : "v"(v0), "v"(v_up), "v"(v_after));

    // fused step: the new row (list entry window - 1) is copied raw like any other
    // row (from kv_new instead of the ring), then rounded through fp8 in LDS by the
    // wavefront that copied it; head group 0 writes it into its ring slot at the end
    const int e_new = FUSED ? p.window - 1 - lo : -1;  // offset in this range
    const bool has_new = FUSED && e_new >= 0 && lo + e_new < hi;
    const int st_new = has_new ? e_new / C::ROWS : -1;
    const int w_new = has_new ? (e_new % C::ROWS) / C::RPW : -1;
    const int u_new = has_new ? e_new % C::RPW : 0;

    const uint16_t *kvb = KV8 ? nullptr : p.kv + (int64_t)bi * p.rows * D;
    const uint8_t *kcb = KV8 ? p.kv8c + (int64_t)bi * p.rows * D : nullptr;
    const uint8_t *ksb = KV8 ? p.kv8s + (int64_t)bi * p.rows * 16 : nullptr;
    const uint32_t smem_base = lds_addr((const SA_LDS void *)smem);
    const uint32_t stg8_base = lds_addr((const SA_LDS void *)stg8);
    const uint32_t q_base = lds_addr((const SA_LDS void *)qbuf);
    const SA_LDS char *lds = (const SA_LDS char *)smem;

    // kv8 fused step: the new row never passes through the fp8 staging.  Wave
    // w_new copies it raw into newbuf with its first copies (a direct copy like
    // the others: a register load would get a wait of the compiler's own, which
    // would also wait for every copy issued before its first use); the lanes that
    // expand its chunks (row u_new of the wave's rows in stage st_new: expansion
    // round k_new) read it there, round it through fp8 in registers and write both
    // the bf16 values (into the stage) and the codes (into the ring, head group 0,
    // at the end)
    const int k_new = u_new / C::RPR;
    const bool holds_new = KV8 && has_new && wave == w_new && lane / (D / 8) == u_new % C::RPR;
    u32x2_t new_codes = {0u, 0u};
    uint32_t new_sb = 127;

    // fused step, head group 0: the list written out
    auto store_idx = [&](int j, int v) {
        const int e = lo + j * C::ROWS + eoff;
        if (FUSED && hg == 0 && p.idx_out && lane < 16 && e < hi) p.idx_out[(int64_t)qi * p.topk + e] = v;
    };
    // Copies of stage j into buffer j % 2: this wave's RPW rows, one wave
    // instruction (one 16-byte chunk per lane of a row) each.  prep() takes the
    // valid mask (bit u: row RPW wave + u) and puts row u's source address in lane
    // u; copy_rows() sends rows [u0, u1).  A wave's memory instructions issue at the
    // memory pipeline's pace, so the next stage's copies are spread over this
    // stage's score product instead of holding the wave up in one block.
    auto prep = [&](int j, int v, uint32_t &okm, uint64_t &src) {
        const bool ok = v >= 0 && (int64_t)v < p.rows;
        okm = (uint32_t)__ballot(ok) & 0xffffu;
        const int u_src_new = (has_new && j == st_new && wave == w_new) ? u_new : -1;
        src = (lane & 15) == u_src_new ? (uint64_t)(p.kv_new + (int64_t)qi * D)
                                       : (uint64_t)(kvb + (int64_t)(ok ? v : 0) * D);
    };
    auto copy_rows = [&](int j, uint32_t okm, uint64_t src, int u0, int u1) {
        const uint32_t buf = smem_base + (uint32_t)((j & 1) * C::STAGE_BYTES + wave * C::RPW * C::RS);
        for (int u = u0; u < u1; ++u) {
            if ((okm >> u) & 1) {
                const uint64_t a = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)(src >> 32), u) << 32) |
                                   (uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)src, u);
                if (chunk_lane) dma_16B(reinterpret_cast<const char *>(a) + 16 * lane, buf + u * C::RS);
            } else if (chunk_lane) {
                *reinterpret_cast<SA_LDS u32x4_t *>((SA_LDS char *)smem + (j & 1) * C::STAGE_BYTES +
                                                    (wave * C::RPW + u) * C::RS + 16 * lane) = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
    };

    // kv8 copies of stage j into staging buffer j % 2: instruction i < NCI8 carries
    // RPI8 rows' codes (lane l: row i RPI8 + l / CPR8 of this wave, chunk l % CPR8),
    // instruction NCI8 the 16 rows' scale records (lane u < 16: row u).  Lanes of an
    // invalid row write zero codes (scale 2^0) instead; the fused step's new row is
    // left to the threads that hold it.
    auto copy8 = [&](int j, uint32_t okm, int rowv, int i0, int i1) {
        const int sbuf = (j & 1) * C::STG8;
        for (int i = i0; i < i1; ++i) {
            if (i < C::NCI8) {
                const int u = i * C::RPI8 + lane / C::CPR8;
                const int row = __shfl(rowv, u, 64);
                const bool live = ((okm >> u) & 1) && !(FUSED && has_new && j == st_new && wave == w_new && u == u_new);
                const int off = sbuf + (wave * C::RPW + i * C::RPI8) * D;
                if (live)
                    dma_16B(kcb + (int64_t)row * D + 16 * (lane % C::CPR8),
                            __builtin_amdgcn_readfirstlane(stg8_base + off));
                else
                    *reinterpret_cast<SA_LDS u32x4_t *>((SA_LDS char *)stg8 + off + 16 * lane) = u32x4_t{0u, 0u, 0u, 0u};
            } else if (lane < 16) {
                const bool live = ((okm >> lane) & 1) && !(FUSED && has_new && j == st_new && wave == w_new && lane == u_new);
                const int off = sbuf + C::ROWS * D + wave * C::RPW * 16;
                if (live)
                    dma_16B(ksb + (int64_t)rowv * 16, __builtin_amdgcn_readfirstlane(stg8_base + off));
                else
                    *reinterpret_cast<SA_LDS u32x4_t *>((SA_LDS char *)stg8 + off + 16 * lane) =
                        u32x4_t{0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu};
            }
        }
    };
    auto prep8 = [&](int v, uint32_t &okm, int &rowv) {
        const bool ok = v >= 0 && (int64_t)v < p.rows;
        okm = (uint32_t)__ballot(ok) & 0xffffu;
        rowv = ok ? v : 0;
    };

    uint32_t okm_cur = 0, okm_nxt = 0;
    uint64_t src_nxt = 0;
    int rowv_nxt = 0;
    int n_early = 0;  // bf16 rows: stage 1's copies, issued in the prologue
    if (nst > 0) {
        store_idx(0, v0);
        // the output rotation's table row for this query (the first stage's wait covers it)
        if (rot && wave == 0) copy_rope_row(p, qi, lane, lds_addr((const SA_LDS void *)rtab));
        // the query's head rows, once per workgroup: wavefront w copies heads 4w .. 4w+3
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int hl = 4 * wave + u;
            const int head = (int)hg * C::HEADS + hl;
            if (head < p.h) {
                if (chunk_lane)
                    dma_16B_nt(p.q + ((int64_t)qi * p.h + head) * D + lane * 8,
                            __builtin_amdgcn_readfirstlane(q_base + hl * C::RS));
            } else if (chunk_lane) {
                *reinterpret_cast<SA_LDS u32x4_t *>((SA_LDS char *)qbuf + hl * C::RS + 16 * lane) =
                    u32x4_t{0u, 0u, 0u, 0u};
            }
        }
        if constexpr (KV8) {
            if (FUSED && has_new && wave == w_new && chunk_lane)
                dma_16B(p.kv_new + (int64_t)qi * D + lane * 8,
                        __builtin_amdgcn_readfirstlane(lds_addr((const SA_LDS void *)newbuf)));
            int rowv0;
            prep8(v0, okm_cur, rowv0);
#pragma unroll 1
            for (int i = 0; i <= C::NCI8; ++i) copy8(0, okm_cur, rowv0, i, i + 1);
        } else {
            uint64_t src0;
            prep(0, v0, okm_cur, src0);
#pragma unroll 1
            for (int u = 0; u < C::RPW; ++u) copy_rows(0, okm_cur, src0, u, u + 1);
            if (nst > 1) {
                // stage 1 goes out right behind stage 0 (its buffer is free): the
                // copies are all in flight before any compute, and stage 0's score
                // product runs without copy issue in between
                store_idx(1, v_up);
                prep(1, v_up, okm_nxt, src_nxt);
#pragma unroll 1
                for (int u = 0; u < C::RPW; ++u) copy_rows(1, okm_nxt, src_nxt, u, u + 1);
                n_early = __builtin_popcount(okm_nxt);  // stage 1's copies (rows of -1 are zero-filled instead)
                v_up = finish_entry(2, v_after);         // entries of stage 2 (stage 3's are fetched later)
            }
        }
    }

    bf16x8_t qreg[C::KS];
    float m_ref = -1e30f;  // reference max (log2 domain), identical in all four wavefronts
    float l_run = 0.0f;    // this lane's share of the running sum over this wave's rows
    f32x4_t acc_o[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc_o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t new_row = {0u, 0u, 0u, 0u};
    constexpr int CPI = C::RPW / (C::KS / 2);  // next-stage copies per score iteration

    for (int t = 0; t < nst; ++t) {
        const int ebase = lo + t * C::ROWS;
        const SA_LDS char *stage = lds + (KV8 ? 0 : (t & 1) * C::STAGE_BYTES);
        // ---- this wave's copies of stage t complete (at stage 0 of the bf16 rows,
        //      stage 1's copies behind them may still fly) ----
        if (!KV8 && t == 0 && nst > 1)
            wait_vmcnt_upto16(n_early);
        else
            asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
        if (!KV8 && FUSED && t == st_new && wave == w_new) {
            // the raw new row has landed: round it through fp8 in place
            SA_LDS u32x4_t *nr = reinterpret_cast<SA_LDS u32x4_t *>((SA_LDS char *)stage +
                                                                      (wave * C::RPW + u_new) * C::RS + 16 * lane);
            const u32x4_t raw = chunk_lane ? *nr : u32x4_t{0u, 0u, 0u, 0u};
            new_row = fp8_round_trip_chunk(raw);
            if (chunk_lane) *nr = new_row;
        }
        lds_barrier();  // every wave's rows (and the head rows) in place; stage t-1 fully consumed
        if constexpr (KV8) {
            // ---- expand this wave's rows of the stage (the ones it copied) into the
            //      bf16 stage buffer.  Its score product reads only these; the other
            //      waves' rows are read (as V) after the barrier that publishes the
            //      maxima, so no barrier is needed here. ----
            const SA_LDS char *s8 = (const SA_LDS char *)stg8 + (t & 1) * C::STG8;
            u32x4_t nb = {0u, 0u, 0u, 0u};
            if (FUSED && has_new && t == st_new && wave == w_new) {  // wave-uniform: every lane rounds
                const u32x4_t new_raw = holds_new ? *reinterpret_cast<const SA_LDS u32x4_t *>(
                                                        (const SA_LDS char *)newbuf + 16 * (lane % (D / 8)))
                                                  : u32x4_t{0u, 0u, 0u, 0u};
                float e[8];
                const float sc = fp8_block_round(new_raw, e);
#pragma unroll
                for (int i = 0; i < 4; ++i) nb[i] = pack_bf16x2(e[2 * i] * sc, e[2 * i + 1] * sc);
                new_sb = __float_as_uint(sc) >> 23;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    new_codes[jj] = e4m3_code(e[4 * jj]) | (e4m3_code(e[4 * jj + 1]) << 8) |
                                    (e4m3_code(e[4 * jj + 2]) << 16) | (e4m3_code(e[4 * jj + 3]) << 24);
            }
#pragma unroll
            for (int k = 0; k < C::XPW; ++k) {
                const int r = C::RPW * wave + k * C::RPR + lane / (D / 8), c = lane % (D / 8);
                u32x4_t o;
                if (FUSED && holds_new && t == st_new && k == k_new) {
                    o = nb;
                } else {
                    const u32x2_t cd = *reinterpret_cast<const SA_LDS u32x2_t *>(s8 + r * D + 8 * c);
                    const uint32_t sb = *reinterpret_cast<const SA_LDS uint8_t *>(s8 + C::ROWS * D + r * 16 + c / 4);
                    o = kv8_expand(cd, sb);
                }
                *reinterpret_cast<SA_LDS u32x4_t *>((SA_LDS char *)smem + r * C::RS + 16 * c) = o;
            }
        }
        const bool more = t + 1 < nst;  // stage t+1 goes into the buffer stage t-1 used
        const bool issue = more && (KV8 || t > 0);  // (bf16 rows: stage 1 went out in the prologue)
        if (issue) {
            store_idx(t + 1, v_up);
            if constexpr (KV8)
                prep8(v_up, okm_nxt, rowv_nxt);
            else
                prep(t + 1, v_up, okm_nxt, src_nxt);
        }
        // The entries three stages ahead are loaded here, not after the score
        // product: a branch between the last score MFMA and the reads of its
        // result hid that dependency from the compiler's wait-state insertion,
        // and the reads came after fewer wait states than the matrix unit needs.
        if (more) {
            if (issue) v_up = finish_entry(t + 2, v_after);  // (bf16 rows: done in the prologue for stage 0)
            v_after = load_entry(t + 3);
        }
        if (t == 0) {
            // Q as the B operand of the scores: lane (g, n) holds q[head n][32 ks + 8 g .. +8]
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                qreg[ks] = lds_read_b128((const SA_LDS char *)qbuf + n * C::RS + 64 * ks + 16 * g);
        }

        // ---- scores S^T for this wave's 16 rows: two accumulation chains ----
        const SA_LDS char *kb = stage + (C::RPW * wave + n) * C::RS + 16 * g;
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ks += 2) {
            const bf16x8_t a0 = lds_read_b128(kb + 64 * ks);
            const bf16x8_t a1 = lds_read_b128(kb + 64 * (ks + 1));
            if (issue) {
                if constexpr (KV8)
                    copy8(t + 1, okm_nxt, rowv_nxt, (ks / 2) * (C::NCI8 + 1) / (C::KS / 2),
                          (ks / 2 + 1) * (C::NCI8 + 1) / (C::KS / 2));
                else
                    copy_rows(t + 1, okm_nxt, src_nxt, (ks / 2) * CPI, (ks / 2 + 1) * CPI);
            }
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[ks + 1], s1, 0, 0, 0);
        }
        // value i of lane (g, n): row RPW wave + 4 g + i, head n
        float sv[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sv[i] = (okm_cur >> (4 * g + i)) & 1 ? (s0[i] + s1[i]) * p.scale_log2 : -INFINITY;
            mx = fmaxf(mx, sv[i]);
        }
        mx = fmaxf(mx, shfl_xor_f32(mx, 16));
        mx = fmaxf(mx, shfl_xor_f32(mx, 32));
        if (g == 0) smax[wave][n] = mx;
        lds_barrier();
        const float ms = fmaxf(fmaxf(smax[0][n], smax[1][n]), fmaxf(smax[2][n], smax[3][n]));
        if (__ballot(ms > m_ref + kRescaleSlack)) {  // same decision in every wave
            const float m_new = fmaxf(m_ref, ms);
            if (__ballot(m_ref > -1e29f)) {
                const float alpha = exp2_fast(m_ref - m_new);
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) acc_o[dt] *= alpha;
                l_run *= alpha;
            }
            m_ref = m_new;
        }
        // weights -> bf16 -> P[head][k] in LDS.  Within each block of 8 rows the
        // contraction index k takes the even rows first, then the odd ones (k = 2 j
        // <-> row 2 j, k = 4 + j <-> row 2 j + 1), the order the V reads below use;
        // this lane's rows RPW wave + 4 g + i sit at k positions (i0, i2) and
        // (i1, i3) of its block half.
        {
            const uint32_t wa = pack_bf16x2(exp2_fast(sv[0] - m_ref), exp2_fast(sv[2] - m_ref));
            const uint32_t wb = pack_bf16x2(exp2_fast(sv[1] - m_ref), exp2_fast(sv[3] - m_ref));
            l_run += __uint_as_float(wa << 16) + __uint_as_float(wb << 16) + __uint_as_float(wa & 0xffff0000u) +
                     __uint_as_float(wb & 0xffff0000u);
            SA_LDS char *pw = (SA_LDS char *)pbuf + n * C::PRS + 2 * (C::RPW * wave + 8 * (g >> 1) + 2 * (g & 1));
            *reinterpret_cast<SA_LDS uint32_t *>(pw) = wa;
            *reinterpret_cast<SA_LDS uint32_t *>(pw + 8) = wb;
        }
        lds_barrier();

        // ---- O^T[this wave's d quarter][16 heads] += V^T P^T over the stage's rows ----
        // (transposing read: the 16 lanes of group g read rows 32 ks + 8 g + 2 (n / 4)
        // (+1 for the upper half of k), d 16 dt + 4 (n % 4) of the quarter; rows two
        // apart put the four 32-byte row pieces of one read on disjoint banks)
        const SA_LDS char *vb = stage + (8 * g + 2 * (n >> 2)) * C::RS + 2 * C::DQ * wave + 8 * (n & 3);
#pragma unroll
        for (int ks = 0; ks < C::ROWS / 32; ++ks) {
            if (32 * ks < hi - ebase) {  // k-steps past the list end hold only zero weights
                const bf16x8_t pb =
                    lds_read_b128((const SA_LDS char *)pbuf + n * C::PRS + 2 * (32 * ks + 8 * g));
                // all of the k-step's V reads go out ahead of its products
                i16x4_t lo4[C::DT], hi4[C::DT];
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    lo4[dt] = lds_read_tr16(vb + (32 * ks) * C::RS + 32 * dt);
                    hi4[dt] = lds_read_tr16(vb + (32 * ks + 1) * C::RS + 32 * dt);
                }
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    const bf16x8_t a = __builtin_bit_cast(
                        bf16x8_t, __builtin_shufflevector(lo4[dt], hi4[dt], 0, 1, 2, 3, 4, 5, 6, 7));
                    acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc_o[dt], 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 2 * C::DT + 1; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                for (int i = 0; i < C::DT; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        }
        okm_cur = okm_nxt;
    }

    // this wave's share of the sum: add the four lane groups, then the four waves
    l_run += shfl_xor_f32(l_run, 16);
    l_run += shfl_xor_f32(l_run, 32);
    if (g == 0) ssum[wave][n] = l_run;
    lds_barrier();
    const float l_tot = (ssum[0][n] + ssum[1][n]) + (ssum[2][n] + ssum[3][n]);

    if constexpr (KV8) {
        if (FUSED && hg == 0 && holds_new) {
            const int c = lane % (D / 8);
            const int64_t rrow = (int64_t)bi * p.rows + p.new_slot;
            *reinterpret_cast<u32x2_t *>(p.kv8c_ring + rrow * D + 8 * c) = new_codes;
            if ((c & 3) == 0) p.kv8s_ring[rrow * 16 + c / 4] = (uint8_t)new_sb;
            if (c == 0)
                for (int j = D / 32; j < 16; ++j) p.kv8s_ring[rrow * 16 + j] = 127;
        }
    } else if (FUSED && hg == 0 && has_new && wave == w_new && chunk_lane) {
        *reinterpret_cast<u32x4_t *>(p.kv_ring + ((int64_t)bi * p.rows + p.new_slot) * D + lane * 8) = new_row;
    }

    if (p.n_sp > 1) {
        if (head_ok) {
            const int64_t prow = ((int64_t)qi * p.n_sp + sp) * p.h + head;
            float *po = p.part_o + prow * D + C::DQ * wave + 4 * g;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) *reinterpret_cast<f32x4_t *>(po + 16 * dt) = acc_o[dt];
            if (wave == 0 && g == 0) {
                p.part_ml[prow * 2] = m_ref;
                p.part_ml[prow * 2 + 1] = l_tot;
            }
        }
        return;
    }
    const float Lt = l_tot + exp2_fast(sink_h * kLog2e - m_ref);
    const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;
    // lane (g, n) holds head n, d = quarter + 16 dt + 4 g + (0..3); the rows are
    // assembled in the head-row buffer (read into registers at the first stage)
    // so that every output store below writes a whole row
    SA_LDS char *orow = (SA_LDS char *)qbuf + n * C::RS + 2 * (C::DQ * wave + 4 * g);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
        const f32x4_t o = acc_o[dt] * inv;
        *reinterpret_cast<SA_LDS u32x2_t *>(orow + 32 * dt) = u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
    lds_barrier();
    // one head row per wave instruction: lane l stores 16-byte chunk l of the row
#pragma unroll
    for (int r = 0; r < C::HEADS / C::NW; ++r) {
        const int hr = wave + C::NW * r;
        const int hglob = (int)hg * C::HEADS + hr;
        if (hglob < p.h && chunk_lane) {
            u32x4_t v = *reinterpret_cast<const SA_LDS u32x4_t *>((const SA_LDS char *)qbuf + hr * C::RS + 16 * lane);
            if (rot) v = unrotate_chunk(v, 8 * lane, D, p.rope_dim, (const SA_LDS float *)rtab);
            store_16B_nt(p.out + ((int64_t)qi * p.h + hglob) * D + lane * 8, v);
        }
    }
}

// Combine of the split variant: thread per (query, head, 8 output values).
// M = max_s m_s;  L = sum_s l_s 2^(m_s - M) + 2^(sink log2 e - M);
// o = sum_s O_s 2^(m_s - M) / L; all-empty splits give 0.
template <int D>
__global__ void __launch_bounds__(256) sa_combine_kernel(const float *__restrict__ part_o,
                                                         const float *__restrict__ part_ml,
                                                         const float *__restrict__ sink,
                                                         uint16_t *__restrict__ out, int64_t nq,
                                                         int32_t h, int32_t n_sp, const float *__restrict__ rope,
                                                         int32_t rope_dim, int64_t rope_pos0, int32_t s_per_seq) {
    constexpr int CPR = D / 8;  // 8-value chunks per row
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nq * h * CPR) return;
    const int c = (int)(t % CPR);
    const int64_t qh = t / CPR;
    const int head = (int)(qh % h);
    const int64_t qi = qh / h;
    float M = -INFINITY;
    for (int s = 0; s < n_sp; ++s) M = fmaxf(M, part_ml[((qi * n_sp + s) * h + head) * 2]);
    float Lt = exp2_fast(sink[head] * kLog2e - M);
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n_sp; ++s) {
        const int64_t prow = (qi * n_sp + s) * h + head;
        const float w = exp2_fast(part_ml[prow * 2] - M);
        Lt += part_ml[prow * 2 + 1] * w;
        const f32x4_t a = *reinterpret_cast<const f32x4_t *>(part_o + prow * D + c * 8);
        const f32x4_t b = *reinterpret_cast<const f32x4_t *>(part_o + prow * D + c * 8 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[i] += a[i] * w;
            o[4 + i] += b[i] * w;
        }
    }
    const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;
    u32x4_t wv = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                  pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
    if (rope && c * 8 >= D - rope_dim) {  // the rounded output, un-rotated
        const float *cs = rope + (rope_pos0 + qi % s_per_seq) * rope_dim + (c * 8 - (D - rope_dim));
        const f32x4_t c0 = *reinterpret_cast<const f32x4_t *>(cs);
        const f32x4_t c1 = *reinterpret_cast<const f32x4_t *>(cs + 4);
        wv[0] = rope_pair(wv[0], c0[0], c0[1], true);
        wv[1] = rope_pair(wv[1], c0[2], c0[3], true);
        wv[2] = rope_pair(wv[2], c1[0], c1[1], true);
        wv[3] = rope_pair(wv[3], c1[2], c1[3], true);
    }
    *reinterpret_cast<u32x4_t *>(out + qh * D + c * 8) = wv;
}

// ------------------------------------------------------------------ dispatch --

struct Variant {
    int kernel;     // SA_KERNEL_WIDE, SA_KERNEL_DECODE or SA_KERNEL_PAIR
    int heads_wg;   // heads per workgroup
    int n_sp;       // index splits across workgroups
    int split_len;  // entries per split
};

int cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

void set_splits(Variant &v, int32_t topk, int n_sp) {
    n_sp = std::max(1, n_sp);
    int len = (std::max(topk, 1) + n_sp - 1) / n_sp;
    len = (len + 31) / 32 * 32;  // whole 32-row stages per split
    v.split_len = len;
    v.n_sp = std::max(1, (topk + len - 1) / len);
}

// Automatic choice from the problem shape and the CU count (thresholds from
// measurements on MI355X).  Short lists in decode-sized batches (fewer
// (query, 64-head group) pairs than two per CU) go to the decode kernel on
// 16-head groups; grids of at least four such pairs per CU to the pair kernel
// (two workgroups per CU overlap each other's prologue and epilogue); the rest
// to the wide kernel.  The index list is split across workgroups (f32 combine
// pass) only when the chosen kernel would leave CUs idle and the list is long
// enough to share.
constexpr int kDecodeMaxTopk = 512;
constexpr int kQueryRun = 128;            // consecutive queries per XCD run (prefill chunks)
constexpr int kQueryRunMinQueries = 4096; // chunk length from which queries go in runs (>= 4 runs per XCD)
constexpr int kPairMinPerCu = 4;
constexpr int kPairShortList = 512;   // pair kernel list chunk for lists up to this many entries
constexpr int kPairLongList = 2176;   // and for longer ones (a 128 + 2048-entry list in one pass)

Variant choose_variant(int64_t nq, int32_t h, int32_t topk, int cus) {
    Variant v{SA_KERNEL_WIDE, 64, 1, std::max(topk, 1)};
    const int64_t wide_wgs = nq * ((h + 63) / 64);
    if (wide_wgs < 2LL * cus && topk <= kDecodeMaxTopk) {
        v.kernel = SA_KERNEL_DECODE;
        v.heads_wg = 16;
    } else if (wide_wgs >= (int64_t)kPairMinPerCu * cus) {
        v.kernel = SA_KERNEL_PAIR;
    }
    const int64_t wgs = nq * ((h + v.heads_wg - 1) / v.heads_wg);
    const int min_len = v.kernel == SA_KERNEL_DECODE ? 128 : 256;
    if (wgs < cus && topk >= 2 * min_len) {
        const int64_t want = (cus + wgs - 1) / wgs;
        set_splits(v, topk, (int)std::min<int64_t>(want, topk / min_len));
    }
    return v;
}

size_t workspace_for(const Variant &v, int64_t nq, int32_t h, int32_t d) {
    if (v.n_sp <= 1) return 0;
    return (size_t)nq * v.n_sp * h * ((size_t)d + 2) * sizeof(float);
}

sa_status resolve_variant(int64_t nq, int32_t h, int32_t topk, int32_t kernel, int32_t splits, Variant *out) {
    Variant v = choose_variant(nq, h, topk, cu_count());
    if (kernel != 0 && kernel != SA_KERNEL_WIDE && kernel != SA_KERNEL_DECODE && kernel != SA_KERNEL_PAIR)
        return SA_ERR_UNSUPPORTED;
    if (splits < 0) return SA_ERR_UNSUPPORTED;
    if (kernel != 0 && kernel != v.kernel) {
        v.kernel = kernel;
        v.heads_wg = kernel == SA_KERNEL_DECODE ? 16 : 64;
        set_splits(v, topk, 1);
    }
    if (splits > 0) set_splits(v, topk, splits);
    *out = v;
    return SA_OK;
}

template <int D, bool FUSED>
hipError_t launch_wide(const AttnParams &p, hipStream_t stream) {
    if (p.n_sp > 1)
        hipLaunchKernelGGL((sa_attn_wide<D, FUSED, true>), dim3((unsigned)p.total_wg), dim3(WideCfg<D>::THREADS), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((sa_attn_wide<D, FUSED, false>), dim3((unsigned)p.total_wg), dim3(WideCfg<D>::THREADS), 0,
                           stream, p);
    return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_pair(const AttnParams &p0, hipStream_t stream) {
    AttnParams p = p0;
    const int cus = cu_count();
    p.stagger_cu = p.total_wg >= 2 * cus ? cus : 0;
    // list chunk capacity: the entries one workgroup handles, rounded up
    const int per_wg = std::min(p.topk, p.split_len);
    if (per_wg <= kPairShortList) {
        if (p.n_sp > 1)
            hipLaunchKernelGGL((sa_attn_pair<D, kPairShortList, MODE, true>), dim3((unsigned)p.total_wg), dim3(128),
                               0, stream, p);
        else
            hipLaunchKernelGGL((sa_attn_pair<D, kPairShortList, MODE, false>), dim3((unsigned)p.total_wg),
                               dim3(128), 0, stream, p);
    } else {
        if (p.n_sp > 1)
            hipLaunchKernelGGL((sa_attn_pair<D, kPairLongList, MODE, true>), dim3((unsigned)p.total_wg), dim3(128),
                               0, stream, p);
        else
            hipLaunchKernelGGL((sa_attn_pair<D, kPairLongList, MODE, false>), dim3((unsigned)p.total_wg),
                               dim3(128), 0, stream, p);
    }
    return hipGetLastError();
}

template <int D, bool FUSED, bool KV8>
hipError_t launch_decode(const AttnParams &p, hipStream_t stream) {
    hipLaunchKernelGGL((sa_attn_decode<D, FUSED, KV8>), dim3((unsigned)p.total_wg), dim3(DecodeCfg<D>::THREADS), 0,
                       stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_combine(const AttnParams &p, hipStream_t stream) {
    const int64_t n = (int64_t)p.nq * p.h * (D / 8);
    hipLaunchKernelGGL((sa_combine_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       p.part_o, p.part_ml, p.sink, p.out, (int64_t)p.nq, p.h, p.n_sp, p.rope, p.rope_dim,
                       p.rope_pos0, p.s);
    return hipGetLastError();
}

bool valid_d(int32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }

// MODE: 0 the index list from memory, 1 the decode step's list built in the
// kernel, 2 the prefill list built in the kernel (the pair kernel only).
template <int MODE, bool KV8>
hipError_t launch_attn(const AttnParams &p, const Variant &v, int32_t d, hipStream_t hs) {
    constexpr bool FUSED = MODE == 1;
    if constexpr (MODE == 2) {
        if (KV8 || v.kernel != SA_KERNEL_PAIR) return hipErrorNotSupported;  // (run_prefill_step asks for it)
        switch (d) {
            case 64: return launch_pair<64, 2>(p, hs);
            case 128: return launch_pair<128, 2>(p, hs);
            case 256: return launch_pair<256, 2>(p, hs);
            default: return launch_pair<512, 2>(p, hs);
        }
    }
    if (v.kernel == SA_KERNEL_DECODE) {
        switch (d) {
            case 64: return launch_decode<64, FUSED, KV8>(p, hs);
            case 128: return launch_decode<128, FUSED, KV8>(p, hs);
            case 256: return launch_decode<256, FUSED, KV8>(p, hs);
            default: return launch_decode<512, FUSED, KV8>(p, hs);
        }
    }
    if (KV8) return hipErrorNotSupported;  // (resolve_variant keeps kv8 on the decode kernel)
    if (v.kernel == SA_KERNEL_PAIR) {
        switch (d) {
            case 64: return launch_pair<64, MODE>(p, hs);
            case 128: return launch_pair<128, MODE>(p, hs);
            case 256: return launch_pair<256, MODE>(p, hs);
            default: return launch_pair<512, MODE>(p, hs);
        }
    }
    switch (d) {
        case 64: return launch_wide<64, FUSED>(p, hs);
        case 128: return launch_wide<128, FUSED>(p, hs);
        case 256: return launch_wide<256, FUSED>(p, hs);
        default: return launch_wide<512, FUSED>(p, hs);
    }
}

hipError_t launch_combine_d(const AttnParams &p, int32_t d, hipStream_t hs) {
    switch (d) {
        case 64: return launch_combine<64>(p, hs);
        case 128: return launch_combine<128>(p, hs);
        case 256: return launch_combine<256>(p, hs);
        default: return launch_combine<512>(p, hs);
    }
}

// Parameters shared by the plain call and the fused decode step; the workspace
// has been checked against the variant.
AttnParams base_params(const uint16_t *q, const uint16_t *kv, const float *sink, int64_t nq, int64_t s, int32_t h,
                       int32_t d, int64_t rows, int32_t topk, float scale, uint16_t *out, void *workspace,
                       const Variant &v) {
    AttnParams p = {};
    p.q = q;
    p.kv = kv;
    p.sink = sink;
    p.out = out;
    const bool ws = v.n_sp > 1;
    p.part_o = ws ? reinterpret_cast<float *>(workspace) : nullptr;
    p.part_ml = ws ? reinterpret_cast<float *>(workspace) + (size_t)nq * v.n_sp * h * d : nullptr;
    p.rows = rows;
    p.nq = (int32_t)nq;
    p.s = (int32_t)s;
    p.h = h;
    p.topk = topk;
    p.n_hg = (h + v.heads_wg - 1) / v.heads_wg;
    p.n_sp = v.n_sp;
    p.split_len = v.split_len;
    p.scale_log2 = scale * kLog2e;
    return p;
}

template <int MODE, bool KV8>
sa_status enqueue(AttnParams &p, const Variant &v, int32_t d, hipStream_t hs) {
    // decode kernel: one block per workgroup; wide and pair kernels: 8 * ceil(nq / 8) queries' worth
    // wide and pair kernels: queries dealt to the XCDs in runs (see wide_unit) --
    // runs of kQueryRun for a chunk of at least kQueryRunMinQueries queries of one
    // sequence (windows of neighbouring queries overlap), single queries otherwise
    p.qchunk = (v.kernel != SA_KERNEL_DECODE && p.s >= kQueryRunMinQueries) ? kQueryRun : 1;
    const int64_t run8 = 8 * (int64_t)p.qchunk;
    const int64_t units = v.kernel == SA_KERNEL_DECODE ? (int64_t)p.nq : run8 * (((int64_t)p.nq + run8 - 1) / run8);
    const int64_t total = units * p.n_hg * v.n_sp;
    if (total > 0x7fffffffLL) return SA_ERR_SHAPE;
    p.total_wg = (int32_t)total;
    if (launch_attn<MODE, KV8>(p, v, d, hs) != hipSuccess) return SA_ERR_HIP;
    if (v.n_sp > 1 && launch_combine_d(p, d, hs) != hipSuccess) return SA_ERR_HIP;
    return SA_OK;
}

sa_status check_workspace(const Variant &v, int64_t nq, int32_t h, int32_t d, void *workspace,
                          size_t workspace_bytes) {
    const size_t need = workspace_for(v, nq, h, d);
    if (need > 0 && (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 16))
        return SA_ERR_SHAPE;
    return SA_OK;
}

// Where the latent rows live: bf16 rows, or fp8-resident codes + scale records.
struct KvRows {
    const uint16_t *kv = nullptr;
    const uint8_t *kc = nullptr;
    const uint8_t *ks = nullptr;
    bool is8 = false;
    bool kv8() const { return is8; }
    bool present() const { return is8 ? (kc != nullptr && ks != nullptr) : kv != nullptr; }
    uintptr_t bits() const {
        return reinterpret_cast<uintptr_t>(kv) | reinterpret_cast<uintptr_t>(kc) | reinterpret_cast<uintptr_t>(ks);
    }
};

// The output's inverse rotation (none when table is null): query s of a
// sequence at position pos0 + s.
struct Rope {
    const float *table = nullptr;
    int64_t n_pos = 0;
    int32_t dim = 0;
    int64_t pos0 = 0;
};

sa_status check_rope(const Rope &r, int32_t d, int64_t s) {
    if (!r.table) return SA_OK;
    if (r.dim < 8 || r.dim % 8 != 0 || r.dim > d || r.n_pos < 0 || r.pos0 < 0) return SA_ERR_SHAPE;
    if (r.pos0 + s > r.n_pos) return SA_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(r.table) % 16) return SA_ERR_SHAPE;
    return SA_OK;
}

void set_rope(AttnParams &p, const Rope &r) {
    p.rope = r.table;
    p.rope_dim = r.table ? r.dim : 0;
    p.rope_pos0 = r.pos0;
}

// kv8 rows are read by the decode kernel only (it walks lists of any length)
sa_status resolve_variant_kv(int64_t nq, int32_t h, int32_t topk, int32_t kernel, int32_t splits, bool kv8,
                             Variant *out) {
    if (kv8 && (kernel == SA_KERNEL_WIDE || kernel == SA_KERNEL_PAIR)) return SA_ERR_UNSUPPORTED;
    return resolve_variant(nq, h, topk, kv8 ? SA_KERNEL_DECODE : kernel, splits, out);
}

sa_status run_sparse_attn(const uint16_t *q, const KvRows &kv, const float *sink, const int32_t *idx,
                          int64_t b, int64_t s, int32_t h, int32_t d, int64_t rows, int32_t topk,
                          float scale, uint16_t *out, void *workspace, size_t workspace_bytes,
                          void *stream, int32_t kernel, int32_t splits, const Rope &rope = Rope()) {
    if (b < 0 || s < 0 || h < 0 || d < 0 || rows < 0 || topk < 0) return SA_ERR_SHAPE;
    if (!valid_d(d)) return SA_ERR_UNSUPPORTED;
    if (!mul_le(b, s, 0x7fffffffLL)) return SA_ERR_SHAPE;
    const int64_t nq = b * s;
    if (check_rope(rope, d, s) != SA_OK) return SA_ERR_SHAPE;
    if (nq == 0 || h == 0) return SA_OK;
    if (!q || !sink || !out || (topk > 0 && !idx) || (rows > 0 && !kv.present())) return SA_ERR_NULL;
    if (rows > 0x7fffffffLL || nq > 0x7fffffffLL) return SA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(q) | kv.bits() | reinterpret_cast<uintptr_t>(out)) % 16) return SA_ERR_SHAPE;
    Variant v;
    sa_status st = resolve_variant_kv(nq, h, topk, kernel, splits, kv.kv8(), &v);
    if (st != SA_OK) return st;
    if ((st = check_workspace(v, nq, h, d, workspace, workspace_bytes)) != SA_OK) return st;
    AttnParams p = base_params(q, kv.kv, sink, nq, s, h, d, rows, topk, scale, out, workspace, v);
    p.kv8c = kv.kc;
    p.kv8s = kv.ks;
    p.idx = idx;
    set_rope(p, rope);
    return kv.kv8() ? enqueue<0, true>(p, v, d, (hipStream_t)stream)
                    : enqueue<0, false>(p, v, d, (hipStream_t)stream);
}

// Fused decode step: ring write of the new row (fp8 round trip), the window list,
// the compressed append and the attention in one launch (plus the combine of a
// split variant).
sa_status run_decode_step(const uint16_t *q, const KvRows &kv, const uint16_t *kv_new, const float *sink,
                          const int32_t *cidx, int32_t *idx_out, int64_t b, int32_t h, int32_t d, int64_t rows,
                          int32_t window, int32_t kc, int64_t start_pos, float scale, uint16_t *out,
                          void *workspace, size_t workspace_bytes, void *stream, int32_t kernel, int32_t splits,
                          Rope rope = Rope()) {
    if (b < 0 || h < 0 || d < 0 || rows < 0 || window <= 0 || kc < 0 || start_pos < 0) return SA_ERR_SHAPE;
    if (!valid_d(d)) return SA_ERR_UNSUPPORTED;
    if (start_pos == 0) return SA_ERR_UNSUPPORTED;  // position 0 is a prefill
    rope.pos0 = start_pos;
    if (check_rope(rope, d, 1) != SA_OK) return SA_ERR_SHAPE;
    if (rows < window || rows > 0x7fffffffLL || b > 0x7fffffffLL) return SA_ERR_SHAPE;
    if ((int64_t)window + kc > 0x7fffffffLL) return SA_ERR_SHAPE;
    if (b == 0 || h == 0) return SA_OK;
    if (!q || !kv.present() || !kv_new || !sink || !out || (kc > 0 && !cidx)) return SA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(q) | kv.bits() | reinterpret_cast<uintptr_t>(kv_new) |
         reinterpret_cast<uintptr_t>(out)) % 16)
        return SA_ERR_SHAPE;
    const int32_t topk = window + kc;
    Variant v;
    sa_status st = resolve_variant_kv(b, h, topk, kernel, splits, kv.kv8(), &v);
    if (st != SA_OK) return st;
    if ((st = check_workspace(v, b, h, d, workspace, workspace_bytes)) != SA_OK) return st;
    AttnParams p = base_params(q, kv.kv, sink, b, 1, h, d, rows, topk, scale, out, workspace, v);
    p.kv_new = kv_new;
    p.kv_ring = const_cast<uint16_t *>(kv.kv);
    p.kv8c = kv.kc;
    p.kv8s = kv.ks;
    p.kv8c_ring = const_cast<uint8_t *>(kv.kc);
    p.kv8s_ring = const_cast<uint8_t *>(kv.ks);
    p.cidx = cidx;
    p.idx_out = idx_out;
    p.pos = start_pos;
    p.window = window;
    p.kc = kc;
    p.wbase = (int32_t)((start_pos + 1) % window);
    p.new_slot = (int32_t)(start_pos % window);
    set_rope(p, rope);
    return kv.kv8() ? enqueue<1, true>(p, v, d, (hipStream_t)stream)
                    : enqueue<1, false>(p, v, d, (hipStream_t)stream);
}

// Prefill in one attention launch: the window list and the compressed append
// built inside the pair kernel (its own instance; the chunk's fp8 round trip,
// which every query's rows need first, is the caller's separate launch).
sa_status run_prefill_step(const uint16_t *q, const uint16_t *kv, const float *sink, const int32_t *cidx,
                           int32_t *idx_out, int64_t b, int64_t s, int32_t h, int32_t d, int64_t rows,
                           int32_t window, int32_t kc, float scale, uint16_t *out, void *workspace,
                           size_t workspace_bytes, void *stream, int32_t kernel, int32_t splits,
                           Rope rope = Rope()) {
    if (b < 0 || s < 0 || h < 0 || d < 0 || rows < 0 || window <= 0 || kc < 0) return SA_ERR_SHAPE;
    if (!valid_d(d)) return SA_ERR_UNSUPPORTED;
    rope.pos0 = 0;
    if (check_rope(rope, d, s) != SA_OK) return SA_ERR_SHAPE;
    if (!mul_le(b, s, 0x7fffffffLL)) return SA_ERR_SHAPE;
    const int64_t nq = b * s;
    if (rows < s || rows > 0x7fffffffLL || s > 0x7fffffffLL) return SA_ERR_SHAPE;
    const int32_t wcols = (int32_t)(s < window ? s : window);
    if ((int64_t)wcols + kc > 0x7fffffffLL) return SA_ERR_SHAPE;
    if (nq == 0 || h == 0) return SA_OK;
    if (!q || !kv || !sink || !out || (kc > 0 && !cidx)) return SA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv) | reinterpret_cast<uintptr_t>(out)) % 16)
        return SA_ERR_SHAPE;
    if (kernel != 0 && kernel != SA_KERNEL_PAIR) return SA_ERR_UNSUPPORTED;  // the pair kernel builds this list
    const int32_t topk = wcols + kc;
    Variant v;
    sa_status st = resolve_variant(nq, h, topk, SA_KERNEL_PAIR, splits, &v);
    if (st != SA_OK) return st;
    if ((st = check_workspace(v, nq, h, d, workspace, workspace_bytes)) != SA_OK) return st;
    AttnParams p = base_params(q, kv, sink, nq, s, h, d, rows, topk, scale, out, workspace, v);
    p.cidx = cidx;
    p.idx_out = idx_out;
    p.pos = -1;  // the prefill list
    p.window = wcols;
    p.kc = kc;
    set_rope(p, rope);
    return enqueue<2, false>(p, v, d, (hipStream_t)stream);
}

KvRows bf16_rows(const uint16_t *kv) {
    KvRows r;
    r.kv = kv;
    return r;
}

KvRows kv8_rows(const uint8_t *kc, const uint8_t *ks) {
    KvRows r;
    r.kc = kc;
    r.ks = ks;
    r.is8 = true;
    return r;
}

// ---------------------------------------------------- allocation-free entry --
//
// Scratch of sa_sparse_attn_noalloc: the split variants' f32 partials, in a
// device array of the library's own, so that the call allocates nothing.  Each
// device the library runs on holds its own copy from the code object's load
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address (one per device) comes from
// hipGetSymbolAddress, and only that address is ever handed to a kernel.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch's device address on the current device, looked up once per
// device (with that device current); null if the lookup fails.
void *scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t sa_sparse_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" sa_status sa_sparse_attn_noalloc(const uint16_t *q, const uint16_t *kv, const float *sink,
                                            const int32_t *idx, int64_t b, int64_t s, int32_t h, int32_t d,
                                            int64_t rows, int32_t topk, float scale, uint16_t *out, void *stream,
                                            int32_t kernel, int32_t splits) {
    // the variant and its partials' size exactly as sa_sparse_attn_ex takes them
    size_t need = 0;
    if (b >= 0 && s >= 0 && h > 0 && topk >= 0 && valid_d(d) && mul_le(b, s, 0x7fffffffLL) && b * s > 0) {
        Variant v;
        sa_status st = resolve_variant(b * s, h, topk, kernel, splits, &v);
        if (st != SA_OK) return st;
        need = workspace_for(v, b * s, h, d);
    }
    if (need > kScratchBytes) return SA_ERR_SHAPE;
    void *ws = nullptr;
    if (need > 0 && !(ws = scratch_address())) return SA_ERR_HIP;
    return run_sparse_attn(q, bf16_rows(kv), sink, idx, b, s, h, d, rows, topk, scale, out, ws,
                           need > 0 ? kScratchBytes : 0, stream, kernel, splits);
}

extern "C" size_t sa_sparse_attn_workspace_bytes(int64_t b, int64_t s, int32_t h, int32_t d, int32_t topk) {
    if (b < 0 || s < 0 || h <= 0 || topk < 0 || !valid_d(d) || !mul_le(b, s, 0x7fffffffLL)) return 0;
    Variant v;
    if (resolve_variant(b * s, h, topk, 0, 0, &v) != SA_OK) return 0;
    return workspace_for(v, b * s, h, d);
}

extern "C" size_t sa_sparse_attn_workspace_bytes_ex(int64_t b, int64_t s, int32_t h, int32_t d, int32_t topk,
                                                    int32_t kernel, int32_t splits) {
    if (b < 0 || s < 0 || h <= 0 || topk < 0 || !valid_d(d) || !mul_le(b, s, 0x7fffffffLL)) return 0;
    Variant v;
    if (resolve_variant(b * s, h, topk, kernel, splits, &v) != SA_OK) return 0;
    return workspace_for(v, b * s, h, d);
}

extern "C" sa_status sa_sparse_attn(const uint16_t *q, const uint16_t *kv, const float *sink,
                                    const int32_t *idx, int64_t b, int64_t s, int32_t h, int32_t d,
                                    int64_t rows, int32_t topk, float scale, uint16_t *out, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    return run_sparse_attn(q, bf16_rows(kv), sink, idx, b, s, h, d, rows, topk, scale, out, workspace,
                           workspace_bytes, stream, 0, 0);
}

extern "C" sa_status sa_sparse_attn_ex(const uint16_t *q, const uint16_t *kv, const float *sink,
                                       const int32_t *idx, int64_t b, int64_t s, int32_t h, int32_t d,
                                       int64_t rows, int32_t topk, float scale, uint16_t *out, void *workspace,
                                       size_t workspace_bytes, void *stream, int32_t kernel, int32_t splits) {
    return run_sparse_attn(q, bf16_rows(kv), sink, idx, b, s, h, d, rows, topk, scale, out, workspace,
                           workspace_bytes, stream, kernel, splits);
}

extern "C" size_t sa_sparse_attn_decode_step_workspace_bytes(int64_t b, int32_t h, int32_t d, int32_t window,
                                                             int32_t kc, int32_t kernel, int32_t splits) {
    if (b < 0 || h <= 0 || window <= 0 || kc < 0 || !valid_d(d) || (int64_t)window + kc > 0x7fffffffLL) return 0;
    Variant v;
    if (resolve_variant(b, h, window + kc, kernel, splits, &v) != SA_OK) return 0;
    return workspace_for(v, b, h, d);
}

extern "C" sa_status sa_sparse_attn_decode_step(const uint16_t *q, uint16_t *kv, const uint16_t *kv_new,
                                                const float *sink, const int32_t *cidx, int32_t *idx_out,
                                                int64_t b, int32_t h, int32_t d, int64_t rows, int32_t window,
                                                int32_t kc, int64_t start_pos, float scale, uint16_t *out,
                                                void *workspace, size_t workspace_bytes, void *stream,
                                                int32_t kernel, int32_t splits) {
    return run_decode_step(q, bf16_rows(kv), kv_new, sink, cidx, idx_out, b, h, d, rows, window, kc, start_pos,
                           scale, out, workspace, workspace_bytes, stream, kernel, splits);
}

extern "C" size_t sa_sparse_attn_prefill_step_workspace_bytes(int64_t b, int64_t s, int32_t h, int32_t d,
                                                              int32_t window, int32_t kc, int32_t kernel,
                                                              int32_t splits) {
    if (b < 0 || s < 0 || h <= 0 || window <= 0 || kc < 0 || !valid_d(d) || !mul_le(b, s, 0x7fffffffLL)) return 0;
    const int64_t wcols = s < window ? s : window;
    if (wcols + kc > 0x7fffffffLL) return 0;
    if (kernel != 0 && kernel != SA_KERNEL_PAIR) return 0;
    Variant v;
    if (resolve_variant(b * s, h, (int32_t)(wcols + kc), SA_KERNEL_PAIR, splits, &v) != SA_OK) return 0;
    return workspace_for(v, b * s, h, d);
}

extern "C" sa_status sa_sparse_attn_prefill_step(const uint16_t *q, const uint16_t *kv, const float *sink,
                                                 const int32_t *cidx, int32_t *idx_out, int64_t b, int64_t s,
                                                 int32_t h, int32_t d, int64_t rows, int32_t window, int32_t kc,
                                                 float scale, uint16_t *out, void *workspace,
                                                 size_t workspace_bytes, void *stream, int32_t kernel,
                                                 int32_t splits) {
    return run_prefill_step(q, kv, sink, cidx, idx_out, b, s, h, d, rows, window, kc, scale, out, workspace,
                            workspace_bytes, stream, kernel, splits);
}

extern "C" sa_status sa_sparse_attn_prefill_step_rope(const uint16_t *q, const uint16_t *kv, const float *sink,
                                                      const int32_t *cidx, int32_t *idx_out, int64_t b, int64_t s,
                                                      int32_t h, int32_t d, int64_t rows, int32_t window,
                                                      int32_t kc, float scale, uint16_t *out, void *workspace,
                                                      size_t workspace_bytes, void *stream, int32_t kernel,
                                                      int32_t splits, const float *rope_table, int64_t n_pos,
                                                      int32_t rope_dim) {
    if (!rope_table) return SA_ERR_NULL;
    Rope r;
    r.table = rope_table;
    r.n_pos = n_pos;
    r.dim = rope_dim;
    return run_prefill_step(q, kv, sink, cidx, idx_out, b, s, h, d, rows, window, kc, scale, out, workspace,
                            workspace_bytes, stream, kernel, splits, r);
}

extern "C" size_t sa_sparse_attn_kv8_workspace_bytes(int64_t b, int64_t s, int32_t h, int32_t d, int32_t topk,
                                                     int32_t splits) {
    if (b < 0 || s < 0 || h <= 0 || topk < 0 || !valid_d(d) || !mul_le(b, s, 0x7fffffffLL)) return 0;
    Variant v;
    if (resolve_variant_kv(b * s, h, topk, 0, splits, true, &v) != SA_OK) return 0;
    return workspace_for(v, b * s, h, d);
}

extern "C" sa_status sa_sparse_attn_kv8(const uint16_t *q, const uint8_t *kv_codes, const uint8_t *kv_scales,
                                        const float *sink, const int32_t *idx, int64_t b, int64_t s, int32_t h,
                                        int32_t d, int64_t rows, int32_t topk, float scale, uint16_t *out,
                                        void *workspace, size_t workspace_bytes, void *stream, int32_t splits) {
    return run_sparse_attn(q, kv8_rows(kv_codes, kv_scales), sink, idx, b, s, h, d, rows, topk, scale, out,
                           workspace, workspace_bytes, stream, 0, splits);
}

extern "C" sa_status sa_sparse_attn_decode_step_kv8(const uint16_t *q, uint8_t *kv_codes, uint8_t *kv_scales,
                                                    const uint16_t *kv_new, const float *sink, const int32_t *cidx,
                                                    int32_t *idx_out, int64_t b, int32_t h, int32_t d, int64_t rows,
                                                    int32_t window, int32_t kc, int64_t start_pos, float scale,
                                                    uint16_t *out, void *workspace, size_t workspace_bytes,
                                                    void *stream, int32_t splits) {
    return run_decode_step(q, kv8_rows(kv_codes, kv_scales), kv_new, sink, cidx, idx_out, b, h, d, rows, window,
                           kc, start_pos, scale, out, workspace, workspace_bytes, stream, 0, splits);
}

extern "C" sa_status sa_sparse_attn_rope(const uint16_t *q, const uint16_t *kv, const float *sink,
                                         const int32_t *idx, int64_t b, int64_t s, int32_t h, int32_t d,
                                         int64_t rows, int32_t topk, float scale, uint16_t *out, void *workspace,
                                         size_t workspace_bytes, void *stream, int32_t kernel, int32_t splits,
                                         const float *rope_table, int64_t n_pos, int32_t rope_dim,
                                         int64_t start_pos) {
    if (!rope_table) return SA_ERR_NULL;
    Rope r;
    r.table = rope_table;
    r.n_pos = n_pos;
    r.dim = rope_dim;
    r.pos0 = start_pos;
    return run_sparse_attn(q, bf16_rows(kv), sink, idx, b, s, h, d, rows, topk, scale, out, workspace,
                           workspace_bytes, stream, kernel, splits, r);
}

extern "C" sa_status sa_sparse_attn_decode_step_rope(const uint16_t *q, uint16_t *kv, const uint16_t *kv_new,
                                                     const float *sink, const int32_t *cidx, int32_t *idx_out,
                                                     int64_t b, int32_t h, int32_t d, int64_t rows, int32_t window,
                                                     int32_t kc, int64_t start_pos, float scale, uint16_t *out,
                                                     void *workspace, size_t workspace_bytes, void *stream,
                                                     int32_t kernel, int32_t splits, const float *rope_table,
                                                     int64_t n_pos, int32_t rope_dim) {
    if (!rope_table) return SA_ERR_NULL;
    Rope r;
    r.table = rope_table;
    r.n_pos = n_pos;
    r.dim = rope_dim;
    return run_decode_step(q, bf16_rows(kv), kv_new, sink, cidx, idx_out, b, h, d, rows, window, kc, start_pos,
                           scale, out, workspace, workspace_bytes, stream, kernel, splits, r);
}
