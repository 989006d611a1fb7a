// sa_select.hip -- the indexer's selection tail on the GPU.
//
// "DeepSeek V4.1 ... attention / query-latent", Indexer.forward after the
// scores: the causal compress_lens mask (prefill), the top-k positions by score,
// re-sorted into position order, shifted by the offset, -1 where unreachable.
// Equal scores: the lower position first (the pages leave the choice open).
//
// One workgroup per query row.  The k-th largest score is found by a radix
// select over order-preserving 32-bit keys (digits of 12, 10 and 10 bits, most
// significant first: a histogram of the keys that match the digits fixed so
// far, then the digit where the count from the top reaches the number still to
// take).  A last pass over the row in position order keeps the keys above that
// threshold and the first few equal to it, with a workgroup prefix sum giving
// each kept position its output column -- so the output comes out in position
// order with no sort.  Rows of up to kKeyCap positions keep their keys in
// registers; longer rows are read again, chunk by chunk, in each pass.
#include <type_traits>

#include "sa_device.h"
#include "../../include/sparse_attn.h"

namespace {

using namespace sa;

constexpr int kSelThreads = 1024;
constexpr int kKeyCap = 16384;  // positions per chunk: 16 keys per thread in registers
constexpr int kMaxBins = 4096;  // the widest digit: 12 bits

// f32 -> u32 with the same order (larger value, larger key); -inf is the
// smallest non-NaN key, and a masked position takes that key.  -0.0 and +0.0
// compare equal as scores, so -0.0 takes +0.0's key: equal scores then fall to
// the lower position, as for any other tie (a ReLU score times a negative
// weight gives -0.0).
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr uint32_t kKeyNegInf = 0x007fffffu;  // order_key(-inf)

// Inclusive prefix sum over a wavefront, in lane order: within each row of 16
// lanes, four steps over DPP row shifts by 1, 2, 4 and 8 (a lane shifted in from
// outside the row reads 0), then each row adds the totals of the rows before it
// (lanes 15, 31, 47).  VALU only: no LDS round trip.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Inclusive prefix sum over each row of 16 lanes (DPP row shifts by 1, 2, 4, 8).
__device__ __forceinline__ uint32_t row_inclusive_sum(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
    return x;
}

// The digit of the need-th largest key among those a histogram counted (BPT
// consecutive bins per thread, bins in thread order), the number of keys in
// the bins above that digit and the number in its own bin.  wsum[w] holds the count of wavefront w's bins.
// Every wavefront finds the digit by itself, with no barrier and no loop over
// the wavefronts: lane l < NW takes wavefront NW - 1 - l's total, so the lanes'
// prefix sum counts from the highest bins down and a ballot names the
// wavefront whose bins hold the digit; that wavefront's bins, read again from
// the histogram, name the lane and then the bin.
template <int NT, int BPT>
__device__ __forceinline__ void find_digit(const uint32_t *hist, const uint32_t *wsum, uint32_t need,
                                           uint32_t &digit, uint32_t &above, uint32_t &count) {
    constexpr int NW = NT / 64;
    static_assert(NW <= 16, "the wave totals are scanned within one row of 16 lanes");
    const int lane = threadIdx.x & 63;
    const uint32_t wt = lane < NW ? wsum[NW - 1 - lane] : 0u;
    const uint32_t top = row_inclusive_sum(wt);  // lanes < NW: keys in wavefronts NW - 1 - lane and above
    const uint64_t mw = __builtin_amdgcn_ballot_w64(lane < NW && top >= need);
    const int lw = mw ? __builtin_ctzll(mw) : NW - 1;
    const int ws = NW - 1 - lw;
    const uint32_t above_w = (uint32_t)__builtin_amdgcn_readlane((int)(top - wt), lw);
    const uint32_t tot_ws = (uint32_t)__builtin_amdgcn_readlane((int)wt, lw);
    const int th = 64 * ws + lane;
    uint32_t bins[BPT];
    if constexpr (BPT == 4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(hist + 4 * th);
        bins[0] = q.x, bins[1] = q.y, bins[2] = q.z, bins[3] = q.w;
    } else {
#pragma unroll
        for (int j = 0; j < BPT; ++j) bins[j] = hist[th * BPT + j];
    }
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) c += bins[j];
    const uint32_t incl = wave_inclusive_sum(c);
    uint32_t cum = above_w + (tot_ws - incl);  // keys in the bins above this lane's
    const bool hit = cum < need && cum + c >= need;
    uint32_t d = (uint32_t)(th * BPT), dc = 0;
    bool done = false;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
        const bool here = !done && cum + bins[j] >= need;
        d = here ? (uint32_t)(th * BPT + j) : d;
        dc = here ? bins[j] : dc;
        cum += (!done && !here) ? bins[j] : 0u;
        done = done || here;
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
    const int src = m ? __builtin_ctzll(m) : 0;
    digit = (uint32_t)__builtin_amdgcn_readlane((int)d, src);
    above = (uint32_t)__builtin_amdgcn_readlane((int)cum, src);
    count = (uint32_t)__builtin_amdgcn_readlane((int)dc, src);
}

// One row per workgroup of NT threads, taken in chunks of kKeyCap positions:
// thread tid holds the keys of positions 4 (tid + NT i) + j of a chunk, j < 4,
// i < TILES, so each load is a 16-byte piece per lane, consecutive across the
// lanes.  A row of up to kKeyCap positions (STREAM false) is loaded once and
// its keys stay in registers; a longer row (STREAM) is read again, chunk by
// chunk, in every pass, the next chunk's loads in flight while the current one
// is counted.  The three histograms are cleared once, up front, so a pass needs
// two barriers (after its atomics, after its wave totals); the first digit's
// atomics follow the loads tile by tile.  The ordered pass takes the same
// layout, tile by tile, with one barrier per chunk.
template <int NT, bool VEC, bool STREAM>
__global__ void __launch_bounds__(NT) indexer_topk_kernel(const float *__restrict__ scores, int64_t s,
                                                          int32_t T, int64_t start_pos, int32_t ratio,
                                                          int32_t topk, int32_t offset,
                                                          int32_t *__restrict__ out, int64_t row_stride,
                                                          int32_t col0) {
    constexpr int NW = NT / 64;
    constexpr int TILES = kKeyCap / (4 * NT);  // tiles of 4 NT positions, two to a count word
    constexpr int KPT = 4 * TILES;             // keys per thread and chunk
    constexpr int HW = kMaxBins + 2 * 1024;     // the three digits' histograms
    __shared__ __attribute__((aligned(16))) uint32_t hist[HW];
    __shared__ __attribute__((aligned(16))) uint32_t wsum[3][NW < 4 ? 4 : NW];
    __shared__ __attribute__((aligned(16))) uint32_t osum[STREAM ? 2 : 1][NW][TILES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t r = blockIdx.x;
    const int64_t si = r % s;
    const int64_t cl64 = start_pos == 0 ? (si + 1) / ratio : (start_pos + s) / ratio;  // compress_lens
    const int cl = (int)(cl64 < T ? cl64 : (int64_t)T);  // positions past the row are never read
    const float *sr = scores + r * T;
    int32_t *orow = out + r * row_stride + col0;

    if (topk >= T) {  // every position is taken
        for (int t = tid; t < T; t += NT) orow[t] = t < cl ? t + offset : -1;
        return;
    }
    const int nchunks = STREAM ? (T + kKeyCap - 1) / kKeyCap : 1;

    // The loads of chunk c: unconditional, from positions clamped into the row
    // (T > topk >= 1), since a branch around them would make the first use wait
    // for all of them (VEC: T a multiple of 4 and the scores 16-byte aligned, so
    // each piece is one load).
    float v[KPT];
    auto issue = [&](int c) {
        const int base = c * kKeyCap;
#pragma unroll
        for (int i = 0; i < TILES; ++i) {
            const int p = base + 4 * (tid + NT * i);
            if constexpr (VEC) {
                const float4 q = *reinterpret_cast<const float4 *>(sr + min(p, T - 4));
                v[4 * i] = q.x, v[4 * i + 1] = q.y, v[4 * i + 2] = q.z, v[4 * i + 3] = q.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[4 * i + j] = sr[min(p + j, T - 1)];
            }
        }
    };
    // Positions past the row end take key 0, below every score's key (-inf's is
    // the smallest): they land in the lowest bins, under the topk < T keys of
    // the row, so the threshold is a key of the row and they are never taken.
    uint32_t k[KPT];
    auto key = [&](int c, int i, int j) {
        const int p = c * kKeyCap + 4 * (tid + NT * i) + j;
        const uint32_t kv = order_key(v[4 * i + j]);
        k[4 * i + j] = p < T ? (p < cl ? kv : kKeyNegInf) : 0u;
    };
    // STREAM: the keys of chunk c, then the loads of the chunk after it (chunk 0
    // after the last: the next pass starts there)
    auto next_chunk = [&](int c) {
#pragma unroll
        for (int i = 0; i < TILES; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) key(c, i, j);
        issue(c + 1 < nchunks ? c + 1 : 0);
    };

    issue(0);
    // the histograms cleared while the loads are in flight
#pragma unroll
    for (int i = tid; i < HW / 4; i += NT) reinterpret_cast<uint4 *>(hist)[i] = uint4{0u, 0u, 0u, 0u};
    lds_barrier();

    // ---- radix select of the threshold key (the topk-th largest): digits of
    //      12, 10 and 10 bits, most significant first.  The wide first digit
    //      (sign, exponent, 3 mantissa bits) spreads scores that share a few
    //      binades over many bins, so the histogram atomics rarely collide; the
    //      later digits only count the few keys still matching. ----
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)topk;  // how many keys matching the prefix are still to take
    uint32_t n_eq = 0;               // keys in the last digit's bin: those equal to the threshold
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int width = pass == 0 ? 12 : 10;
        const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
        const int nb = 1 << width;
        constexpr int bpt0 = kMaxBins / NT, bpt1 = 1024 / NT;
        const int bpt = pass == 0 ? bpt0 : bpt1;
        const uint32_t dmask = (uint32_t)nb - 1u;
        uint32_t *h = hist + (pass == 0 ? 0 : kMaxBins + 1024 * (pass - 1));
        if constexpr (STREAM) {
            for (int c = 0; c < nchunks; ++c) {
                next_chunk(c);
#pragma unroll
                for (int q = 0; q < KPT; ++q)
                    if ((k[q] & pmask) == prefix) atomicAdd(&h[(k[q] >> shift) & dmask], 1u);
            }
        } else if (pass == 0) {
#pragma unroll
            for (int i = 0; i < TILES; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    key(0, i, j);
                    atomicAdd(&h[k[4 * i + j] >> 20], 1u);
                }
        } else {
#pragma unroll
            for (int q = 0; q < KPT; ++q)
                if ((k[q] & pmask) == prefix) atomicAdd(&h[(k[q] >> shift) & dmask], 1u);
        }
        lds_barrier();
        uint32_t c = 0;
        for (int j = 0; j < bpt; ++j) c += h[tid * bpt + j];
        const uint32_t x = wave_inclusive_sum(c);
        if (lane == 63) wsum[pass][wave] = x;
        lds_barrier();
        uint32_t digit, above;
        if (pass == 0)
            find_digit<NT, bpt0>(h, wsum[pass], need, digit, above, n_eq);
        else
            find_digit<NT, bpt1>(h, wsum[pass], need, digit, above, n_eq);
        prefix |= digit << shift;
        pmask |= dmask << shift;
        need -= above;
    }
    const uint32_t thr = prefix;  // keys above are all taken, `need` of those equal to it

    // ---- ordered pass, chunk by chunk: per tile, the keys taken counted two
    //      tiles to a word (16-bit fields: a tile holds 4 NT positions).  When
    //      every key equal to the threshold is taken (n_eq == need: the usual
    //      case, no tie at the cut) that is one count, of the keys at or above
    //      it; otherwise words [0, TILES / 2) count the keys above and the rest
    //      the equal ones, which are taken in position order while their rank
    //      among the equal keys is below need.  STREAM alternates two sets of
    //      wave totals, so a chunk's barrier also orders the reads of the totals
    //      two chunks back before their rewrite. ----
    // compress_lens again, opaque to the compiler: otherwise it keeps the 16 lane
    // masks of the key step alive across the passes for the test below
    int cl_out = cl;
    asm volatile("" : "+s"(cl_out));
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t gt_tiles = 0, eq_tiles = 0;  // keys of each kind in the tiles before
    auto ordered_chunk = [&](int c, auto all_tag) {
        constexpr bool ALL = decltype(all_tag)::value;
        constexpr int NC = ALL ? TILES / 2 : TILES;  // count words
        if constexpr (STREAM) next_chunk(c);
        uint32_t(*os)[TILES] = osum[STREAM ? (c & 1) : 0];
        uint32_t cnt[NC] = {};
#pragma unroll
        for (int i = 0; i < TILES; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q = 4 * i + j;
                const uint32_t f = 1u << (16 * (i & 1));
                if constexpr (ALL) {
                    cnt[i >> 1] += k[q] >= thr ? f : 0u;
                } else {
                    cnt[i >> 1] += k[q] > thr ? f : 0u;
                    cnt[TILES / 2 + (i >> 1)] += k[q] == thr ? f : 0u;
                }
            }
        uint32_t excl[NC];
#pragma unroll
        for (int w = 0; w < NC; ++w) {
            excl[w] = wave_inclusive_sum(cnt[w]) - cnt[w];
            if (lane == 63) os[wave][w] = excl[w] + cnt[w];
        }
        lds_barrier();
        // the wavefronts' totals: lane l < NW takes wavefront l's, a prefix sum
        // over the lanes gives the counts before this wavefront and the tiles'
        // totals
        uint32_t before[NC], total[NC];
#pragma unroll
        for (int f = 0; f < NC; ++f) {
            const uint32_t o = lane < NW ? os[lane][f] : 0u;
            const uint32_t incl = row_inclusive_sum(o);
            before[f] = (uint32_t)__builtin_amdgcn_readlane((int)(incl - o), wave_u);
            total[f] = (uint32_t)__builtin_amdgcn_readlane((int)incl, NW - 1);
        }
#pragma unroll
        for (int i = 0; i < TILES; ++i) {
            const int f = i >> 1, sh = 16 * (i & 1);
            const int t0 = c * kKeyCap + 4 * (tid + NT * i);
            const uint32_t gt_before = gt_tiles + (((before[f] + excl[f]) >> sh) & 0xffffu);
            if constexpr (ALL) {
                uint32_t pos = gt_before;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool take = k[4 * i + j] >= thr;
                    if (take && pos < (uint32_t)topk) orow[pos] = t0 + j < cl_out ? t0 + j + offset : -1;
                    pos += take ? 1u : 0u;
                }
            } else {
                const uint32_t eq_before =
                    eq_tiles + (((before[TILES / 2 + f] + excl[TILES / 2 + f]) >> sh) & 0xffffu);
                uint32_t pos = gt_before + min(eq_before, need);
                uint32_t eq_rank = eq_before;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int q = 4 * i + j;
                    bool take = k[q] > thr;
                    if (k[q] == thr) take = eq_rank++ < need;
                    if (take && pos < (uint32_t)topk) orow[pos] = t0 + j < cl_out ? t0 + j + offset : -1;
                    pos += take ? 1u : 0u;
                }
                eq_tiles += (total[TILES / 2 + f] >> sh) & 0xffffu;
            }
            gt_tiles += (total[f] >> sh) & 0xffffu;
        }
    };
    const bool all_eq = n_eq == need;
    for (int c = 0; c < nchunks; ++c) {
        if (all_eq)
            ordered_chunk(c, std::true_type{});
        else
            ordered_chunk(c, std::false_type{});
    }
}

template <bool VEC, bool STREAM>
void launch_topk(const float *scores, int64_t rows, int64_t s, int32_t n_cols, int64_t start_pos, int32_t ratio,
                 int32_t topk, int32_t offset, int32_t *idx, int64_t row_stride, int32_t col0, hipStream_t stream) {
    hipLaunchKernelGGL((indexer_topk_kernel<kSelThreads, VEC, STREAM>), dim3((unsigned)rows), dim3(kSelThreads), 0,
                       stream, scores, s, n_cols, start_pos, ratio, topk, offset, idx, row_stride, col0);
}

}  // namespace

extern "C" sa_status sa_indexer_topk(const float *scores, int64_t b, int64_t s, int32_t n_cols, int64_t start_pos,
                                     int32_t ratio, int32_t index_topk, int32_t offset, int32_t *idx,
                                     int64_t row_stride, int32_t col0, void *stream) {
    if (b < 0 || s < 0 || n_cols < 0 || start_pos < 0 || ratio <= 0 || index_topk < 0 || offset < 0 || col0 < 0)
        return SA_ERR_SHAPE;
    if ((int64_t)n_cols != (start_pos + s) / ratio) return SA_ERR_SHAPE;
    const int32_t topk = index_topk < n_cols ? index_topk : n_cols;
    if (row_stride < (int64_t)col0 + topk) return SA_ERR_SHAPE;
    const int64_t rows = b * s;
    if (rows == 0 || topk == 0) return SA_OK;
    if (!scores || !idx) return SA_ERR_NULL;
    if (rows > 0x7fffffffLL || n_cols > 0x7fff0000) return SA_ERR_SHAPE;  // chunk positions stay in int
    const bool vec = (n_cols & 3) == 0 && ((uintptr_t)scores & 15) == 0;
    const hipStream_t st = (hipStream_t)stream;
    if (n_cols <= kKeyCap) {
        if (vec) launch_topk<true, false>(scores, rows, s, n_cols, start_pos, ratio, topk, offset, idx, row_stride, col0, st);
        else launch_topk<false, false>(scores, rows, s, n_cols, start_pos, ratio, topk, offset, idx, row_stride, col0, st);
    } else {
        if (vec) launch_topk<true, true>(scores, rows, s, n_cols, start_pos, ratio, topk, offset, idx, row_stride, col0, st);
        else launch_topk<false, true>(scores, rows, s, n_cols, start_pos, ratio, topk, offset, idx, row_stride, col0, st);
    }
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}
