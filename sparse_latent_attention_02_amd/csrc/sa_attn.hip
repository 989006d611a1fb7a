// sa_attn.hip -- sparse latent attention for CDNA4 (gfx950).
//
// Operation ("DeepSeek V4.1 ... attention / attend": sparse_attn_kernel and its
// wrapper; "Module attn" rustdoc: sparse_attn): for every query and head, a
// softmax over the latent KV rows its index list selects (-1 skipped), the
// per-head sink adding to the denominator only, f32 arithmetic, bf16 result.
// One latent row is both key and value and is shared by every head, so a
// workgroup gathers each selected row into LDS once and all its heads use it.
//
// Kernel structure (one workgroup per (query, head group[, index split])):
//  1. compaction: the query's index entries are scanned and the valid ones
//     (0 <= idx < rows) packed into an LDS list, so -1 entries cost no MFMA work
//     and no traffic;
//  2. gather: stages of 32 rows per row-wavefront are copied HBM -> LDS with the
//     direct global->LDS path (16 B per lane, one 1 KiB row per wave instruction
//     at d = 512), double-buffered so the copy of stage t+1 overlaps the maths
//     of stage t; the 16-byte chunks of a row are XOR-swizzled by row so the
//     MFMA operand reads below hit distinct LDS banks;
//  3. scores: S^T[row][head] = K[row][:] . Q[head][:] on MFMA 16x16x32 bf16
//     (A = 16 gathered rows from LDS, B = 16 heads of Q held in registers for
//     the whole kernel), f32 accumulation;
//  4. online softmax in the base-2 domain (scale * log2 e folded once): the
//     accumulator layout puts one head per lane column, so the running max needs
//     only two cross-lane steps and the running sum none until the end; the
//     running max starts at the finite -1e30 of the pages' kernel, so a list
//     with no valid entry yields zeros rather than NaN;
//  5. O^T[d][head] += V^T[d][rows] . P^T[rows][head] on the same MFMA, with P
//     rounded to bf16 straight from the score registers (no shuffle) and V^T read
//     from LDS with the gfx950 transposing read ds_read_b64_tr_b16;
//  6. sink fold, normalisation, bf16 store -- or, for split variants, f32
//     partials (running max, sum, unnormalised O) combined by a second pass.
//
// Rows within a 16-row MFMA tile are visited in the order rho(m) (even rows,
// then odd) so that the transposing reads of one half-wave touch distinct
// banks under the swizzle; any row order is valid because each row's score and
// its value travel together.
#include "sa_device.h"
#include "../../include/sparse_attn.h"

#include <algorithm>

namespace {

using namespace sa;

constexpr int kBlk = 32;        // index entries per row-wavefront per stage (two MFMA tiles)
constexpr int kListCap = 2048;  // compacted entries held in LDS at once

struct AttnParams {
    const uint16_t *q;
    const uint16_t *kv;
    const float *sink;
    const int32_t *idx;
    uint16_t *out;
    float *part_o;   // [nq][n_sp][h][d] f32 (split variant only)
    float *part_ml;  // [nq][n_sp][h][2] f32: running max (log2 units), running sum
    int64_t nq;      // b * s
    int64_t s;       // queries per sequence
    int64_t rows;    // kv rows per sequence
    int64_t total_wg;
    int32_t h;
    int32_t topk;
    int32_t n_hg;       // head groups
    int32_t n_sp;       // index splits
    int32_t split_len;  // index entries per split
    float scale_log2;   // softmax scale * log2(e)
};

template <int D>
__device__ __forceinline__ int swz(int r) {
    // XOR applied to the 16-byte chunk index of a row held in LDS
    return D >= 128 ? (r & 15) : ((r >> 1) & 7);
}

__device__ __forceinline__ int rho(int m) { return m < 8 ? 2 * m : 2 * (m - 8) + 1; }

__device__ __forceinline__ bf16x8_t lds_read_b128(const SA_LDS char *p) {
    return *reinterpret_cast<const SA_LDS bf16x8_t *>(p);
}

__device__ __forceinline__ i16x4_t lds_read_tr16(const SA_LDS char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<SA_LDS i16x4_t *>(const_cast<SA_LDS char *>(p)));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int WH, int WR>
struct Cfg {
    static constexpr int NW = WH * WR;
    static constexpr int NT = 64 * NW;
    static constexpr int ROW_BYTES = 2 * D;
    static constexpr int CH = D / 8;   // 16-byte chunks per row
    static constexpr int KS = D / 32;  // k-steps of the score product
    static constexpr int DT = D / 16;  // 16-wide d tiles of the output
    static constexpr int ROWS_STAGE = kBlk * WR;
    static constexpr int STAGE_BYTES = ROWS_STAGE * ROW_BYTES;
    static constexpr int NBUF = WR <= 2 ? 2 : 1;
    static constexpr int RPI = 1024 / ROW_BYTES;            // rows per copy instruction
    static constexpr int INST_STAGE = STAGE_BYTES / 1024;   // copy instructions per stage
    static constexpr int IPW = INST_STAGE / NW;             // ... per wavefront
    static constexpr int KV_BYTES = NBUF * STAGE_BYTES;
    static constexpr int PART_BYTES = WR > 1 ? NW * D * 64 : 0;  // f32 partials of all waves
    static_assert(INST_STAGE % NW == 0 && IPW >= 1, "copy split");
    static_assert(PART_BYTES <= KV_BYTES, "partials reuse the KV buffers");
};

template <int D, int WH, int WR>
__global__ void __launch_bounds__(64 * WH * WR) sa_attn_kernel(const AttnParams p) {
    using C = Cfg<D, WH, WR>;
    __shared__ __attribute__((aligned(1024))) char smem[C::KV_BYTES];
    __shared__ int list[kListCap];
    __shared__ int wcnt[C::NW];
    __shared__ float mls[WR > 1 ? C::NW * 32 : 1];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int hw = wave % WH;  // head tile of this wavefront
    const int wr = wave / WH;  // row split of this wavefront
    const int g = lane >> 4;
    const int n = lane & 15;

    // Logical workgroup id: the dispatcher hands workgroups to the 8 XCDs round
    // robin; remap so each XCD runs a contiguous range of (query, head group,
    // split), keeping rows shared by neighbours in that XCD's L2.
    int64_t L;
    {
        const int64_t T = p.total_wg, per = T >> 3, rem = T & 7;
        const int64_t hwid = blockIdx.x, x = hwid & 7, k = hwid >> 3;
        L = x < rem ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
    }
    const int sp = (int)(L % p.n_sp);
    const int64_t t2 = L / p.n_sp;
    const int hg = (int)(t2 % p.n_hg);
    const int64_t qi = t2 / p.n_hg;
    const int64_t bi = qi / p.s;

    const int head = (hg * WH + hw) * 16 + n;
    const bool head_ok = head < p.h;

    // Q as the B operand: lane (g, n) holds q[head n][32 ks + 8 g .. +8] for every ks.
    bf16x8_t qreg[C::KS];
    {
        const uint16_t *qrow = p.q + (qi * p.h + (head_ok ? head : 0)) * (int64_t)D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            if (head_ok)
                qreg[ks] = *reinterpret_cast<const bf16x8_t *>(qrow + 32 * ks);
            else
                qreg[ks] = bf16x8_t{};
        }
    }

    float m_run = -1e30f;  // running max (log2 domain); finite start as in the pages' kernel
    float l_run = 0.0f;    // this lane's share of the running sum
    f32x4_t acc_o[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc_o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int lo = sp * p.split_len;
    const int hi = min(p.topk, lo + p.split_len);
    const int32_t *idxq = p.idx + qi * (int64_t)p.topk;
    const uint16_t *kvb = p.kv + bi * p.rows * (int64_t)D;
    const uint32_t smem_base = lds_addr((const SA_LDS void *)smem);

    for (int c0 = lo; c0 < hi; c0 += kListCap) {
        const int c1 = min(hi, c0 + kListCap);
        // ---- 1. compaction of idx[c0, c1) into list[0, nv) ----
        int nv = 0;
        for (int base = c0; base < c1; base += C::NT) {
            const int t = base + tid;
            const int v = t < c1 ? idxq[t] : -1;
            const bool ok = v >= 0 && (int64_t)v < p.rows;
            const uint64_t mask = __ballot(ok);
            const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
            if (lane == 0) wcnt[wave] = __popcll(mask);
            __syncthreads();
            int pre = 0, tot = 0;
#pragma unroll
            for (int w = 0; w < C::NW; ++w) {
                const int cw = wcnt[w];
                pre += w < wave ? cw : 0;
                tot += cw;
            }
            if (ok) list[nv + pre + pos] = v;
            nv += tot;
            __syncthreads();
        }
        if (nv == 0) continue;

        // ---- 2. gather pipeline ----
        const int nst = (nv + C::ROWS_STAGE - 1) / C::ROWS_STAGE;
        auto issue = [&](int st) {
            const uint32_t buf = smem_base + (uint32_t)((st % C::NBUF) * C::STAGE_BYTES);
#pragma unroll
            for (int u = 0; u < C::IPW; ++u) {
                const int inst = wave * C::IPW + u;
                const int r = inst * C::RPI + lane / C::CH;  // row within the stage
                const int e = min(st * C::ROWS_STAGE + r, nv - 1);  // past the end: repeat a valid row
                const int row = list[e];
                const int chunk = (lane % C::CH) ^ swz<D>(r);
                const uint16_t *src = kvb + (int64_t)row * D + chunk * 8;
                dma_16B(src, __builtin_amdgcn_readfirstlane(buf + inst * 1024));
            }
        };

        issue(0);
        for (int st = 0; st < nst; ++st) {
            if (C::NBUF == 2 && st + 1 < nst) {
                issue(st + 1);
                wait_vmcnt_barrier<C::IPW>();
            } else {
                wait_vmcnt_barrier<0>();
            }
            const SA_LDS char *buf = (const SA_LDS char *)smem +
                                     (st % C::NBUF) * C::STAGE_BYTES + wr * kBlk * C::ROW_BYTES;
            const int ebase = st * C::ROWS_STAGE + wr * kBlk;

            // ---- 3. scores S^T for this wave's 32 rows x 16 heads ----
            f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            {
                const int ra0 = rho(n), ra1 = 16 + rho(n);
                const SA_LDS char *p0 = buf + ra0 * C::ROW_BYTES;
                const SA_LDS char *p1 = buf + ra1 * C::ROW_BYTES;
                const int z0 = swz<D>(ra0), z1 = swz<D>(ra1);
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    const int c = 4 * ks + g;
                    const bf16x8_t a0 = lds_read_b128(p0 + ((c ^ z0) << 4));
                    const bf16x8_t a1 = lds_read_b128(p1 + ((c ^ z1) << 4));
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[ks], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[ks], s1, 0, 0, 0);
                }
            }

            // ---- 4. online softmax (lane column = head n; rows rho(4g+i)) ----
            float sc[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rho(4 * g + i);
                sc[i] = ebase + r < nv ? s0[i] * p.scale_log2 : -INFINITY;
                sc[4 + i] = ebase + 16 + r < nv ? s1[i] * p.scale_log2 : -INFINITY;
            }
            float mx = sc[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
            mx = fmaxf(mx, shfl_xor_f32(mx, 16));
            mx = fmaxf(mx, shfl_xor_f32(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2_fast(m_run - m_new);
            uint32_t pk[4];
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t bits = pack_bf16x2(exp2_fast(sc[2 * i] - m_new),
                                                  exp2_fast(sc[2 * i + 1] - m_new));
                pk[i] = bits;
                psum += __uint_as_float(bits << 16) + __uint_as_float(bits & 0xffff0000u);
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            if (__ballot(alpha != 1.0f)) {
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) acc_o[dt] *= alpha;
            }
            bf16x8_t pb;
            {
                u32x4_t pw = {pk[0], pk[1], pk[2], pk[3]};
                pb = __builtin_bit_cast(bf16x8_t, pw);
            }

            // ---- 5. O^T += V^T P^T ----
            {
                const int rr0 = rho(4 * g + (n >> 2)), rr1 = 16 + rr0;
                const SA_LDS char *p0 = buf + rr0 * C::ROW_BYTES + ((n & 1) << 3);
                const SA_LDS char *p1 = buf + rr1 * C::ROW_BYTES + ((n & 1) << 3);
                const int z0 = swz<D>(rr0), z1 = swz<D>(rr1);
                const int csub = (n & 3) >> 1;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    const int c = 2 * dt + csub;
                    const i16x4_t lo4 = lds_read_tr16(p0 + ((c ^ z0) << 4));
                    const i16x4_t hi4 = lds_read_tr16(p1 + ((c ^ z1) << 4));
                    const bf16x8_t a = __builtin_bit_cast(
                        bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
                    acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc_o[dt], 0, 0, 0);
                }
            }
            lds_barrier();  // every wave is done with this buffer
            if (C::NBUF == 1 && st + 1 < nst) issue(st + 1);
        }
    }

    // full running sum of the head: add the shares of the four lane groups
    l_run += shfl_xor_f32(l_run, 16);
    l_run += shfl_xor_f32(l_run, 32);

    if (p.n_sp > 1) {
        // ---- 6b. split partials: unnormalised O, running max and sum, no sink ----
        if (head_ok) {
            const int64_t prow = (qi * p.n_sp + sp) * p.h + head;
            float *po = p.part_o + prow * D + 4 * g;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) *reinterpret_cast<f32x4_t *>(po + 16 * dt) = acc_o[dt];
            if (g == 0) {
                p.part_ml[prow * 2] = m_run;
                p.part_ml[prow * 2 + 1] = l_run;
            }
        }
        return;
    }

    const float sink_l2 = head_ok ? p.sink[head] * kLog2e : 0.f;
    uint16_t *orow = p.out + (qi * p.h + (head_ok ? head : 0)) * (int64_t)D + 4 * g;

    if (WR == 1) {
        // ---- 6. sink fold + normalise + store ----
        if (!head_ok) return;
        const float Lt = l_run + exp2_fast(sink_l2 - m_run);
        const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;  // empty list: 0 / inf or guarded 0 / 0
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            const f32x4_t o = acc_o[dt] * inv;
            u32x2_t w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            *reinterpret_cast<u32x2_t *>(orow + 16 * dt) = w;
        }
        return;
    }

    // ---- 6c. in-workgroup combine of the WR row-split waves of each head tile ----
    {
        float *part = reinterpret_cast<float *>(smem);
        const int slot = hw * WR + wr;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
            *reinterpret_cast<f32x4_t *>(part + ((slot * C::DT + dt) * 64 + lane) * 4) = acc_o[dt];
        if (g == 0) {
            mls[(slot * 16 + n) * 2] = m_run;
            mls[(slot * 16 + n) * 2 + 1] = l_run;
        }
        lds_barrier();
        float mr[WR], wgt[WR];
        float M = -INFINITY;
#pragma unroll
        for (int r = 0; r < WR; ++r) {
            mr[r] = mls[((hw * WR + r) * 16 + n) * 2];
            M = fmaxf(M, mr[r]);
        }
        float Lt = 0.f;
#pragma unroll
        for (int r = 0; r < WR; ++r) {
            wgt[r] = exp2_fast(mr[r] - M);
            Lt += mls[((hw * WR + r) * 16 + n) * 2 + 1] * wgt[r];
        }
        Lt += exp2_fast(sink_l2 - M);
        const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;
        if (!head_ok) return;
        constexpr int DPW = C::DT / WR;  // d tiles finalised by each row-split wave
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
            const int dt = wr * DPW + j;
            f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < WR; ++r)
                o += *reinterpret_cast<const f32x4_t *>(part + (((hw * WR + r) * C::DT + dt) * 64 + lane) * 4) *
                     wgt[r];
            o *= inv;
            u32x2_t w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            *reinterpret_cast<u32x2_t *>(orow + 16 * dt) = w;
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
                                                         int32_t h, int32_t n_sp) {
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
    *reinterpret_cast<u32x4_t *>(out + qh * D + c * 8) = wv;
}

// ------------------------------------------------------------------ dispatch --

struct Variant {
    int wh, wr, n_sp, split_len;
};

int cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

// Chooses the variant from the problem shape and the CU count.
//  - heads are tiled 16 per wavefront; a workgroup takes up to 4 head tiles;
//  - with too few (query, head group) workgroups to fill the chip, heads are
//    split into single-tile groups whose four wavefronts split the index list
//    and combine in LDS (rows are shared through L2 between the groups of one
//    query), and only then is the list split across workgroups with an f32
//    combine pass.
Variant choose_variant(int64_t nq, int32_t h, int32_t topk, int cus) {
    const int n_ht = (h + 15) / 16;
    Variant v{std::min(4, n_ht), 1, 1, std::max(topk, 1)};
    const int64_t target = 2LL * cus;
    int64_t wgs = nq * ((n_ht + v.wh - 1) / v.wh);
    if (wgs >= target) return v;
    if (topk > 2 * kBlk) {
        // spread heads over more workgroups, filling each with row-split waves
        v.wh = 1;
        v.wr = 4;
        wgs = nq * n_ht;
        if (wgs >= cus) return v;
        // still too few: split the list across workgroups as well
        v.wr = 1;
        v.wh = std::min(4, n_ht);
        wgs = nq * ((n_ht + v.wh - 1) / v.wh);
        int n_sp = (int)std::min<int64_t>((target + wgs - 1) / wgs, (topk + 127) / 128);
        n_sp = std::max(1, std::min(n_sp, 64));
        v.n_sp = n_sp;
        v.split_len = (topk + n_sp - 1) / n_sp;
        v.split_len = (v.split_len + kBlk - 1) / kBlk * kBlk;
        v.n_sp = (topk + v.split_len - 1) / v.split_len;
    }
    return v;
}

size_t workspace_for(const Variant &v, int64_t nq, int32_t h, int32_t d) {
    if (v.n_sp <= 1) return 0;
    return (size_t)nq * v.n_sp * h * ((size_t)d + 2) * sizeof(float);
}

template <int D, int WH, int WR>
hipError_t launch_attn(const AttnParams &p, hipStream_t stream) {
    hipLaunchKernelGGL((sa_attn_kernel<D, WH, WR>), dim3((unsigned)p.total_wg), dim3(64 * WH * WR), 0,
                       stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams &p, int wh, int wr, hipStream_t stream) {
    if (wr == 1) {
        if (wh == 1) return launch_attn<D, 1, 1>(p, stream);
        if (wh == 2) return launch_attn<D, 2, 1>(p, stream);
        return launch_attn<D, 4, 1>(p, stream);
    }
    if (wr == 2) {
        if (wh == 1) return launch_attn<D, 1, 2>(p, stream);
        return launch_attn<D, 2, 2>(p, stream);
    }
    return launch_attn<D, 1, 4>(p, stream);
}

template <int D>
hipError_t launch_combine(const AttnParams &p, hipStream_t stream) {
    const int64_t n = p.nq * p.h * (D / 8);
    hipLaunchKernelGGL((sa_combine_kernel<D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       p.part_o, p.part_ml, p.sink, p.out, p.nq, p.h, p.n_sp);
    return hipGetLastError();
}

bool valid_d(int32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }

sa_status resolve_variant(int64_t nq, int32_t h, int32_t topk, int32_t heads_per_wg, int32_t row_waves,
                          int32_t splits, Variant *out) {
    Variant v = choose_variant(nq, h, topk, cu_count());
    if (heads_per_wg || row_waves || splits) {
        const int wh = heads_per_wg ? heads_per_wg / 16 : v.wh;
        const int wr = row_waves ? row_waves : (heads_per_wg ? 1 : v.wr);
        const int sp = splits ? splits : 1;
        if (heads_per_wg && heads_per_wg != 16 && heads_per_wg != 32 && heads_per_wg != 64)
            return SA_ERR_UNSUPPORTED;
        if (wr != 1 && wr != 2 && wr != 4) return SA_ERR_UNSUPPORTED;
        if (wh * wr > 4 || (wr == 2 && wh > 2) || (wr == 4 && wh > 1)) return SA_ERR_UNSUPPORTED;
        if (sp < 1 || (sp > 1 && wr != 1)) return SA_ERR_UNSUPPORTED;
        v.wh = wh;
        v.wr = wr;
        v.n_sp = sp;
        v.split_len = std::max(1, (topk + sp - 1) / sp);
        if (sp > 1) v.n_sp = std::max(1, (topk + v.split_len - 1) / v.split_len);
    }
    *out = v;
    return SA_OK;
}

sa_status run_sparse_attn(const uint16_t *q, const uint16_t *kv, const float *sink, const int32_t *idx,
                          int64_t b, int64_t s, int32_t h, int32_t d, int64_t rows, int32_t topk,
                          float scale, uint16_t *out, void *workspace, size_t workspace_bytes,
                          void *stream, int32_t heads_per_wg, int32_t row_waves, int32_t splits) {
    if (b < 0 || s < 0 || h < 0 || d < 0 || rows < 0 || topk < 0) return SA_ERR_SHAPE;
    if (!valid_d(d)) return SA_ERR_UNSUPPORTED;
    const int64_t nq = b * s;
    if (nq == 0 || h == 0) return SA_OK;
    if (!q || !sink || !out || (topk > 0 && !idx) || (rows > 0 && !kv)) return SA_ERR_NULL;
    if (rows > 0x7fffffffLL) return SA_ERR_SHAPE;  // int32 indices
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv) | reinterpret_cast<uintptr_t>(out)) % 16)
        return SA_ERR_SHAPE;
    Variant v;
    sa_status st = resolve_variant(nq, h, topk, heads_per_wg, row_waves, splits, &v);
    if (st != SA_OK) return st;
    const size_t need = workspace_for(v, nq, h, d);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SA_ERR_SHAPE;
    const int n_ht = (h + 15) / 16;
    AttnParams p;
    p.q = q;
    p.kv = kv;
    p.sink = sink;
    p.idx = idx;
    p.out = out;
    p.part_o = need ? reinterpret_cast<float *>(workspace) : nullptr;
    p.part_ml = need ? reinterpret_cast<float *>(workspace) + (size_t)nq * v.n_sp * h * d : nullptr;
    p.nq = nq;
    p.s = s;
    p.rows = rows;
    p.h = h;
    p.topk = topk;
    p.n_hg = (n_ht + v.wh - 1) / v.wh;
    p.n_sp = v.n_sp;
    p.split_len = v.split_len;
    p.scale_log2 = scale * kLog2e;
    p.total_wg = nq * p.n_hg * v.n_sp;
    if (p.total_wg > 0x7fffffffLL) return SA_ERR_SHAPE;
    hipStream_t hs = (hipStream_t)stream;
    hipError_t e;
    switch (d) {
        case 64: e = launch_d<64>(p, v.wh, v.wr, hs); break;
        case 128: e = launch_d<128>(p, v.wh, v.wr, hs); break;
        case 256: e = launch_d<256>(p, v.wh, v.wr, hs); break;
        default: e = launch_d<512>(p, v.wh, v.wr, hs); break;
    }
    if (e != hipSuccess) return SA_ERR_HIP;
    if (v.n_sp > 1) {
        switch (d) {
            case 64: e = launch_combine<64>(p, hs); break;
            case 128: e = launch_combine<128>(p, hs); break;
            case 256: e = launch_combine<256>(p, hs); break;
            default: e = launch_combine<512>(p, hs); break;
        }
        if (e != hipSuccess) return SA_ERR_HIP;
    }
    return SA_OK;
}

}  // namespace

extern "C" size_t sa_sparse_attn_workspace_bytes(int64_t b, int64_t s, int32_t h, int32_t d, int32_t topk) {
    if (b < 0 || s < 0 || h <= 0 || topk < 0 || !valid_d(d)) return 0;
    Variant v;
    if (resolve_variant(b * s, h, topk, 0, 0, 0, &v) != SA_OK) return 0;
    return workspace_for(v, b * s, h, d);
}

extern "C" size_t sa_sparse_attn_workspace_bytes_ex(int64_t b, int64_t s, int32_t h, int32_t d, int32_t topk,
                                                    int32_t heads_per_wg, int32_t row_waves, int32_t splits) {
    if (b < 0 || s < 0 || h <= 0 || topk < 0 || !valid_d(d)) return 0;
    Variant v;
    if (resolve_variant(b * s, h, topk, heads_per_wg, row_waves, splits, &v) != SA_OK) return 0;
    return workspace_for(v, b * s, h, d);
}

extern "C" sa_status sa_sparse_attn(const uint16_t *q, const uint16_t *kv, const float *sink,
                                    const int32_t *idx, int64_t b, int64_t s, int32_t h, int32_t d,
                                    int64_t rows, int32_t topk, float scale, uint16_t *out, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    return run_sparse_attn(q, kv, sink, idx, b, s, h, d, rows, topk, scale, out, workspace, workspace_bytes,
                           stream, 0, 0, 0);
}

extern "C" sa_status sa_sparse_attn_ex(const uint16_t *q, const uint16_t *kv, const float *sink,
                                       const int32_t *idx, int64_t b, int64_t s, int32_t h, int32_t d,
                                       int64_t rows, int32_t topk, float scale, uint16_t *out, void *workspace,
                                       size_t workspace_bytes, void *stream, int32_t heads_per_wg,
                                       int32_t row_waves, int32_t splits) {
    return run_sparse_attn(q, kv, sink, idx, b, s, h, d, rows, topk, scale, out, workspace, workspace_bytes,
                           stream, heads_per_wg, row_waves, splits);
}
