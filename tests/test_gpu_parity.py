"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Integer and fp8 work must match bit for bit; attention outputs must lie within
max(2 bf16 ulp, 1e-2) of the oracle's f32 value, element by element.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_latent_attention_02_amd as sa
from sparse_latent_attention_02_amd import workloads as wl
from helpers import act_quant_blocks, assert_parity, bits, from_bits, require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    sa.lib()
    oracle.lib()


def to_dev(t):
    return t.contiguous().to(DEV)


# ------------------------------------------------------------- index lists --

@pytest.mark.parametrize("W,bsz,seqlen,pos,extra", [
    (8, 1, 12, 0, 0), (8, 1, 1, 12, 0), (8, 1, 1, 13, 0), (8, 3, 1, 3, 0), (1, 2, 5, 0, 0),
    (128, 64, 1, 5000, 0), (128, 1, 4096, 0, 2048), (128, 2, 300, 0, 5), (128, 128, 1, 5000, 2048),
    (5, 2, 3, 0, 1), (128, 1, 1, 1, 0)])
def test_window_idx_bitexact(W, bsz, seqlen, pos, extra):
    rows, cols = oracle.window_topk_idxs_shape(W, seqlen, pos)
    assert sa.window_topk_idxs_shape(W, seqlen, pos) == (rows, cols)
    ref = np.full((bsz, rows, cols + extra), 77, dtype=np.int32)
    oracle.window_topk_idxs_into(ref, W, bsz, seqlen, pos)
    out = torch.full((bsz, rows, cols + extra), 77, dtype=torch.int32, device=DEV)
    sa.window_topk_idxs(W, bsz, seqlen, pos, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)


def test_append_compressed_bitexact():
    g = torch.Generator().manual_seed(3)
    cidx = torch.randint(-1, 500, (7, 3, 300), generator=g, dtype=torch.int32)
    ref = np.full((7, 3, 333), 5, dtype=np.int32)
    oracle.append_compressed_idxs(ref, 33, cidx.numpy(), 128)
    out = torch.full((7, 3, 333), 5, dtype=torch.int32, device=DEV)
    sa.append_compressed_idxs(out, 33, to_dev(cidx), 128)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)


# ------------------------------------------------------------ fp8 round trip --

def test_act_quant_exhaustive_bitexact():
    blocks = act_quant_blocks()
    ref = oracle.act_quant_fp8(blocks)
    x = to_dev(from_bits(blocks))
    sa.act_quant_fp8_(x)
    torch.cuda.synchronize()
    got = bits(x)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} mismatching values"


@pytest.mark.parametrize("rows,row_len", [(1, 32), (3, 64), (4096, 512), (17, 96)])
def test_act_quant_random_bitexact(rows, row_len):
    g = torch.Generator().manual_seed(rows)
    x = (torch.randn((rows, row_len), generator=g) * torch.exp(torch.randn((rows, 1), generator=g) * 3)).to(torch.bfloat16)
    ref = oracle.act_quant_fp8(bits(x))
    xd = to_dev(x)
    sa.act_quant_fp8_(xd)
    torch.cuda.synchronize()
    assert np.array_equal(bits(xd), ref)


# -------------------------------------------------------------- sparse_attn --

def run_both(case, variant=None, scale=None):
    q, kv, sink, idx = case["q"], case["kv"], case["sink"], case["idx"]
    d = q.shape[-1]
    scale = d ** -0.5 if scale is None else scale
    idx_o = idx.clone()
    idx_o[(idx_o < -1) | (idx_o >= kv.shape[1])] = -1  # the GPU treats out-of-range entries as -1
    _, ref32 = oracle.sparse_attn(bits(q), bits(kv), sink.numpy(), idx_o.numpy(), scale, want_f32=True)
    out = sa.sparse_attn(to_dev(q), to_dev(kv), to_dev(sink), to_dev(idx), scale, variant=variant)
    torch.cuda.synchronize()
    return bits(out), ref32


SMALL = [
    # seed, b, s, h, d, rows, topk, p_invalid
    (1, 1, 3, 4, 64, 12, 8, 0.0),
    (2, 2, 3, 1, 64, 50, 63, 0.2),
    (3, 2, 2, 16, 64, 100, 64, 0.0),
    (4, 1, 5, 20, 64, 90, 65, 0.3),
    (5, 2, 3, 64, 512, 300, 65, 0.1),
    (6, 1, 4, 128, 512, 200, 129, 0.05),
    (7, 3, 2, 64, 512, 500, 200, 0.5),
    (8, 1, 2, 16, 512, 40, 1, 0.0),
    (9, 2, 2, 48, 512, 70, 100, 0.0),
    (10, 1, 3, 4, 512, 33, 31, 0.0),
    (11, 2, 1, 64, 64, 6000, 5000, 0.1),   # longer than one compaction chunk
    (12, 1, 1, 16, 128, 80, 70, 0.1),
    (13, 1, 1, 16, 256, 80, 70, 0.1),
    (14, 1, 2, 64, 512, 1000, 512, 0.2),    # the pair kernel's short-list chunk, full
    (15, 2, 2, 64, 512, 1000, 513, 0.2),    # ... one entry past it: the long-list chunk
    (16, 1, 2, 64, 512, 3000, 2176, 0.1),   # a 128 + 2048-entry list in one chunk
    (17, 1, 2, 64, 512, 5000, 2177, 0.0),   # one entry past it: two chunks
]
VARIANTS = [None, (1, 1), (1, 2), (1, 3), (1, 7), (2, 1), (2, 2), (2, 5), (3, 1), (3, 2), (3, 5)]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"s{c[0]}_h{c[3]}_d{c[4]}_k{c[6]}")
@pytest.mark.parametrize("variant", VARIANTS, ids=lambda v: "auto" if v is None else "k%d_sp%d" % v)
def test_sparse_attn_small(case, variant):
    seed, b, s, h, d, rows, topk, p_inv = case
    c = wl.small_case(seed, b, s, h, d, rows, topk, p_inv)
    got, ref = run_both(c, variant)
    assert_parity(got, ref, f"case {case} variant {variant}")


@pytest.mark.parametrize("b,s", [(1, 4100), (2, 4099)], ids=["one_sequence", "two_sequences"])
@pytest.mark.parametrize("variant", [None, (1, 1), (3, 2)], ids=lambda v: "auto" if v is None else "k%d_sp%d" % v)
def test_sparse_attn_long_chunks_in_xcd_runs(b, s, variant):
    """Chunks of 4096 or more queries go to the XCDs in runs of consecutive queries
    (the grid padded to whole runs): a ragged query count, and runs that straddle
    two sequences, every query compared with the oracle, output pre-filled with NaN."""
    print(f"xcd runs b={b} s={s} variant {variant}", flush=True)
    c = wl.small_case(40 + b, b, s, 16, 64, 300, 48, p_invalid=0.1)
    q, kv, sink, idx = to_dev(c["q"]), to_dev(c["kv"]), to_dev(c["sink"]), to_dev(c["idx"])
    out = torch.full_like(q, float("nan"))
    sa.sparse_attn(q, kv, sink, idx, 0.125, out=out, variant=variant)
    torch.cuda.synchronize()
    _, ref32 = oracle.sparse_attn(bits(c["q"]), bits(c["kv"]), c["sink"].numpy(), c["idx"].numpy(), 0.125,
                                  want_f32=True)
    assert_parity(bits(out), ref32, f"xcd runs b={b} s={s} {variant}")


@pytest.mark.parametrize("d", [64, 256, 512])
@pytest.mark.parametrize("variant", [None, (1, 1), (1, 2), (2, 1), (3, 1), (3, 2)], ids=lambda v: "auto" if v is None else "k%d_sp%d" % v)
def test_sparse_attn_scores_outrunning_the_first_stage(d, variant):
    """The wide kernel takes the weights against the first max it sees and replays the
    list when a later stage outruns it by more than 2^32.  Rows built from one query's
    head row make that happen once (row 130, third 64-entry stage) and then again
    (row 250, fourth stage, about 2^60 above the first replay's reference); the
    result must still be the plain softmax."""
    g = torch.Generator().manual_seed(77)
    b, s, h, rows, topk = 2, 2, 64, 400, 320
    q = torch.randn((b, s, h, d), generator=g).to(torch.bfloat16)
    kv = (0.05 * torch.randn((b, rows, d), generator=g)).to(torch.bfloat16)
    c1 = 60.0 / (d ** 0.5 * 1.4426950408889634)   # log2-domain score about 60 above the rest
    for bi in range(b):
        kv[bi, 130] = (c1 * q[bi, 0, 5].float()).to(torch.bfloat16)
        kv[bi, 250] = (2.2 * c1 * q[bi, 0, 5].float()).to(torch.bfloat16)
    idx = torch.arange(topk, dtype=torch.int32).repeat(b, s, 1).contiguous()
    sink = torch.randn(h, generator=g)
    got, ref = run_both(dict(q=q, kv=kv, sink=sink, idx=idx), variant)
    assert_parity(got, ref, f"d {d} variant {variant}")
    # the head the rows were built from is dominated by the last one
    r = ref.reshape(b, s, h, d)[:, 0, 5]
    assert np.allclose(r, kv[:, 250].float().numpy(), rtol=2e-2, atol=2e-2)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("topk", [64, 130])
@pytest.mark.parametrize("variant", [None, (1, 1), (1, 2), (2, 1), (2, 2), (3, 1), (3, 2)],
                         ids=lambda v: "auto" if v is None else "k%d_sp%d" % v)
def test_sparse_attn_one_hot_rows_and_heads(d, topk, variant):
    """Row i of the cache is (1 + i // d) at dim i % d and 0 elsewhere; each (query,
    head) has one nonzero query value, at a dim of its own.  Every row then lands at a
    known dim of the output with a known weight, so a row or a head-row chunk copied to
    the wrong place, or read by the wrong wavefront, changes the output exactly where
    it shows.  Three launches in a row must agree bit for bit."""
    b, s, h = 1, 2, 32
    rows = max(topk, d)
    kv = torch.zeros((b, rows, d))
    for i in range(rows):
        kv[0, i, i % d] = 1.0 + i // d
    q = torch.zeros((b, s, h, d))
    for qi in range(s):
        for hh in range(h):
            q[0, qi, hh, (7 * hh + qi) % d] = 2.0
    kv, q = kv.to(torch.bfloat16), q.to(torch.bfloat16)
    sink = torch.full((h,), -30.0)
    idx = torch.arange(topk, dtype=torch.int32).view(1, 1, topk).repeat(b, s, 1).contiguous()
    got, ref = run_both(dict(q=q, kv=kv, sink=sink, idx=idx), variant, scale=1.0)
    # the closed form: softmax over the rows (the sink adds e^-30 to the denominator)
    ii = np.arange(topk)
    val = 1.0 + ii // d
    want = np.zeros((s, h, d))
    for qi in range(s):
        for hh in range(h):
            j = (7 * hh + qi) % d
            sc = np.where(ii % d == j, 2.0 * val, 0.0)
            w = np.exp(sc - sc.max())
            w /= w.sum() + np.exp(-30.0 - sc.max())
            np.add.at(want[qi, hh], ii % d, w * val)
    assert np.allclose(ref.reshape(s, h, d), want, rtol=1e-5, atol=1e-6)
    assert_parity(got, ref, f"one-hot d {d} topk {topk} variant {variant}")
    for _ in range(2):
        again = sa.sparse_attn(to_dev(q), to_dev(kv), to_dev(sink), to_dev(idx), 1.0, variant=variant)
        torch.cuda.synchronize()
        assert np.array_equal(bits(again), got)


def test_sparse_attn_edge_cases():
    # all -1, topk 0, sink -inf, invalid entries
    c = wl.small_case(21, 2, 3, 16, 512, 40, 40, 0.0)
    c["idx"][0] = -1
    c["idx"][1, 0, :7] = 40                 # past the end: treated as -1
    c["idx"][1, 1, 3] = -5                  # below -1: treated as -1
    got, ref = run_both(c)
    assert_parity(got, ref, "mixed invalid")
    assert not np.any(got[0])
    c["sink"][:] = -math.inf
    got, ref = run_both(c)
    assert_parity(got, ref, "sink -inf")
    assert not np.any(got[0])               # all -1 with no sink term: 0, not NaN
    c0 = dict(c, idx=torch.zeros((2, 3, 0), dtype=torch.int32))
    for v in (None, (1, 1), (1, 2), (2, 1), (2, 3)):
        got = bits(sa.sparse_attn(to_dev(c0["q"]), to_dev(c0["kv"]), to_dev(c0["sink"]), to_dev(c0["idx"]),
                                  0.1, variant=v))
        assert not np.any(got)


def test_sparse_attn_nan_in_unreferenced_rows_and_determinism():
    c = wl.small_case(22, 2, 4, 64, 512, 300, 150, 0.2)
    base = sa.sparse_attn(to_dev(c["q"]), to_dev(c["kv"]), to_dev(c["sink"]), to_dev(c["idx"]), 0.05)
    again = sa.sparse_attn(to_dev(c["q"]), to_dev(c["kv"]), to_dev(c["sink"]), to_dev(c["idx"]), 0.05)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), again.view(torch.int16))
    kv = c["kv"].clone()
    used = torch.zeros((2, 300), dtype=torch.bool)
    for bi in range(2):
        ii = c["idx"][bi].flatten()
        used[bi, ii[ii >= 0].long()] = True
    kv[~used] = float("nan")
    poisoned = sa.sparse_attn(to_dev(c["q"]), to_dev(kv), to_dev(c["sink"]), to_dev(c["idx"]), 0.05)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), poisoned.view(torch.int16))


def test_sparse_attn_argument_errors():
    L = sa.lib()
    ws = sa.workspace_bytes(1, 1, 16, 512, 8)
    assert ws == 0
    q = torch.zeros((1, 1, 16, 96), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((1, 4, 96), dtype=torch.bfloat16, device=DEV)
    sink = torch.zeros(16, device=DEV)
    idx = torch.zeros((1, 1, 4), dtype=torch.int32, device=DEV)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn(q, kv, sink, idx, 0.1)
    assert e.value.status == sa.SA_ERR_UNSUPPORTED
    assert L.sa_sparse_attn(None, None, None, None, 1, 1, 16, 512, 4, 4, 0.1, None, None, 0, None) == sa.SA_ERR_NULL
    assert L.sa_act_quant_fp8_inplace(None, 2, 48, None) == sa.SA_ERR_SHAPE
    x = torch.zeros((2, 64), dtype=torch.bfloat16, device=DEV)
    assert L.sa_act_quant_fp8_inplace(x.data_ptr(), 2, 48, None) == sa.SA_ERR_SHAPE
    assert L.sa_window_topk_idxs(8, 1, 4, 3, None, 8, None) == sa.SA_ERR_UNSUPPORTED
    out = torch.zeros((1, 12, 8), dtype=torch.int32, device=DEV)
    assert L.sa_window_topk_idxs(8, 1, 12, 0, out.data_ptr(), 7, None) == sa.SA_ERR_SHAPE
    # forced split (64 entries -> two 32-entry pieces) without workspace; unknown kernel
    q = torch.zeros((1, 1, 16, 512), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((1, 4, 512), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((1, 1, 64), dtype=torch.int32, device=DEV)
    assert sa.workspace_bytes(1, 1, 16, 512, 64, (1, 2)) > 0
    assert L.sa_sparse_attn_ex(q.data_ptr(), kv.data_ptr(), sink.data_ptr(), idx.data_ptr(), 1, 1, 16, 512, 4, 64,
                               0.1, q.data_ptr(), None, 0, None, 1, 2) == sa.SA_ERR_SHAPE
    assert L.sa_sparse_attn_ex(q.data_ptr(), kv.data_ptr(), sink.data_ptr(), idx.data_ptr(), 1, 1, 16, 512, 4, 64,
                               0.1, q.data_ptr(), None, 0, None, 9, 1) == sa.SA_ERR_UNSUPPORTED
