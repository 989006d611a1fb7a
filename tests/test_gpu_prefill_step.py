"""GPU parity of the prefill with its lists built in the attention kernel
(sa_sparse_attn_prefill_step): the window list of the chunk and the compressed
indices appended after it are formed in LDS by the kernel.

Against the oracle's own list functions and attention on the same inputs: the
written list bit for bit, the output within max(2 bf16 ulp, 1e-2) of the
oracle's f32 value.  Against the separate GPU calls (sa_window_topk_idxs,
sa_append_compressed_idxs, sa_sparse_attn_ex with the same variant): the output
bit for bit, since both run the same arithmetic on the same list.  Cases cover
chunks shorter and longer than the window (several stages and a ragged tail),
no compressed columns, every head dim and the index splits (the pair kernel
builds this list; other kernels are refused).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_latent_attention_02_amd as sa
from helpers import assert_parity, bits, require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    sa.lib()
    oracle.lib()


def make_case(seed, b, s, h, d, W, n_comp_rows, kc, p_hole=0.1):
    g = torch.Generator().manual_seed(seed)
    rows = s + n_comp_rows
    q = torch.randn((b, s, h, d), generator=g).to(torch.bfloat16)
    kv = torch.randn((b, rows, d), generator=g).to(torch.bfloat16)
    sink = torch.randn((h,), generator=g)
    cidx = None
    if kc:
        cidx = torch.randint(0, max(n_comp_rows, 1), (b, s, kc), generator=g, dtype=torch.int32)
        cidx[torch.rand((b, s, kc), generator=g) < p_hole] = -1
    return dict(q=q, kv=kv, sink=sink, cidx=cidx, W=W, s=s, h=h, d=d, kc=kc)


def oracle_case(c):
    b, s, W, kc = c["q"].shape[0], c["s"], c["W"], c["kc"]
    wcols = min(s, W)
    idx = np.full((b, s, wcols + kc), -9, dtype=np.int32)
    oracle.window_topk_idxs_into(idx, W, b, s, 0)
    if kc:
        oracle.append_compressed_idxs(idx, wcols, np.ascontiguousarray(c["cidx"].numpy()), s)
    _, ref = oracle.sparse_attn(bits(c["q"]), bits(c["kv"]), c["sink"].numpy(), idx, c["d"] ** -0.5,
                                want_f32=True)
    return idx, ref


def gpu_fused(c, variant=None):
    b, s, W, kc = c["q"].shape[0], c["s"], c["W"], c["kc"]
    idx_out = torch.full((b, s, min(s, W) + kc), -7, dtype=torch.int32, device=DEV)
    out = torch.empty_like(c["q"], device=DEV)
    out.view(torch.int16).fill_(-1)                  # NaN: an element never written shows
    sa.sparse_attn_prefill_step(c["q"].to(DEV), c["kv"].to(DEV), c["sink"].to(DEV), W, c["d"] ** -0.5,
                                cidx=c["cidx"].to(DEV) if kc else None, out=out, idx_out=idx_out, variant=variant)
    torch.cuda.synchronize()
    return idx_out.cpu().numpy(), bits(out)


def gpu_separate(c, variant):
    b, s, W, kc, h, d = c["q"].shape[0], c["s"], c["W"], c["kc"], c["h"], c["d"]
    wcols = min(s, W)
    idx = torch.full((b, s, wcols + kc), -7, dtype=torch.int32, device=DEV)
    sa.window_topk_idxs(W, b, s, 0, out=idx)
    if kc:
        sa.append_compressed_idxs(idx, wcols, c["cidx"].to(DEV), s)
    out = sa.sparse_attn(c["q"].to(DEV), c["kv"].to(DEV), c["sink"].to(DEV), idx, d ** -0.5, variant=variant)
    torch.cuda.synchronize()
    return bits(out)


CASES = [
    # (seed, b, s, h, d, W, compressed rows, kc)
    (1, 1, 300, 64, 512, 64, 200, 96),     # chunk longer than the window, several stages, ragged tail
    (2, 2, 40, 16, 128, 128, 64, 30),      # chunk shorter than the window (40 window columns)
    (3, 1, 257, 8, 64, 128, 0, 0),         # window only
    (4, 3, 33, 24, 256, 16, 500, 180),     # ragged heads, long compressed part
    (5, 1, 1, 4, 512, 8, 10, 5),           # a single query
    (6, 1, 70, 16, 128, 64, 3000, 2500),   # 2564-entry lists: compacted in two chunks
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_prefill_step_vs_oracle(case):
    seed, b, s, h, d, W, ncr, kc = case
    print(f"prefill step case {case}", flush=True)
    c = make_case(seed, b, s, h, d, W, ncr, kc)
    idx_ref, ref = oracle_case(c)
    idx_got, got = gpu_fused(c)
    assert np.array_equal(idx_got, idx_ref), "written list"
    assert_parity(got, ref, f"prefill step {case}")


VARIANTS = [(sa.SA_KERNEL_PAIR, 1), (sa.SA_KERNEL_PAIR, 2), (sa.SA_KERNEL_PAIR, 3)]


@pytest.mark.parametrize("variant", VARIANTS, ids=[f"k{k}-sp{sp}" for k, sp in VARIANTS])
def test_prefill_step_splits_match_separate_calls(variant):
    c = make_case(11, 1, 150, 64, 512, 64, 300, 120)
    print(f"prefill step variant {variant}", flush=True)
    idx_ref, ref = oracle_case(c)
    idx_got, got = gpu_fused(c, variant)
    assert np.array_equal(idx_got, idx_ref), "written list"
    assert_parity(got, ref, f"prefill step {variant}")
    assert np.array_equal(got, gpu_separate(c, variant)), "bit for bit against the separate calls"


def test_prefill_step_errors():
    q = torch.zeros((1, 4, 2, 64), dtype=torch.bfloat16, device=DEV)
    sink = torch.zeros(2, device=DEV)
    with pytest.raises(sa.SparseAttnError) as e:      # fewer kv rows than chunk rows
        sa.sparse_attn_prefill_step(q, torch.zeros((1, 3, 64), dtype=torch.bfloat16, device=DEV), sink, 4, 0.1)
    assert e.value.status == sa.SA_ERR_SHAPE
    with pytest.raises(sa.SparseAttnError) as e:      # window of 0
        sa.sparse_attn_prefill_step(q, torch.zeros((1, 4, 64), dtype=torch.bfloat16, device=DEV), sink, 0, 0.1)
    assert e.value.status == sa.SA_ERR_SHAPE
    for k in (sa.SA_KERNEL_WIDE, sa.SA_KERNEL_DECODE):  # only the pair kernel builds this list
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_prefill_step(q, torch.zeros((1, 4, 64), dtype=torch.bfloat16, device=DEV), sink, 4, 0.1,
                                        variant=(k, 1))
        assert e.value.status == sa.SA_ERR_UNSUPPORTED


def test_prefill_step_with_rotation_matches_separate_calls():
    """The output's inverse rotation fused into the prefill step: bit for bit the
    separate calls with the rotation fused into sa_sparse_attn (itself checked
    against the oracle's exact rotation)."""
    from sparse_latent_attention_02_amd.workloads import rope_table
    c = make_case(21, 2, 200, 32, 512, 64, 150, 80)
    b, s, W, kc, d = 2, 200, 64, 80, 512
    table = rope_table(77, s, 64).to(DEV)
    variant = (sa.SA_KERNEL_PAIR, 1)                 # one variant on both sides: the same arithmetic
    out = sa.sparse_attn_prefill_step(c["q"].to(DEV), c["kv"].to(DEV), c["sink"].to(DEV), W, d ** -0.5,
                                      cidx=c["cidx"].to(DEV), rope=(table, 64), variant=variant)
    idx = torch.full((b, s, min(s, W) + kc), -7, dtype=torch.int32, device=DEV)
    sa.window_topk_idxs(W, b, s, 0, out=idx)
    sa.append_compressed_idxs(idx, min(s, W), c["cidx"].to(DEV), s)
    ref = sa.sparse_attn(c["q"].to(DEV), c["kv"].to(DEV), c["sink"].to(DEV), idx, d ** -0.5, rope=(table, 64, 0),
                         variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))



@pytest.mark.parametrize("d", [64, 512])
def test_prefill_step_scores_outrunning_the_first_stage(d):
    """The pair kernel takes the weights against the first stage max it sees and
    replays the list (copied again from memory, window entries formed again) when
    a later stage outruns it by too much.  Two compressed rows built from query 3's
    head row 5 sit at list entries 130 and 250; the result must still be the plain
    softmax, dominated there by the second."""
    g = torch.Generator().manual_seed(78)
    b, s, h, W, kc = 1, 4, 64, 4, 300
    q = torch.randn((b, s, h, d), generator=g).to(torch.bfloat16)
    kv = (0.05 * torch.randn((b, s + kc, d), generator=g)).to(torch.bfloat16)
    c1 = 60.0 / (d ** 0.5 * 1.4426950408889634)   # log2-domain score about 60 above the rest
    kv[0, s + 130 - W] = (c1 * q[0, 3, 5].float()).to(torch.bfloat16)
    kv[0, s + 250 - W] = (2.2 * c1 * q[0, 3, 5].float()).to(torch.bfloat16)
    cidx = torch.arange(kc, dtype=torch.int32).repeat(b, s, 1).contiguous()
    sink = torch.randn(h, generator=g)
    c = dict(q=q, kv=kv, sink=sink, cidx=cidx, W=W, s=s, h=h, d=d, kc=kc)
    idx_ref, ref = oracle_case(c)
    idx_got, got = gpu_fused(c)
    assert np.array_equal(idx_got, idx_ref), "written list"
    assert_parity(got, ref, f"prefill replay d {d}")
    r = ref.reshape(b, s, h, d)[0, 3, 5]
    assert np.allclose(r, kv[0, s + 250 - W].float().numpy(), rtol=2e-2, atol=2e-2)
