"""GPU test of the allocation-free entry point (sa_sparse_attn_noalloc), through
the C ABI: its output equals, bit for bit, that of sa_sparse_attn_ex with the
same variant and a caller-allocated workspace, on two calls in a row (the
second with a smaller input, so it runs on what the first left in the
library's scratch), for variants that split the index list (partials in the
scratch) and ones that do not; a call whose partials exceed the scratch is
rejected with nothing written."""
import numpy as np
import pytest
import torch

import oracle
import sparse_latent_attention_02_amd as sa
from sparse_latent_attention_02_amd import workloads as wl
from helpers import assert_parity, bits, from_bits, require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    sa.lib()
    oracle.lib()


def inputs(seed, b, s, h, d, rows, topk):
    c = wl.small_case(seed, b, s, h, d, rows, topk, p_invalid=0.1)
    kvb = bits(c["kv"]).copy()
    oracle.act_quant_fp8_inplace(kvb)
    return c, kvb


# (kernel, splits) and two shapes (seed, b, s, h, d, rows, topk): the second smaller
CASES = [
    ((sa.SA_KERNEL_DECODE, 3), (1, 6, 1, 64, 512, 700, 640), (2, 2, 1, 20, 512, 300, 200)),
    ((sa.SA_KERNEL_WIDE, 4), (3, 3, 2, 128, 512, 3000, 2176), (4, 1, 1, 64, 512, 500, 300)),
    ((sa.SA_KERNEL_PAIR, 2), (5, 1, 5, 64, 512, 900, 700), (6, 1, 2, 33, 256, 100, 90)),
    ((sa.SA_KERNEL_AUTO, 0), (7, 4, 1, 128, 512, 4000, 2176), (8, 2, 1, 64, 128, 100, 64)),   # automatic split
    ((sa.SA_KERNEL_DECODE, 1), (9, 4, 1, 64, 512, 200, 128), (10, 1, 1, 16, 64, 40, 16)),      # no partials
]


@pytest.mark.parametrize("variant,first,second", CASES, ids=[f"{c[0]}" for c in CASES])
def test_noalloc_equals_workspace_entry(variant, first, second):
    assert sa.noalloc_scratch_bytes() == 32 << 20
    for shape in (first, second):
        seed, b, s, h, d, rows, topk = shape
        print(f"noalloc variant {variant} shape {shape}", flush=True)
        c, kvb = inputs(seed, b, s, h, d, rows, topk)
        q, kv, sink, idx = c["q"].to(DEV), from_bits(kvb).to(DEV), c["sink"].to(DEV), c["idx"].to(DEV)
        need = sa.workspace_bytes(b, s, h, d, topk, variant)
        if variant[1] > 1:
            assert need > 0, "the case must put partials in the scratch"
        out_na = torch.full_like(q, float("nan"))
        sa.sparse_attn_noalloc(q, kv, sink, idx, d ** -0.5, out_na, variant=variant)
        ref = sa.sparse_attn(q, kv, sink, idx, d ** -0.5, variant=variant)     # caller-allocated workspace
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_na), bits(ref)), f"{variant} {shape}"
        _, ref32 = oracle.sparse_attn(bits(c["q"]), kvb, c["sink"].numpy(), c["idx"].numpy(), d ** -0.5,
                                      want_f32=True)
        assert_parity(bits(out_na), ref32, f"noalloc {variant} {shape}")


def test_noalloc_rejects_partials_past_the_scratch():
    # wide kernel, 8 splits, 64 queries x 128 heads: 64 * 8 * 128 * 514 * 4 B > 32 MiB
    b, s, h, d, topk = 64, 1, 128, 512, 2176
    variant = (sa.SA_KERNEL_WIDE, 8)
    assert sa.workspace_bytes(b, s, h, d, topk, variant) > sa.noalloc_scratch_bytes()
    q = torch.zeros((b, s, h, d), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((b, 4, d), dtype=torch.bfloat16, device=DEV)
    idx = torch.full((b, s, topk), -1, dtype=torch.int32, device=DEV)
    sink = torch.zeros((h,), device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_noalloc(q, kv, sink, idx, 0.1, out, variant=variant)
    assert e.value.status == sa.SA_ERR_SHAPE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "nothing enqueued on a rejected call"
