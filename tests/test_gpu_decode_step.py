"""GPU parity of the fused decode step (sa_sparse_attn_decode_step): the ring
write with its fp8 round trip, the window list, the compressed append and the
attention in one launch.

Against the oracle applying its own step functions to the same raw inputs:
the KV buffer after the step and the written index list bit for bit, the
output within max(2 bf16 ulp, 1e-2) of the oracle's f32 value.  Against the
separate GPU calls (sa_window_kv_update, sa_window_topk_idxs,
sa_append_compressed_idxs, sa_sparse_attn_ex with the same variant): the output
bit for bit, since both run the same arithmetic on the same list.
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


def make_case(seed, b, h, d, W, n_comp_rows, kc, pos, p_hole=0.1):
    g = torch.Generator().manual_seed(seed)
    rows = W + n_comp_rows
    q = torch.randn((b, h, d), generator=g).to(torch.bfloat16)
    kv = torch.randn((b, rows, d), generator=g).to(torch.bfloat16)
    kv_new = torch.randn((b, d), generator=g).to(torch.bfloat16)
    sink = torch.randn((h,), generator=g)
    kv_bits = bits(kv).copy()
    oracle.act_quant_fp8_inplace(kv_bits)          # the cache before the step
    cidx = None
    if kc:
        cidx = torch.randint(0, max(n_comp_rows, 1), (b, kc), generator=g, dtype=torch.int32)
        holes = torch.rand((b, kc), generator=g) < p_hole
        cidx[holes] = -1
    return dict(q=q, kv_bits=kv_bits, kv_new=kv_new, sink=sink, cidx=cidx, rows=rows, W=W, pos=pos, h=h, d=d)


def oracle_step(c):
    b, W, d = c["kv_bits"].shape[0], c["W"], c["d"]
    kv = c["kv_bits"].copy()
    new = bits(c["kv_new"]).reshape(b, 1, d).copy()
    oracle.act_quant_fp8_inplace(new)
    ring = np.ascontiguousarray(kv[:, :W])
    oracle.ring_write(ring, new, c["pos"])
    kv[:, :W] = ring
    kc = 0 if c["cidx"] is None else c["cidx"].shape[1]
    idx = np.full((b, 1, W + kc), -9, dtype=np.int32)
    oracle.window_topk_idxs_into(idx, W, b, 1, c["pos"])
    if kc:
        oracle.append_compressed_idxs(idx, W, np.ascontiguousarray(c["cidx"].numpy()).reshape(b, 1, kc), W)
    _, ref = oracle.sparse_attn(bits(c["q"]).reshape(b, 1, c["h"], d), kv, c["sink"].numpy(), idx,
                                c["d"] ** -0.5, want_f32=True)
    return kv, idx.reshape(b, W + kc), ref.reshape(b, c["h"], d)


def gpu_step(c, variant=None, with_idx=True):
    b, W = c["kv_bits"].shape[0], c["W"]
    kc = 0 if c["cidx"] is None else c["cidx"].shape[1]
    kv = torch.from_numpy(c["kv_bits"].view(np.int16)).view(torch.bfloat16).to(DEV)
    kv_new = c["kv_new"].to(DEV)
    idx_out = torch.full((b, W + kc), -7, dtype=torch.int32, device=DEV) if with_idx else None
    out = sa.sparse_attn_decode_step(c["q"].to(DEV), kv, kv_new, c["sink"].to(DEV), W, c["pos"], c["d"] ** -0.5,
                                     cidx=c["cidx"].to(DEV) if kc else None, idx_out=idx_out, variant=variant)
    torch.cuda.synchronize()
    assert torch.equal(kv_new.cpu(), c["kv_new"]), "kv_new must stay untouched"
    return bits(kv), (idx_out.cpu().numpy() if with_idx else None), bits(out)


def gpu_separate(c, variant):
    b, W, d, h = c["kv_bits"].shape[0], c["W"], c["d"], c["h"]
    kc = 0 if c["cidx"] is None else c["cidx"].shape[1]
    kv = torch.from_numpy(c["kv_bits"].view(np.int16)).view(torch.bfloat16).to(DEV)
    new = c["kv_new"].reshape(b, 1, d).to(DEV).contiguous()
    sa.window_kv_update(kv, new, c["pos"], window=W)
    idx = torch.empty((b, 1, W + kc), dtype=torch.int32, device=DEV)
    sa.window_topk_idxs(W, b, 1, c["pos"], out=idx)
    if kc:
        sa.append_compressed_idxs(idx, W, c["cidx"].reshape(b, 1, kc).to(DEV).contiguous(), W)
    out = sa.sparse_attn(c["q"].reshape(b, 1, h, d).to(DEV), kv, c["sink"].to(DEV), idx, d ** -0.5,
                         variant=variant)
    torch.cuda.synchronize()
    return bits(out).reshape(b, h, d)


CASES = [
    # (seed, b, h, d, W, comp rows, kc, pos)
    (1, 4, 64, 512, 128, 0, 0, 5000),        # decode window, the benchmark's shape per sequence
    (2, 3, 64, 512, 128, 0, 0, 3),           # ring still filling: most slots -1
    (3, 2, 20, 512, 128, 0, 0, 127),         # ring just full; heads not a multiple of 16
    (4, 3, 16, 256, 200, 0, 0, 1000),        # new row in the second 128-entry stage
    (5, 2, 4, 64, 8, 0, 0, 13),              # the worked example's ring size
    (6, 2, 33, 128, 64, 300, 200, 777),      # window + compressed, short list
    (7, 2, 128, 512, 128, 4096, 2048, 5000), # decode + compressed (long list)
    (8, 1, 64, 512, 128, 1000, 900, 129),    # compressed with the ring wrapped once
]
VARIANTS = [None, (1, 1), (1, 3), (2, 1), (2, 2), (2, 5), (3, 1), (3, 3)]


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
@pytest.mark.parametrize("variant", VARIANTS, ids=[str(v) for v in VARIANTS])
def test_decode_step_vs_oracle(case, variant):
    seed, b, h, d, W, ncr, kc, pos = case
    c = make_case(seed, b, h, d, W, ncr, kc, pos)
    print(f"decode step case {case} variant {variant}", flush=True)
    kv_ref, idx_ref, out_ref = oracle_step(c)
    kv_g, idx_g, out_g = gpu_step(c, variant)
    assert np.array_equal(kv_g, kv_ref), "KV buffer after the step"
    assert np.array_equal(idx_g, idx_ref), "index list written out"
    assert_parity(out_g, out_ref, f"decode step {case} {variant}")


@pytest.mark.parametrize("case", CASES[:4] + CASES[5:7], ids=[f"case{c[0]}" for c in CASES[:4] + CASES[5:7]])
@pytest.mark.parametrize("variant", [(1, 1), (2, 1), (2, 3), (1, 2), (3, 1), (3, 2)], ids=str)
def test_decode_step_equals_separate_calls(case, variant):
    seed, b, h, d, W, ncr, kc, pos = case
    c = make_case(seed, b, h, d, W, ncr, kc, pos)
    print(f"fused vs separate case {case} variant {variant}", flush=True)
    _, _, fused = gpu_step(c, variant, with_idx=False)
    sep = gpu_separate(c, variant)
    assert np.array_equal(fused, sep)


def test_decode_step_repeat_is_deterministic():
    c = make_case(11, 8, 64, 512, 128, 0, 0, 4242)
    a = gpu_step(c)
    b2 = gpu_step(c)
    for x, y in zip(a, b2):
        assert np.array_equal(x, y)


def test_decode_step_argument_errors():
    c = make_case(12, 2, 4, 64, 8, 0, 0, 9)
    q, kv, kv_new, sink = c["q"].to(DEV), torch.zeros((2, 8, 64), dtype=torch.bfloat16, device=DEV), \
        c["kv_new"].to(DEV), c["sink"].to(DEV)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_decode_step(q, kv, kv_new, sink, 8, 0, 0.125)
    assert e.value.status == sa.SA_ERR_UNSUPPORTED
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_decode_step(q, kv, kv_new, sink, 9, 5, 0.125)
    assert e.value.status == sa.SA_ERR_SHAPE
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_decode_step(q, kv, kv_new, sink, 8, 5, 0.125, variant=(4, 0))
    assert e.value.status == sa.SA_ERR_UNSUPPORTED
