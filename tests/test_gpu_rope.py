"""GPU parity of the rotary embedding (sa_apply_rotary) and of the output's
inverse rotation fused into the attention epilogue (sa_sparse_attn_rope,
sa_sparse_attn_decode_step_rope).

sa_apply_rotary against the oracle bit for bit (both take the f32 products and
sum of the pages' precision contract, with no fused multiply-add).  The fused
epilogue against the unfused pair of GPU calls bit for bit (it rotates the same
rounded bf16 output with the same arithmetic), and against the oracle's
attention followed by the oracle's inverse rotation within the attention
tolerance carried through the rotation.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_latent_attention_02_amd as sa
from sparse_latent_attention_02_amd import workloads as wl
from helpers import bf16_f32, bf16_ulp, bits, from_bits, parity_tolerance, require_gpu
from test_gpu_decode_step import make_case, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    sa.lib()
    oracle.lib()


ROT_CASES = [
    # (seed, b, s, h, row_len, rope_dim, start_pos)
    (1, 2, 5, 3, 128, 64, 7),
    (2, 1, 12, 4, 64, 64, 0),       # the whole row rotated
    (3, 3, 1, 64, 512, 64, 5000),   # a decode step's output
    (4, 1, 33, 1, 96, 2, 100),      # one pair, [b][s][row_len] rows
]


@pytest.mark.parametrize("case", ROT_CASES, ids=[f"case{c[0]}" for c in ROT_CASES])
@pytest.mark.parametrize("inverse", [False, True], ids=["fwd", "inv"])
def test_apply_rotary_bitexact(case, inverse):
    seed, b, s, h, row_len, rd, pos0 = case
    g = torch.Generator().manual_seed(seed)
    shape = (b, s, h, row_len) if h > 1 else (b, s, row_len)
    x = (torch.randn(shape, generator=g) * torch.exp(torch.randn(shape[:-1] + (1,), generator=g) * 3)).to(
        torch.bfloat16)
    table = wl.rope_table(seed, pos0 + s + 3, rd)
    xd = x.to(DEV)
    sa.apply_rotary(xd, table.to(DEV), rd, pos0, inverse)
    torch.cuda.synchronize()
    ref = oracle.apply_rotary(bits(x), table.numpy(), rd, pos0, inverse)
    assert np.array_equal(bits(xd), ref)


def rotated_parity(gpu_bits, ref_f32, rd, pos0, table, what):
    """GPU output (rotated) vs the oracle's f32 attention output rotated exactly:
    the attention tolerance of a pair's two values carries through the rotation,
    plus the last rounding."""
    d = ref_f32.shape[-1]
    g = bf16_f32(gpu_bits).astype(np.float64)
    r = ref_f32.astype(np.float64)
    tol = parity_tolerance(r)
    s = r.shape[1]
    w = table[pos0:pos0 + s].astype(np.float64)                   # [s][rd/2][2]
    c = w[None, :, None, :, 0]
    sn = w[None, :, None, :, 1]
    a, b_ = r[..., d - rd::2], r[..., d - rd + 1::2]
    re, im = a * c + b_ * sn, b_ * c - a * sn
    ta, tb = tol[..., d - rd::2], tol[..., d - rd + 1::2]
    rot_tol = ta + tb
    assert np.all(np.abs(g[..., :d - rd] - r[..., :d - rd]) <= tol[..., :d - rd]), what
    assert np.all(np.abs(g[..., d - rd::2] - re) <= rot_tol + bf16_ulp(re)), what
    assert np.all(np.abs(g[..., d - rd + 1::2] - im) <= rot_tol + bf16_ulp(im)), what


ATTN_CASES = [
    # (seed, b, s, h, d, rows, topk, rope_dim, start_pos)
    (11, 1, 40, 64, 512, 300, 128, 64, 0),      # prefill-like: one position per query
    (12, 4, 1, 64, 512, 200, 128, 64, 4999),    # decode-like
    (13, 2, 3, 20, 256, 90, 77, 32, 10),        # heads not a multiple of 16, ragged list
    (14, 1, 5, 8, 64, 40, 16, 64, 2),           # the whole row rotated
    (15, 1, 3, 16, 512, 64, 64, 512, 0),        # a table row of two copy instructions
    (16, 2, 2, 16, 512, 64, 50, 264, 3),        # ... the second one partial
    (17, 1, 3, 64, 512, 3000, 1500, 64, 100),   # a long list (the pair kernel's long-list chunk)
]
VARIANTS = [None, (1, 1), (1, 3), (2, 1), (2, 4), (3, 1), (3, 3)]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[f"case{c[0]}" for c in ATTN_CASES])
@pytest.mark.parametrize("variant", VARIANTS, ids=str)
def test_attn_rope_fused_vs_unfused_and_oracle(case, variant):
    seed, b, s, h, d, rows, topk, rd, pos0 = case
    print(f"attention + inverse rotation case {case} variant {variant}", flush=True)
    c = wl.small_case(seed, b, s, h, d, rows, topk, p_invalid=0.1)
    kvb = bits(c["kv"]).copy()
    oracle.act_quant_fp8_inplace(kvb)
    table = wl.rope_table(seed, pos0 + s, rd)
    q, kv, sink, idx = c["q"].to(DEV), from_bits(kvb).to(DEV), c["sink"].to(DEV), c["idx"].to(DEV)
    tabd = table.to(DEV)
    fused = sa.sparse_attn(q, kv, sink, idx, d ** -0.5, variant=variant, rope=(tabd, rd, pos0))
    plain = sa.sparse_attn(q, kv, sink, idx, d ** -0.5, variant=variant)
    sa.apply_rotary(plain, tabd, rd, pos0, inverse=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(fused), bits(plain)), "fused epilogue == attention, then sa_apply_rotary"
    _, ref = oracle.sparse_attn(bits(c["q"]), kvb, c["sink"].numpy(), c["idx"].numpy(), d ** -0.5, want_f32=True)
    rotated_parity(bits(fused), ref, rd, pos0, table.numpy(), f"{case} {variant}")


STEP_CASES = [
    # (seed, b, h, d, W, comp rows, kc, pos)
    (21, 4, 64, 512, 128, 0, 0, 5000),
    (22, 2, 33, 128, 64, 300, 200, 777),
    (23, 2, 128, 512, 128, 4096, 2048, 5000),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[f"case{c[0]}" for c in STEP_CASES])
@pytest.mark.parametrize("variant", [None, (1, 1), (2, 1), (2, 3)], ids=str)
def test_decode_step_rope(case, variant):
    seed, b, h, d, W, ncr, kc, pos = case
    rd = 64
    print(f"decode step + inverse rotation case {case} variant {variant}", flush=True)
    c = make_case(seed, b, h, d, W, ncr, kc, pos)
    table = wl.rope_table(seed, pos + 1, rd)
    tabd = table.to(DEV)
    outs = []
    for rope in ((tabd, rd), None):
        kv = from_bits(c["kv_bits"]).to(DEV)
        o = sa.sparse_attn_decode_step(c["q"].to(DEV), kv, c["kv_new"].to(DEV), c["sink"].to(DEV), W, pos,
                                       d ** -0.5, cidx=c["cidx"].to(DEV) if kc else None, variant=variant,
                                       rope=rope)
        outs.append(o)
    sa.apply_rotary(outs[1].view(b, 1, h, d), tabd, rd, pos, inverse=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(outs[0]), bits(outs[1]))
    _, _, ref = oracle_step(c)
    rotated_parity(bits(outs[0]).reshape(b, 1, h, d), ref.reshape(b, 1, h, d), rd, pos, table.numpy(),
                   f"step {case} {variant}")


def test_rope_argument_errors():
    c = wl.small_case(31, 1, 2, 4, 64, 8, 4)
    q, kv, sink, idx = c["q"].to(DEV), c["kv"].to(DEV), c["sink"].to(DEV), c["idx"].to(DEV)
    for rd, n_pos, pos0, st in ((12, 8, 0, sa.SA_ERR_SHAPE),     # not a multiple of 8
                                (72, 8, 0, sa.SA_ERR_SHAPE),     # longer than the row
                                (16, 3, 2, sa.SA_ERR_SHAPE)):    # positions past the table
        table = wl.rope_table(1, n_pos, max(rd, 2)).to(DEV)
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn(q, kv, sink, idx, 0.125, rope=(table, rd, pos0))
        assert e.value.status == st
    lib = sa.lib()
    st = lib.sa_sparse_attn_rope(q.data_ptr(), kv.data_ptr(), sink.data_ptr(), idx.data_ptr(), 1, 2, 4, 64, 8, 4,
                                 0.125, q.data_ptr(), None, 0, None, 0, 0, None, 8, 16, 0)
    assert st == sa.SA_ERR_NULL
    x = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.apply_rotary(x, wl.rope_table(1, 4, 16).to(DEV), 15, 0)
    assert e.value.status == sa.SA_ERR_SHAPE
