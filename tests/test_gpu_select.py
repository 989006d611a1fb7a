"""GPU parity of the indexer's selection tail (sa_indexer_topk): bit for bit
against the oracle (both take equal scores at the lower position first), on
decode rows held in registers and longer ones read in chunks, causal prefill masks, the
take-everything case, heavy ties, -inf scores, zeros of both signs straddling
the k-th score (equal scores: -0.0 and +0.0 rank alike), and writes into the
compressed columns of a wider index buffer (other columns untouched)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_latent_attention_02_amd as sa
from helpers import require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    sa.lib()
    oracle.lib()


CASES = [
    # (seed, b, s, start_pos, ratio, index_topk, offset, score kind)
    (1, 128, 1, 65535, 4, 2048, 128, "normal"),    # decode: 16384 positions (keys in LDS)
    (2, 8, 1, 131071, 4, 2048, 128, "normal"),     # decode: 32768 positions (re-read from memory)
    (3, 1, 2048, 0, 4, 100, 2048, "normal"),       # prefill: causal mask, -inf ties past compress_lens
    (4, 1, 8192, 0, 4, 2048, 8192, "normal"),      # prefill: topk = T, everything in order
    (5, 16, 1, 40000, 4, 700, 128, "ties"),        # few distinct values: ties at the threshold
    (6, 4, 1, 20000, 4, 300, 0, "neginf"),         # -inf scores among finite ones
    (7, 3, 5, 77, 3, 9, 17, "normal"),             # a chunk after position 0
    (8, 2, 1, 4095, 1, 4096, 5, "ties"),           # ratio 1, topk = T
    (9, 16, 1, 16383, 4, 1000, 128, "zeros"),      # decode: +0 and -0 on both sides of the k-th score
    (10, 1, 2048, 0, 4, 200, 2048, "zeros"),       # prefill: the same, under the causal mask
    (11, 8, 1, 65535, 4, 2048, 128, "relu"),       # decode: ReLU scores times signed weights (many -0)
    (12, 2, 1, 131071, 4, 2048, 128, "zeros"),     # decode: rows re-read from memory, signed zeros
    (13, 6, 1, 40000, 3, 1500, 128, "normal"),     # decode: 13333 positions (odd: element loads, all tiles)
    (14, 4, 1, 65536, 4, 2048, 128, "normal"),     # decode: T = 16384, the register form's cap
    (15, 3, 1, 65539, 4, 3000, 128, "normal"),     # decode: T = 16385, one past the cap (streaming form)
    (17, 2, 1, 100000, 3, 2048, 128, "normal"),    # decode: T = 33333, streaming with element loads
    (18, 2, 1, 524287, 4, 4096, 128, "ties"),      # decode: T = 131072, equal keys taken across 8 chunks
]


def make_scores(seed, b, s, T, kind):
    g = torch.Generator().manual_seed(seed)
    if kind == "ties":
        return torch.randint(0, 4, (b, s, T), generator=g).to(torch.float32)
    if kind == "zeros":
        # 10% +1, 10% -1, the rest zeros of random sign: the k-th largest score
        # is a zero, with +0 and -0 entries on both sides of the cut
        u = torch.rand((b, s, T), generator=g)
        sign = torch.where(torch.rand((b, s, T), generator=g) < 0.5, -1.0, 1.0)
        return torch.where(u < 0.1, 1.0, torch.where(u < 0.2, -1.0, 0.0 * sign)).to(torch.float32)
    if kind == "relu":
        # the indexer's score form: ReLU of a logit times a signed weight
        x = torch.relu(torch.randn((b, s, T), generator=g))
        wgt = torch.randn((b, s, T), generator=g)
        return (x * wgt).to(torch.float32)
    sc = torch.randn((b, s, T), generator=g)
    if kind == "neginf":
        sc[torch.rand((b, s, T), generator=g) < 0.3] = -torch.inf
    return sc


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_indexer_topk_vs_oracle(case):
    seed, b, s, start_pos, ratio, index_topk, offset, kind = case
    T = (start_pos + s) // ratio
    print(f"indexer tail case {case} T={T}", flush=True)
    sc = make_scores(seed, b, s, T, kind)
    if kind in ("zeros", "relu"):
        z = sc == 0
        assert bool((z & torch.signbit(sc)).any()) and bool((z & ~torch.signbit(sc)).any())
    ref = oracle.indexer_topk(sc.numpy(), start_pos, ratio, index_topk, offset)
    got = sa.indexer_topk(sc.to(DEV), start_pos, ratio, index_topk, offset)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


def test_indexer_topk_misaligned_scores():
    """Rows whose length is a multiple of 4 but whose base is not 16-byte aligned
    take the element-load form."""
    b, s, start_pos, ratio, topk = 5, 1, 40959, 4, 1024
    T = (start_pos + s) // ratio
    sc = make_scores(16, b, s, T, "normal")
    flat = torch.empty(b * s * T + 1, dtype=torch.float32, device=DEV)
    view = flat[1:].view(b, s, T)
    view.copy_(sc.to(DEV))
    assert view.data_ptr() % 16 != 0 and T % 4 == 0
    got = sa.indexer_topk(view, start_pos, ratio, topk, 128)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.indexer_topk(sc.numpy(), start_pos, ratio, topk, 128))


def test_indexer_topk_into_the_compressed_columns():
    b, s, start_pos, ratio, topk, W = 4, 1, 9999, 4, 512, 128
    T = (start_pos + s) // ratio
    sc = make_scores(11, b, s, T, "normal")
    buf = torch.full((b, s, W + topk + 3), -9, dtype=torch.int32, device=DEV)
    sa.indexer_topk(sc.to(DEV), start_pos, ratio, topk, W, out=buf, col0=W)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.all(got[..., :W] == -9) and np.all(got[..., W + topk:] == -9)
    assert np.array_equal(got[..., W:W + topk], oracle.indexer_topk(sc.numpy(), start_pos, ratio, topk, W))


def test_indexer_topk_errors():
    sc = torch.zeros((1, 1, 10), device=DEV)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.indexer_topk(sc, 50, 4, 4, 0)                     # T != (start_pos + s) // ratio
    assert e.value.status == sa.SA_ERR_SHAPE
    out = torch.zeros((1, 1, 3), dtype=torch.int32, device=DEV)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.indexer_topk(sc, 40, 4, 4, 0, out=out)            # buffer narrower than topk
    assert e.value.status == sa.SA_ERR_SHAPE
