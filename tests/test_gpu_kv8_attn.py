"""GPU parity of the attention over fp8-resident rows (sa_sparse_attn_kv8,
sa_sparse_attn_decode_step_kv8).

The rows are packed by the oracle (e4m3fn codes + E8M0 scale bytes) and the
oracle's attention runs on its own expansion of them: output within
max(2 bf16 ulp, 1e-2) of the oracle's f32 value.  Since the kernel expands each
row to exactly the bf16 values of that expansion, the output must also equal,
bit for bit, the bf16 decode kernel's (same splits) on the expanded rows.  The
decode step's ring write is checked as codes + scale record, bit for bit,
against the oracle's packing of the oracle's KV buffer after the step.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_latent_attention_02_amd as sa
from helpers import assert_parity, bits, from_bits, require_gpu
from test_gpu_decode_step import make_case, oracle_step

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    sa.lib()
    oracle.lib()


def records(scales: np.ndarray) -> np.ndarray:
    """Oracle scale bytes [..., d / 32] -> the library's 16-byte scale records."""
    rec = np.full(scales.shape[:-1] + (sa.KV8_SCALE_BYTES,), 127, dtype=np.uint8)
    rec[..., : scales.shape[-1]] = scales
    return rec


def kv8_case(seed, b, s, h, d, rows, topk, p_hole=0.15, spread=4.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((b, s, h, d), generator=g).to(torch.bfloat16)
    # row magnitudes spread over many binades, so the blocks' scale bytes differ widely
    kv = (torch.randn((b, rows, d), generator=g) * torch.exp(torch.randn((b, rows, 1), generator=g) * spread))
    kv = kv.to(torch.bfloat16)
    sink = torch.randn((h,), generator=g)
    idx = torch.randint(0, max(rows, 1), (b, s, topk), generator=g, dtype=torch.int32)
    idx[torch.rand((b, s, topk), generator=g) < p_hole] = -1
    if rows == 0:
        idx.fill_(-1)
    codes, scales = oracle.kv8_pack(bits(kv))
    kv_rt = oracle.kv8_unpack(codes, scales)
    return q, codes, records(scales), kv_rt, sink, idx


CASES = [
    # (seed, b, s, h, d, rows, topk)
    (1, 2, 1, 64, 512, 300, 128),        # a decode step's window list
    (2, 1, 2, 20, 512, 3000, 2176),      # window + compressed: long list, heads not a multiple of 16
    (3, 2, 2, 16, 256, 500, 300),        # ragged last stage
    (4, 3, 1, 33, 128, 200, 77),
    (5, 2, 3, 8, 64, 100, 64),
    (6, 1, 4, 64, 512, 1024, 200),       # several queries of a prefill chunk
    (7, 2, 1, 16, 512, 40, 0),           # empty list: zeros
    (8, 1, 1, 16, 512, 0, 33),           # no rows, every entry -1: zeros
]
SPLITS = [0, 1, 3]


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
@pytest.mark.parametrize("splits", SPLITS, ids=[f"sp{s}" for s in SPLITS])
def test_kv8_attn_vs_oracle_and_bf16_kernel(case, splits):
    seed, b, s, h, d, rows, topk = case
    print(f"kv8 attention case {case} splits {splits}", flush=True)
    q, codes, recs, kv_rt, sink, idx = kv8_case(seed, b, s, h, d, rows, topk)
    qd, sinkd, idxd = q.to(DEV), sink.to(DEV), idx.to(DEV)
    out = sa.sparse_attn_kv8(qd, torch.from_numpy(codes).to(DEV), torch.from_numpy(recs).to(DEV), sinkd, idxd,
                             d ** -0.5, splits=splits)
    kvd = from_bits(kv_rt).to(DEV) if rows else torch.zeros((b, 1, d), dtype=torch.bfloat16, device=DEV)
    ref16 = sa.sparse_attn(qd, kvd, sinkd, idxd, d ** -0.5, variant=(sa.SA_KERNEL_DECODE, splits))
    torch.cuda.synchronize()
    _, ref = oracle.sparse_attn(bits(q), kv_rt.reshape(b, rows, d), sink.numpy(), idx.numpy(), d ** -0.5,
                                want_f32=True)
    assert_parity(bits(out), ref, f"kv8 {case} splits {splits}")
    assert np.array_equal(bits(out), bits(ref16)), "kv8 rows must give the bf16 kernel's result bit for bit"


def test_kv8_attn_out_of_range_entries_are_skipped():
    q, codes, recs, kv_rt, sink, idx = kv8_case(21, 2, 1, 16, 512, 64, 100)
    idx_bad = idx.clone()
    idx_bad[:, :, ::7] = 64 + 5            # past the last row: treated as -1
    idx_ref = idx.clone()
    idx_ref[:, :, ::7] = -1
    args = (torch.from_numpy(codes).to(DEV), torch.from_numpy(recs).to(DEV), sink.to(DEV))
    a = sa.sparse_attn_kv8(q.to(DEV), *args, idx_bad.to(DEV), 0.0625)
    r = sa.sparse_attn_kv8(q.to(DEV), *args, idx_ref.to(DEV), 0.0625)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(r))


def assert_same(got: np.ndarray, ref: np.ndarray, what: str):
    if np.array_equal(got, ref):
        return
    bad = np.argwhere(got != ref)
    rows = sorted({tuple(int(v) for v in r[:-1]) for r in bad})
    first = tuple(int(v) for v in bad[0])
    raise AssertionError(f"{what}: {len(bad)} elements differ in rows {rows[:8]}; first {first}: "
                         f"got {got[first]} want {ref[first]}")


def expected_records(c):
    """The kv8 cache after a step: the new row's slot holds the oracle's packing
    of the raw new row (its expansion is the round-tripped row the bf16 step
    writes); every other row is unchanged."""
    b, d, slot = c["kv_bits"].shape[0], c["d"], c["pos"] % c["W"]
    codes, scales = oracle.kv8_pack(c["kv_bits"])
    nc, ns = oracle.kv8_pack(bits(c["kv_new"]).reshape(b, d))
    codes[:, slot], scales[:, slot] = nc, ns
    return codes, scales


def kv8_decode_case(case):
    seed, b, h, d, W, ncr, kc, pos = case
    c = make_case(seed, b, h, d, W, ncr, kc, pos)
    codes, scales = oracle.kv8_pack(c["kv_bits"])
    c["codes"], c["recs"] = codes, records(scales)
    # the bf16 cache the kv8 one stands for (the round trip is idempotent, so this is kv_bits)
    assert np.array_equal(oracle.kv8_unpack(codes, scales), c["kv_bits"])
    return c


DECODE_CASES = [
    # (seed, b, h, d, W, comp rows, kc, pos)
    (1, 4, 64, 512, 128, 0, 0, 5000),
    (2, 3, 64, 512, 128, 0, 0, 3),
    (3, 2, 20, 512, 128, 0, 0, 127),
    (4, 3, 16, 256, 200, 0, 0, 1000),
    (5, 2, 4, 64, 8, 0, 0, 13),
    (6, 2, 33, 128, 64, 300, 200, 777),
    (7, 2, 128, 512, 128, 4096, 2048, 5000),
    (8, 1, 64, 512, 128, 1000, 900, 129),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"case{c[0]}" for c in DECODE_CASES])
@pytest.mark.parametrize("splits", [0, 1, 3], ids=lambda s: f"sp{s}")
def test_kv8_decode_step_vs_oracle(case, splits):
    c = kv8_decode_case(case)
    b, W, d, h = c["kv_bits"].shape[0], c["W"], c["d"], c["h"]
    kc = 0 if c["cidx"] is None else c["cidx"].shape[1]
    print(f"kv8 decode step case {case} splits {splits}", flush=True)
    kv_ref, idx_ref, out_ref = oracle_step(c)
    codes = torch.from_numpy(c["codes"]).to(DEV)
    recs = torch.from_numpy(c["recs"]).to(DEV)
    kv_new = c["kv_new"].to(DEV)
    idx_out = torch.full((b, W + kc), -7, dtype=torch.int32, device=DEV)
    cidx = c["cidx"].to(DEV) if kc else None
    out = sa.sparse_attn_decode_step_kv8(c["q"].to(DEV), codes, recs, kv_new, c["sink"].to(DEV), W, c["pos"],
                                         d ** -0.5, cidx=cidx, idx_out=idx_out, splits=splits)
    # the bf16 step on the same cache, same kernel and splits
    kv16 = from_bits(c["kv_bits"]).to(DEV)
    out16 = sa.sparse_attn_decode_step(c["q"].to(DEV), kv16, kv_new, c["sink"].to(DEV), W, c["pos"], d ** -0.5,
                                       cidx=cidx, variant=(sa.SA_KERNEL_DECODE, splits))
    torch.cuda.synchronize()
    assert torch.equal(kv_new.cpu(), c["kv_new"]), "kv_new must stay untouched"
    rc, rs = expected_records(c)
    assert np.array_equal(oracle.kv8_unpack(rc, rs), kv_ref)   # (oracle-side consistency)
    assert_same(codes.cpu().numpy(), rc, "codes after the step")
    assert_same(recs.cpu().numpy(), records(rs), "scale records after the step")
    assert np.array_equal(idx_out.cpu().numpy(), idx_ref), "index list written out"
    assert_parity(bits(out), out_ref, f"kv8 decode step {case} splits {splits}")
    assert np.array_equal(bits(out), bits(out16)), "kv8 step must give the bf16 step's result bit for bit"


def test_kv8_decode_step_chain():
    """Eight steps in a row on one kv8 cache (each step attends to the rows the
    previous ones wrote) against the oracle's steps on its bf16 cache."""
    b, h, d, W = 2, 16, 512, 8
    g = torch.Generator().manual_seed(99)
    kv_bits = bits(torch.zeros((b, W, d), dtype=torch.bfloat16))
    codes, scales = oracle.kv8_pack(kv_bits)
    codes_d, recs_d = torch.from_numpy(codes).to(DEV), torch.from_numpy(records(scales)).to(DEV)
    sink = torch.randn((h,), generator=g)
    for pos in range(5, 13):
        q = torch.randn((b, h, d), generator=g).to(torch.bfloat16)
        kv_new = (torch.randn((b, d), generator=g) * 3).to(torch.bfloat16)
        c = dict(q=q, kv_bits=kv_bits, kv_new=kv_new, sink=sink, cidx=None, rows=W, W=W, pos=pos, h=h, d=d)
        kv_bits, _, out_ref = oracle_step(c)
        out = sa.sparse_attn_decode_step_kv8(q.to(DEV), codes_d, recs_d, kv_new.to(DEV), sink.to(DEV), W, pos,
                                             d ** -0.5)
        torch.cuda.synchronize()
        assert_parity(bits(out), out_ref, f"chain step {pos}")
        codes[:, pos % W], scales[:, pos % W] = oracle.kv8_pack(bits(kv_new))
        assert np.array_equal(oracle.kv8_unpack(codes, scales), kv_bits)
        assert_same(codes_d.cpu().numpy(), codes, f"codes after step {pos}")
        assert_same(recs_d.cpu().numpy(), records(scales), f"scale records after step {pos}")


def test_kv8_argument_errors():
    q = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16, device=DEV)
    codes = torch.zeros((1, 8, 64), dtype=torch.uint8, device=DEV)
    recs = torch.full((1, 8, 16), 127, dtype=torch.uint8, device=DEV)
    sink = torch.zeros((4,), device=DEV)
    idx = torch.zeros((1, 1, 4), dtype=torch.int32, device=DEV)
    lib = sa.lib()
    # misaligned codes
    st = lib.sa_sparse_attn_kv8(q.data_ptr(), codes.data_ptr() + 1, recs.data_ptr(), sink.data_ptr(),
                                idx.data_ptr(), 1, 1, 4, 64, 8, 4, 0.125, q.data_ptr(), None, 0, None, 0)
    assert st == sa.SA_ERR_SHAPE
    # missing scale records
    st = lib.sa_sparse_attn_kv8(q.data_ptr(), codes.data_ptr(), None, sink.data_ptr(), idx.data_ptr(),
                                1, 1, 4, 64, 8, 4, 0.125, q.data_ptr(), None, 0, None, 0)
    assert st == sa.SA_ERR_NULL
    # head dim outside the supported set
    st = lib.sa_sparse_attn_kv8(q.data_ptr(), codes.data_ptr(), recs.data_ptr(), sink.data_ptr(),
                                idx.data_ptr(), 1, 1, 4, 96, 8, 4, 0.125, q.data_ptr(), None, 0, None, 0)
    assert st == sa.SA_ERR_UNSUPPORTED
    # decode step at position 0
    kv_new = torch.zeros((1, 64), dtype=torch.bfloat16, device=DEV)
    st = lib.sa_sparse_attn_decode_step_kv8(q.data_ptr(), codes.data_ptr(), recs.data_ptr(), kv_new.data_ptr(),
                                            sink.data_ptr(), None, None, 1, 4, 64, 8, 8, 0, 0, 0.125,
                                            q.data_ptr(), None, 0, None, 0)
    assert st == sa.SA_ERR_UNSUPPORTED
    # split workspace too small
    idx_long = torch.zeros((1, 1, 1024), dtype=torch.int32, device=DEV)
    need = sa.kv8_workspace_bytes(1, 1, 4, 64, 1024, 2)
    assert need > 0
    st = lib.sa_sparse_attn_kv8(q.data_ptr(), codes.data_ptr(), recs.data_ptr(), sink.data_ptr(),
                                idx_long.data_ptr(), 1, 1, 4, 64, 8, 1024, 0.125, q.data_ptr(), None, 0, None, 2)
    assert st in (sa.SA_ERR_NULL, sa.SA_ERR_SHAPE)
