"""GPU parity of the fp8-resident KV rows (kv8): sa_kv8_pack against the
oracle's codes and scale bytes bit for bit, sa_kv8_unpack against the oracle's
expansion bit for bit (every code at many scales), and the expansion of a
packed row against the fp8 round trip of the row."""
import numpy as np
import pytest
import torch

import oracle
import sparse_latent_attention_02_amd as sa
from helpers import act_quant_blocks, bits, from_bits, require_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    sa.lib()
    oracle.lib()


def test_kv8_pack_exhaustive_bitexact():
    blocks = act_quant_blocks()                     # every finite bf16 under many block scales
    rows = blocks.reshape(-1, 32)
    codes, scales = sa.kv8_pack(from_bits(rows).to(DEV))
    torch.cuda.synchronize()
    rc, rs = oracle.kv8_pack(rows)
    assert np.array_equal(codes.cpu().numpy(), rc)
    s = scales.cpu().numpy()
    assert np.array_equal(s[:, :1], rs)
    assert np.all(s[:, 1:] == 127)


@pytest.mark.parametrize("row_len", [32, 64, 128, 256, 512])
def test_kv8_round_trip_random_rows(row_len):
    g = torch.Generator().manual_seed(row_len)
    x = (torch.randn((300, row_len), generator=g) * torch.exp(torch.randn((300, 1), generator=g) * 6)).to(torch.bfloat16)
    xd = x.to(DEV)
    codes, scales = sa.kv8_pack(xd)
    back = sa.kv8_unpack(codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.kv8_pack(bits(x))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy()[:, : row_len // 32], rs)
    assert np.array_equal(bits(back), oracle.act_quant_fp8(bits(x)))


def test_kv8_unpack_every_code_at_many_scales():
    codes = np.tile(np.arange(256, dtype=np.uint8), 64).reshape(-1, 32)     # 512 rows of 32
    codes[(codes == 0x7f) | (codes == 0xff)] = 0                             # NaN codes are never produced
    sbytes = np.arange(105, 105 + codes.shape[0]) % 143 + 105                # scales 2^-22 .. 2^120
    scales = np.full((codes.shape[0], 16), 127, dtype=np.uint8)
    scales[:, 0] = sbytes
    got = sa.kv8_unpack(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.kv8_unpack(codes, scales[:, :1].copy())
    assert np.array_equal(bits(got), ref)


def test_kv8_argument_errors():
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.kv8_pack(x)
    assert e.value.status == sa.SA_ERR_SHAPE
    x = torch.zeros((4, 1024), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.kv8_pack(x)
    assert e.value.status == sa.SA_ERR_UNSUPPORTED
