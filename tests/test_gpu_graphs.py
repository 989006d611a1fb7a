"""HIP graph capture of the hot path: every replay must reproduce the eager result
bit for bit (the kernels are deterministic), with eager work and synchronizations
between the replays."""
import pytest
import torch

import sparse_latent_attention_02_amd as sa
from sparse_latent_attention_02_amd import pipeline
from sparse_latent_attention_02_amd import workloads as wl
from helpers import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    sa.lib()


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_step_graph_replays():
    st = pipeline.prepare(2, wl.generate(2))
    eager = pipeline.step(st).clone()
    idx_eager = st.idx.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pipeline.step(st)
    for r in range(5):
        st.out.zero_()
        st.idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(st.out, eager), f"replay {r}: output differs"
        assert torch.equal(st.idx, idx_eager), f"replay {r}: index lists differ"
        _ = (st.q.float() * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("variant", [(1, 1), (1, 3), (2, 1), (2, 2), (3, 1), (3, 3)], ids=lambda v: "k%d_sp%d" % v)
def test_attention_graph_replays_split_and_kernels(variant):
    c = wl.small_case(31, 3, 4, 64, 512, 700, 600, 0.1)
    q, kv, sink, idx = (c[k].cuda() for k in ("q", "kv", "sink", "idx"))
    need = sa.workspace_bytes(3, 4, 64, 512, 600, variant)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    eager = sa.sparse_attn(q, kv, sink, idx, 0.05, out=out, workspace=ws, variant=variant).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sa.sparse_attn(q, kv, sink, idx, 0.05, out=out, workspace=ws, variant=variant)
    for r in range(4):
        out.fill_(3.0)
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(out, eager), f"replay {r} differs"
