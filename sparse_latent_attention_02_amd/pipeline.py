"""One step of the sparse-attention hot path on the GPU, for the five workloads.

A step is what one layer does per forward call on its attention inputs:
  1. new KV rows are rounded through fp8 in place and written into the
     sliding-window ring (sa_window_kv_update);
  2. the window slot lists are built (sa_window_topk_idxs), straight into the
     leading columns of the index buffer;
  3. compressed positions, when the workload has them, are appended after the
     window columns, shifted past the window rows (sa_append_compressed_idxs);
  4. sparse attention over the selected rows (sa_sparse_attn).
Everything runs through the C ABI on the current stream; torch only allocates.
A decode step can also run as one launch (``step_fused``): the same four steps
inside the attention kernel.  With ``kv8`` the cache is held fp8-resident
(e4m3fn codes + E8M0 block scales, sa_kv8_pack) and the one-launch step reads
and writes it in that form (``step_fused_kv8``); the results are bitwise those
of the bf16 cache.

KV rows that exist before the step -- the ring contents at a decode step and
the compressed cache -- are rounded through fp8 once in ``prepare``, as the cache
holds them after earlier steps.
"""
from __future__ import annotations

from types import SimpleNamespace

import torch

from . import sparse_attn, window_kv_update, window_topk_idxs, append_compressed_idxs, act_quant_fp8_
from . import workspace_bytes, sparse_attn_decode_step, decode_step_workspace_bytes
from . import sparse_attn_prefill_step, prefill_step_workspace_bytes
from . import kv8_pack, kv8_workspace_bytes, sparse_attn_decode_step_kv8
from .workloads import WORKLOADS, rope_table

ROPE_DIM = 64  # the rotated part of each latent row (the model's rope head dim)


def prepare(wid: int, raw: dict, device: str = "cuda", kv8: bool = False, rope_dim: int = 0) -> SimpleNamespace:
    w = WORKLOADS[wid]
    st = SimpleNamespace(w=w, wid=wid, kv8=kv8, rope=None)
    if rope_dim:
        # one table row per position the step's queries sit at
        st.rope = (rope_table(2000 + wid, w.start_pos + w.s, rope_dim).to(device), rope_dim)
    if kv8 and w.start_pos == 0:
        raise ValueError("the fp8-resident cache is read by the decode step only")
    st.sink = raw["sink"].to(device)
    if wid == 1:
        st.q_prefill = raw["q_prefill"].to(device)
        st.q_dec = raw["q_dec"].to(device)
        st.kv_prefill_raw = raw["kv_prefill"].to(device)
        st.kv_dec_raw = raw["kv_dec"].to(device)
        return st
    st.q = raw["q"].to(device)
    st.kv = raw["kv"].to(device)
    st.out = torch.empty_like(st.q)
    st.idx = torch.empty((w.b, w.s, w.topk), dtype=torch.int32, device=device)
    st.comp = raw["comp"].to(device) if raw["comp"] is not None else None
    if w.start_pos > 0:
        act_quant_fp8_(st.kv)                              # ring + compressed cache before the step
        slot = w.start_pos % w.window
        st.new_rows = raw["kv"][:, slot:slot + 1].contiguous().to(device)  # this step's token, raw
    else:
        if w.rows > w.win_rows:
            for bi in range(w.b):                          # compressed cache (produced upstream)
                act_quant_fp8_(st.kv[bi, w.win_rows:])
        st.chunk = st.kv[:, : w.win_rows] if w.b == 1 else None
        assert st.chunk is not None and st.chunk.is_contiguous()
        st.ring = torch.zeros((w.b, w.window, w.d), dtype=torch.bfloat16, device=device)
    nws = workspace_bytes(w.b, w.s, w.h, w.d, w.topk)
    if w.start_pos > 0:
        nws = max(nws, decode_step_workspace_bytes(w.b, w.h, w.d, w.window, w.n_comp))
    else:
        nws = max(nws, prefill_step_workspace_bytes(w.b, w.s, w.h, w.d, w.window, w.n_comp))
    if kv8:
        st.kc, st.ks = kv8_pack(st.kv)                     # the cache held as codes + scale records
        st.kv = None
        nws = max(nws, kv8_workspace_bytes(w.b, 1, w.h, w.d, w.topk))
    st.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=device)
    return st


def build_index(st: SimpleNamespace) -> None:
    """Steps 2-3: the index list into ``st.idx``."""
    w = st.w
    window_topk_idxs(w.window, w.b, w.s, w.start_pos, out=st.idx)
    if st.comp is not None:
        append_compressed_idxs(st.idx, w.win_cols, st.comp, w.win_rows)


def update_and_index(st: SimpleNamespace) -> None:
    """Steps 1-3: ring update (with the fp8 round trip) and the index list."""
    w = st.w
    if w.start_pos > 0:
        window_kv_update(st.kv, st.new_rows, w.start_pos, window=w.window)
    else:
        window_kv_update(st.ring, st.chunk, 0)
    build_index(st)


def attend(st: SimpleNamespace) -> torch.Tensor:
    """Step 4."""
    w = st.w
    rope = (st.rope[0], st.rope[1], w.start_pos) if st.rope else None
    return sparse_attn(st.q, st.kv, st.sink, st.idx, w.scale, out=st.out, workspace=st.ws, rope=rope)


def step(st: SimpleNamespace) -> torch.Tensor:
    update_and_index(st)
    return attend(st)


def ring_run(st: SimpleNamespace) -> dict:
    """Workload 1: prefill of 12 tokens, then decode positions 12 and 13, through one
    8-slot ring.  Returns the outputs and the ring after each decode step."""
    w = st.w
    dev = st.sink.device
    ring = torch.zeros((1, w.window, w.d), dtype=torch.bfloat16, device=dev)
    chunk = st.kv_prefill_raw.clone()
    window_kv_update(ring, chunk, 0)                      # chunk rounded in place, last 8 into the ring
    res = {"ring_after_prefill": ring.clone()}
    idx = window_topk_idxs(w.window, 1, w.s, 0, device=dev)
    res["prefill"] = sparse_attn(st.q_prefill, chunk, st.sink, idx, w.scale)
    for i, pos in enumerate((12, 13)):
        row = st.kv_dec_raw[i].clone()                     # [1][1][d]
        window_kv_update(ring, row, pos)
        idx = window_topk_idxs(w.window, 1, 1, pos, device=dev)
        res[f"decode{pos}"] = sparse_attn(st.q_dec[i], ring, st.sink, idx, w.scale)
        res[f"ring{pos}"] = ring.clone()
    return res


def step_fused(st: SimpleNamespace) -> torch.Tensor:
    """Steps 1-4 of a decode step in one launch (sa_sparse_attn_decode_step): the
    new row is rounded and written into the ring, the list is built inside the
    kernel and also written to ``st.idx``."""
    w = st.w
    assert w.start_pos > 0, "the fused step is a decode step"
    return sparse_attn_decode_step(st.q, st.kv, st.new_rows.view(w.b, w.d), st.sink, w.window, w.start_pos,
                                   w.scale, cidx=st.comp.view(w.b, w.n_comp) if st.comp is not None else None,
                                   out=st.out, idx_out=st.idx, workspace=st.ws, rope=st.rope)


def attend_fused_prefill(st: SimpleNamespace) -> torch.Tensor:
    """Step 4 of a prefill with steps 2-3 inside it (sa_sparse_attn_prefill_step):
    the window list and the compressed append are built in the attention kernel."""
    w = st.w
    assert w.start_pos == 0, "the prefill list starts at position 0"
    return sparse_attn_prefill_step(st.q, st.kv, st.sink, w.window, w.scale, cidx=st.comp, out=st.out,
                                    workspace=st.ws, rope=st.rope)


def step_fused_prefill(st: SimpleNamespace) -> torch.Tensor:
    """A prefill step in two launches: the chunk's fp8 round trip (and its last rows
    into the ring), then the attention with the list built inside it."""
    window_kv_update(st.ring, st.chunk, 0)
    return attend_fused_prefill(st)


def step_fused_kv8(st: SimpleNamespace) -> torch.Tensor:
    """step_fused on the fp8-resident cache (sa_sparse_attn_decode_step_kv8): the
    new row's codes and scale record go into its ring slot."""
    w = st.w
    return sparse_attn_decode_step_kv8(st.q, st.kc, st.ks, st.new_rows.view(w.b, w.d), st.sink, w.window,
                                       w.start_pos, w.scale,
                                       cidx=st.comp.view(w.b, w.n_comp) if st.comp is not None else None,
                                       out=st.out, idx_out=st.idx, workspace=st.ws)
