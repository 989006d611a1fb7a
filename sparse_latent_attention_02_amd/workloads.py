"""Seeded synthetic inputs for the five sparse-attention workloads.

Only random draws and shapes live here -- none of the method's arithmetic (no
window selection, no fp8 rounding, no index offsetting).  Both the GPU path and
the CPU oracle take their inputs from this module and then apply their own
implementation of every method step (fp8 round trip of the KV rows, window
slot lists, concatenation with the compressed positions).

Recipe (the pages run on model caches; Gaussian data stands in for them):
  * one ``torch.Generator`` on the CPU seeded ``1000 + workload id``, drawing in
    the order q, kv, sink, index randomness;
  * q and kv: N(0, 1) in f32, rounded to bf16 (round to nearest even); kv is
    raw here, the fp8 round trip is a method step applied by each side;
  * sink: f32 N(0, 1), one per head;
  * scale = head_dim ** -0.5 (the Attention module's softmax scale);
  * compressed positions are raw (not yet shifted past the window rows, -1 where
    a slot is empty).

Workloads (sizes as the benchmark configurations give them):
  1 ring      : h=4, d=64, window 8; prefill 12 tokens, then decode positions 12
                and 13 through one ring (the rustdoc worked example's shape).
  2 decode    : b=64 single-query steps at position 5000, h=64, d=512, a full
                128-slot ring per sequence.
  3 prefill   : 4096 queries from position 0, h=64, d=512, kv = the chunk.
  4 decode+c  : b=128, h=128, d=512; ring 128 rows + 16384 compressed rows per
                sequence; 2048 distinct uniform compressed positions per query,
                sorted ascending (the indexer re-sorts into position order),
                205 (= 10 %) of them replaced by -1.
  5 prefill+c : 8192 queries, h=64, d=512, kv = 8192 chunk rows + 2048
                compressed rows; query p sees the (p + 1) // 4 compressed
                positions it has passed (all of them, since that is <= 2048), in
                random order, padded with trailing -1 to 2048.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    b: int                 # batch (sequences)
    s: int                 # queries per sequence
    h: int                 # heads
    d: int                 # latent head dim
    window: int            # ring slots
    start_pos: int         # position of the first query
    rows: int              # kv rows per sequence (window/chunk rows + compressed rows)
    win_rows: int          # rows that hold window/chunk KV (compressed rows follow)
    n_comp: int = 0        # compressed columns per query (index_topk)
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def win_cols(self) -> int:
        return min(self.s, self.window) if self.start_pos == 0 else self.window

    @property
    def topk(self) -> int:
        return self.win_cols + self.n_comp

    @property
    def scale(self) -> float:
        return self.d ** -0.5

    @property
    def query_heads(self) -> int:
        return self.b * self.s * self.h


WORKLOADS = {
    1: Workload(1, "ring: prefill 12 + decode 12, 13; h=4 d=64 window 8", 1, 12, 4, 64, 8, 0, 12, 12),
    2: Workload(2, "decode window: b=64 pos 5000, h=64 d=512, ring 128", 64, 1, 64, 512, 128, 5000, 128, 128),
    3: Workload(3, "prefill window: 4096 queries, h=64 d=512, window 128", 1, 4096, 64, 512, 128, 0, 4096, 4096),
    4: Workload(4, "decode + compressed: b=128 pos 5000, h=128 d=512, 128 + 2048 idx", 128, 1, 128, 512,
                128, 5000, 128 + 16384, 128, 2048),
    5: Workload(5, "prefill + compressed: 8192 queries, h=64 d=512, 128 + 2048 idx", 1, 8192, 64, 512,
                128, 0, 8192 + 2048, 8192, 2048),
}


def _bf16_normal(g: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def generate(wid: int, seed_offset: int = 0) -> dict:
    """Raw inputs of workload ``wid`` as CPU tensors.

    Keys: q (bf16 [b][s][h][d]), kv (bf16 [b][rows][d], before the fp8 round trip),
    sink (f32 [h]), comp (int32 [b][s][n_comp] raw compressed positions or None).
    Workload 1 instead returns the three regimes of the ring run:
    q_prefill [1][12][4][64], kv_prefill [1][12][64], q_dec [2][1][1][4][64],
    kv_dec [2][1][1][64] (the new rows at positions 12 and 13), sink [4].
    """
    w = WORKLOADS[wid]
    g = torch.Generator().manual_seed(1000 + wid + seed_offset)
    if wid == 1:
        q_prefill = _bf16_normal(g, (1, 12, w.h, w.d))
        q_dec = _bf16_normal(g, (2, 1, 1, w.h, w.d))
        kv_prefill = _bf16_normal(g, (1, 12, w.d))
        kv_dec = _bf16_normal(g, (2, 1, 1, w.d))
        sink = torch.randn(w.h, generator=g, dtype=torch.float32)
        return dict(q_prefill=q_prefill, q_dec=q_dec, kv_prefill=kv_prefill, kv_dec=kv_dec,
                    sink=sink, comp=None)
    q = _bf16_normal(g, (w.b, w.s, w.h, w.d))
    kv = _bf16_normal(g, (w.b, w.rows, w.d))
    sink = torch.randn(w.h, generator=g, dtype=torch.float32)
    comp = None
    if wid == 4:
        n_cache = w.rows - w.win_rows
        keys = torch.rand((w.b * w.s, n_cache), generator=g)
        comp = keys.argsort(dim=1)[:, : w.n_comp].sort(dim=1).values.to(torch.int32)
        holes = torch.rand((w.b * w.s, w.n_comp), generator=g).argsort(dim=1)[:, : round(0.1 * w.n_comp)]
        comp.scatter_(1, holes, -1)
        comp = comp.view(w.b, w.s, w.n_comp)
    elif wid == 5:
        n_cache = w.rows - w.win_rows
        visible = (torch.arange(w.s) + 1) // 4                      # positions passed so far
        visible = visible.clamp(max=n_cache).unsqueeze(1)
        col = torch.arange(w.n_comp).unsqueeze(0)
        keys = torch.rand((w.s, w.n_comp), generator=g)
        keys = torch.where(col < visible, keys, torch.full_like(keys, 2.0))
        perm = keys.argsort(dim=1).to(torch.int32)                  # random order of 0..visible-1 first
        comp = torch.where(col < visible, perm, torch.full_like(perm, -1)).view(1, w.s, w.n_comp)
    return dict(q=q, kv=kv, sink=sink, comp=comp)


def small_case(seed: int, b: int, s: int, h: int, d: int, rows: int, topk: int,
               p_invalid: float = 0.0, allow_dup: bool = True) -> dict:
    """A random sparse-attention case for parity sweeps: uniform indices in
    [0, rows) (with repeats when ``allow_dup``), a fraction ``p_invalid`` of them -1."""
    g = torch.Generator().manual_seed(seed)
    q = _bf16_normal(g, (b, s, h, d))
    kv = _bf16_normal(g, (b, rows, d))
    sink = torch.randn(h, generator=g, dtype=torch.float32)
    if rows > 0 and topk > 0:
        if allow_dup:
            idx = torch.randint(0, rows, (b, s, topk), generator=g, dtype=torch.int64)
        else:
            idx = torch.rand((b * s, rows), generator=g).argsort(dim=1)[:, :topk].view(b, s, topk)
        holes = torch.rand((b, s, topk), generator=g) < p_invalid
        idx = torch.where(holes, torch.full_like(idx, -1), idx)
    else:
        idx = torch.full((b, s, topk), -1, dtype=torch.int64)
    return dict(q=q, kv=kv, sink=sink, idx=idx.to(torch.int32))


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 CPU tensor's bit patterns."""
    import numpy as np
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def rope_table(seed: int, n_pos: int, rope_dim: int) -> torch.Tensor:
    """A rotation table [n_pos][rope_dim / 2][2] f32 of (cos, sin) pairs at angles
    drawn uniformly from [-pi, pi): the rotary embedding is defined for any table
    of unit complex numbers, so random angles stand in for a model's frequencies."""
    g = torch.Generator().manual_seed(seed)
    th = (torch.rand((n_pos, rope_dim // 2), generator=g, dtype=torch.float64) * 2 - 1) * torch.pi
    return torch.stack([torch.cos(th), torch.sin(th)], dim=-1).to(torch.float32).contiguous()


# The indexer selection tail's workload: the compressed half of the decode +
# compressed configuration -- 128 single-query sequences whose indexer scores
# 16384 compressed positions (start_pos 65535, ratio 4) and keeps 2048 of them,
# placed after the 128 window columns.  Scores are N(0, 1) f32 (the pages'
# scores come from trained weights).
SELECT_WORKLOAD = dict(b=128, s=1, start_pos=65535, ratio=4, index_topk=2048, offset=128)


def indexer_scores(seed: int, b: int, s: int, n_cols: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randn((b, s, n_cols), generator=g, dtype=torch.float32)
