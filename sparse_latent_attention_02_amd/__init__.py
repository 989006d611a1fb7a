"""MI355X (gfx950) sparse latent attention -- Python binding of libsparse_attn.so.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/sparse_attn.h``.  PyTorch supplies device memory and the
current stream.  There is no CPU fallback: if the library is missing or the
tensors are not on a GPU, the calls raise.

Names follow the C ABI:
  window_topk_idxs / window_topk_idxs_shape -- window slot lists
  append_compressed_idxs                   -- compressed positions after the window
  act_quant_fp8_                           -- fp8 (e4m3) round trip of bf16 rows, in place
  window_kv_update                         -- fp8 round trip of new rows + ring-cache write
  sparse_attn                              -- the attention itself
  sparse_attn_noalloc                      -- the same with no workspace argument, allocating nothing
  sparse_attn_decode_step                  -- a whole decode step (ring write, lists, attention) in one launch
  kv8_pack / kv8_unpack                    -- fp8-resident KV rows (e4m3fn codes + E8M0 block scales)
  sparse_attn_kv8 / sparse_attn_decode_step_kv8 -- the attention and the decode step over kv8 rows
  apply_rotary                             -- rotary embedding of the last rope_dim values (or its inverse)
  rope= on sparse_attn / sparse_attn_decode_step -- the output's inverse rotation fused into the epilogue
  indexer_topk                             -- the indexer's selection tail (compressed positions of the list)
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime this library then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_attn.so")
_lib = None

SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_UNSUPPORTED, SA_ERR_HIP = 0, 1, 2, 3, 4
SA_KERNEL_AUTO, SA_KERNEL_WIDE, SA_KERNEL_DECODE, SA_KERNEL_PAIR = 0, 1, 2, 3
KV8_SCALE_BYTES = 16


class SparseAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        name = lib().sa_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn}: {name}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_latent_attention_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, f32, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        L.sa_status_string.argtypes = [ctypes.c_int]
        L.sa_status_string.restype = ctypes.c_char_p
        L.sa_window_topk_idxs_shape.argtypes = [i32, i32, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.sa_window_topk_idxs.argtypes = [i32, i32, i32, i64, vp, i64, vp]
        L.sa_append_compressed_idxs.argtypes = [vp, i64, i32, vp, i64, i32, i32, vp]
        L.sa_act_quant_fp8_inplace.argtypes = [vp, i64, i32, vp]
        L.sa_window_kv_update.argtypes = [vp, i64, vp, i32, i32, i32, i64, i32, vp]
        L.sa_sparse_attn_workspace_bytes.argtypes = [i64, i64, i32, i32, i32]
        L.sa_sparse_attn_workspace_bytes.restype = sz
        L.sa_sparse_attn_workspace_bytes_ex.argtypes = [i64, i64, i32, i32, i32, i32, i32]
        L.sa_sparse_attn_workspace_bytes_ex.restype = sz
        L.sa_sparse_attn.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i64, i32, f32, vp, vp, sz, vp]
        L.sa_sparse_attn_ex.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i64, i32, f32, vp, vp, sz, vp,
                                        i32, i32]
        L.sa_kv8_pack.argtypes = [vp, vp, vp, i64, i32, vp]
        L.sa_kv8_unpack.argtypes = [vp, vp, vp, i64, i32, vp]
        L.sa_sparse_attn_decode_step_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32, i32]
        L.sa_sparse_attn_decode_step_workspace_bytes.restype = sz
        L.sa_sparse_attn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i64, i32, i32, i64, f32,
                                                 vp, vp, sz, vp, i32, i32]
        L.sa_sparse_attn_kv8_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
        L.sa_sparse_attn_kv8_workspace_bytes.restype = sz
        L.sa_sparse_attn_kv8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i64, i32, f32, vp, vp, sz, vp,
                                         i32]
        L.sa_sparse_attn_decode_step_kv8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i64, i32, i32,
                                                     i64, f32, vp, vp, sz, vp, i32]
        L.sa_apply_rotary.argtypes = [vp, i64, i64, i32, i32, i32, vp, i64, i64, i32, vp]
        L.sa_sparse_attn_rope.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i64, i32, f32, vp, vp, sz, vp,
                                          i32, i32, vp, i64, i32, i64]
        L.sa_sparse_attn_decode_step_rope.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i64, i32, i32, i64,
                                                      f32, vp, vp, sz, vp, i32, i32, vp, i64, i32]
        L.sa_indexer_topk.argtypes = [vp, i64, i64, i32, i64, i32, i32, i32, vp, i64, i32, vp]
        L.sa_sparse_attn_noalloc_scratch_bytes.argtypes = []
        L.sa_sparse_attn_noalloc_scratch_bytes.restype = sz
        L.sa_sparse_attn_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i64, i32, f32, vp, vp, i32, i32]
        L.sa_sparse_attn_prefill_step_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32, i32, i32]
        L.sa_sparse_attn_prefill_step_workspace_bytes.restype = sz
        L.sa_sparse_attn_prefill_step.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i64, i32, i32, f32, vp,
                                                  vp, sz, vp, i32, i32]
        L.sa_sparse_attn_prefill_step_rope.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i64, i32, i32, f32,
                                                       vp, vp, sz, vp, i32, i32, vp, i64, i32]
        for fn in ("sa_window_topk_idxs_shape", "sa_window_topk_idxs", "sa_append_compressed_idxs",
                   "sa_act_quant_fp8_inplace", "sa_window_kv_update", "sa_sparse_attn", "sa_sparse_attn_ex",
                   "sa_sparse_attn_decode_step", "sa_kv8_pack", "sa_kv8_unpack", "sa_sparse_attn_kv8",
                   "sa_sparse_attn_decode_step_kv8", "sa_apply_rotary", "sa_sparse_attn_rope",
                   "sa_sparse_attn_decode_step_rope", "sa_indexer_topk", "sa_sparse_attn_noalloc",
                   "sa_sparse_attn_prefill_step", "sa_sparse_attn_prefill_step_rope"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != SA_OK:
        raise SparseAttnError(fn, status)


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def window_topk_idxs_shape(window: int, seqlen: int, start_pos: int) -> tuple[int, int]:
    r, c = ctypes.c_int32(), ctypes.c_int32()
    _check("sa_window_topk_idxs_shape",
           lib().sa_window_topk_idxs_shape(window, seqlen, start_pos, ctypes.byref(r), ctypes.byref(c)))
    return r.value, c.value


def window_topk_idxs(window: int, bsz: int, seqlen: int, start_pos: int, out: torch.Tensor | None = None,
                     device=None, stream=None) -> torch.Tensor:
    """int32 [bsz][rows][cols] window slot lists (-1 = empty slot).  With ``out``
    ([bsz][rows][stride], stride >= cols) the lists fill its leading columns."""
    rows, cols = window_topk_idxs_shape(window, seqlen, start_pos)
    if out is None:
        out = torch.empty((bsz, rows, cols), dtype=torch.int32, device=device or "cuda")
    _dev(out, "out", torch.int32)
    if out.dim() != 3 or out.shape[0] != bsz or out.shape[1] != rows:
        raise ValueError(f"out must be [{bsz}][{rows}][>= {cols}], got {tuple(out.shape)}")
    _check("sa_window_topk_idxs",
           lib().sa_window_topk_idxs(window, bsz, seqlen, start_pos, out.data_ptr(), out.shape[-1],
                                     _stream(stream)))
    return out


def append_compressed_idxs(idx: torch.Tensor, col0: int, cidx: torch.Tensor, offset: int, stream=None) -> None:
    """idx[..., col0 + j] = cidx[..., j] + offset (or -1 where cidx < 0), in place."""
    _dev(idx, "idx", torch.int32)
    _dev(cidx, "cidx", torch.int32)
    kc = cidx.shape[-1]
    n_rows = cidx.numel() // kc if kc else 0
    if idx.numel() // idx.shape[-1] != n_rows and kc:
        raise ValueError("idx and cidx have different row counts")
    _check("sa_append_compressed_idxs",
           lib().sa_append_compressed_idxs(idx.data_ptr(), idx.shape[-1], col0, cidx.data_ptr(), n_rows, kc,
                                           offset, _stream(stream)))


def act_quant_fp8_(x: torch.Tensor, stream=None) -> torch.Tensor:
    """fp8 e4m3 round trip (block 32, power-of-two scale) of bf16 rows, in place."""
    _dev(x, "x", torch.bfloat16)
    row_len = x.shape[-1]
    n_rows = x.numel() // row_len if row_len else 0
    _check("sa_act_quant_fp8_inplace",
           lib().sa_act_quant_fp8_inplace(x.data_ptr(), n_rows, row_len, _stream(stream)))
    return x


def window_kv_update(ring: torch.Tensor, rows: torch.Tensor, start_pos: int, window: int | None = None,
                     stream=None) -> None:
    """Rounds the new rows [bsz][seqlen][d] through fp8 in place and writes the
    surviving ones into the ring at slot position % window.  ``ring`` is
    [bsz][stride][d]; its first ``window`` rows per batch element (default: all
    of them) form the ring."""
    _dev(ring, "ring", torch.bfloat16)
    _dev(rows, "rows", torch.bfloat16)
    bsz, stride, d = ring.shape
    window = stride if window is None else window
    if rows.dim() != 3 or rows.shape[0] != bsz or rows.shape[2] != d:
        raise ValueError(f"rows must be [{bsz}][seqlen][{d}], got {tuple(rows.shape)}")
    _check("sa_window_kv_update",
           lib().sa_window_kv_update(ring.data_ptr(), stride, rows.data_ptr(), bsz, window, d, start_pos,
                                     rows.shape[1], _stream(stream)))


def workspace_bytes(b: int, s: int, h: int, d: int, topk: int, variant: tuple | None = None) -> int:
    if variant is None:
        return int(lib().sa_sparse_attn_workspace_bytes(b, s, h, d, topk))
    return int(lib().sa_sparse_attn_workspace_bytes_ex(b, s, h, d, topk, *variant))


def sparse_attn(q: torch.Tensor, kv: torch.Tensor, sink: torch.Tensor, idx: torch.Tensor, scale: float,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                variant: tuple | None = None, stream=None, rope: tuple | None = None) -> torch.Tensor:
    """q [b][s][h][d] bf16, kv [b][rows][d] bf16, sink [h] f32, idx [b][s][topk] int32 -> [b][s][h][d] bf16.

    ``variant`` = (kernel, splits) forces a kernel variant (see sa_kernel; 0 = automatic).
    ``rope`` = (table [n_pos][rope_dim/2][2] f32, rope_dim, start_pos) un-rotates the
    output's last rope_dim values in the epilogue (query s at position start_pos + s)."""
    _dev(q, "q", torch.bfloat16)
    _dev(kv, "kv", torch.bfloat16)
    _dev(sink, "sink", torch.float32)
    _dev(idx, "idx", torch.int32)
    b, s, h, d = q.shape
    if kv.dim() != 3 or kv.shape[0] != b or kv.shape[2] != d:
        raise ValueError(f"kv must be [{b}][rows][{d}], got {tuple(kv.shape)}")
    if idx.dim() != 3 or idx.shape[0] != b or idx.shape[1] != s:
        raise ValueError(f"idx must be [{b}][{s}][topk], got {tuple(idx.shape)}")
    if sink.shape != (h,):
        raise ValueError(f"sink must be [{h}]")
    rows, topk = kv.shape[1], idx.shape[2]
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", torch.bfloat16)
    need = workspace_bytes(b, s, h, d, topk, variant)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (q.data_ptr(), kv.data_ptr(), sink.data_ptr(), idx.data_ptr(), b, s, h, d, rows, topk, float(scale),
            out.data_ptr(), ws_ptr, ws_bytes, _stream(stream))
    if rope is not None:
        table, rope_dim, start_pos = rope
        _dev(table, "rope table", torch.float32)
        k, sp = variant if variant is not None else (0, 0)
        _check("sa_sparse_attn_rope", lib().sa_sparse_attn_rope(*args, k, sp, table.data_ptr(), table.shape[0],
                                                                 rope_dim, start_pos))
        return out
    if variant is None:
        _check("sa_sparse_attn", lib().sa_sparse_attn(*args))
    else:
        _check("sa_sparse_attn_ex", lib().sa_sparse_attn_ex(*args, *variant))
    return out


def noalloc_scratch_bytes() -> int:
    """Size of the library's own per-device scratch used by sparse_attn_noalloc."""
    return int(lib().sa_sparse_attn_noalloc_scratch_bytes())


def sparse_attn_noalloc(q: torch.Tensor, kv: torch.Tensor, sink: torch.Tensor, idx: torch.Tensor, scale: float,
                        out: torch.Tensor, variant: tuple | None = None, stream=None) -> torch.Tensor:
    """sparse_attn with no workspace argument: the library allocates nothing and
    keeps split partials in its own per-device scratch (sa_sparse_attn_noalloc).
    ``out`` is required (the call allocates nothing).  Calls whose work overlaps
    on one device race on the scratch."""
    _dev(q, "q", torch.bfloat16)
    _dev(kv, "kv", torch.bfloat16)
    _dev(sink, "sink", torch.float32)
    _dev(idx, "idx", torch.int32)
    _dev(out, "out", torch.bfloat16)
    b, s, h, d = q.shape
    if kv.dim() != 3 or kv.shape[0] != b or kv.shape[2] != d:
        raise ValueError(f"kv must be [{b}][rows][{d}], got {tuple(kv.shape)}")
    if idx.dim() != 3 or idx.shape[0] != b or idx.shape[1] != s:
        raise ValueError(f"idx must be [{b}][{s}][topk], got {tuple(idx.shape)}")
    if sink.shape != (h,) or out.shape != q.shape:
        raise ValueError("sink must be [h] and out shaped like q")
    k, sp = variant if variant is not None else (0, 0)
    _check("sa_sparse_attn_noalloc",
           lib().sa_sparse_attn_noalloc(q.data_ptr(), kv.data_ptr(), sink.data_ptr(), idx.data_ptr(), b, s, h, d,
                                        kv.shape[1], idx.shape[2], float(scale), out.data_ptr(), _stream(stream),
                                        k, sp))
    return out


def decode_step_workspace_bytes(b: int, h: int, d: int, window: int, kc: int, variant: tuple | None = None) -> int:
    k, sp = variant if variant is not None else (0, 0)
    return int(lib().sa_sparse_attn_decode_step_workspace_bytes(b, h, d, window, kc, k, sp))


def sparse_attn_decode_step(q: torch.Tensor, kv: torch.Tensor, kv_new: torch.Tensor, sink: torch.Tensor,
                            window: int, start_pos: int, scale: float, cidx: torch.Tensor | None = None,
                            out: torch.Tensor | None = None, idx_out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, variant: tuple | None = None,
                            stream=None, rope: tuple | None = None) -> torch.Tensor:
    """One decode step in one launch: kv_new [b][d] rounded through fp8 into ring slot
    start_pos % window of kv [b][rows][d] (rows [0, window) = ring, compressed rows
    after), the window list + cidx [b][kc] (+window) as the index list, sparse
    attention of q [b][h][d] (or [b][1][h][d]).  kv_new is not modified.  ``idx_out``
    ([b][window + kc] int32) receives the list when given.  ``rope`` = (table,
    rope_dim) un-rotates the output's last rope_dim values at position start_pos."""
    _dev(q, "q", torch.bfloat16)
    _dev(kv, "kv", torch.bfloat16)
    _dev(kv_new, "kv_new", torch.bfloat16)
    _dev(sink, "sink", torch.float32)
    b, rows, d = kv.shape
    h = q.shape[-2]
    if q.numel() != b * h * d or q.shape[0] != b or q.shape[-1] != d:
        raise ValueError(f"q must be [{b}][{h}][{d}] (or [{b}][1][{h}][{d}]), got {tuple(q.shape)}")
    if kv_new.numel() != b * d or kv_new.shape[0] != b:
        raise ValueError(f"kv_new must be [{b}][{d}], got {tuple(kv_new.shape)}")
    if sink.shape != (h,):
        raise ValueError(f"sink must be [{h}]")
    kc = 0
    if cidx is not None:
        _dev(cidx, "cidx", torch.int32)
        kc = cidx.shape[-1]
        if cidx.numel() != b * kc:
            raise ValueError(f"cidx must be [{b}][kc], got {tuple(cidx.shape)}")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", torch.bfloat16)
    if idx_out is not None:
        _dev(idx_out, "idx_out", torch.int32)
        if idx_out.numel() != b * (window + kc):
            raise ValueError(f"idx_out must hold [{b}][{window + kc}]")
    k, sp = variant if variant is not None else (0, 0)
    need = decode_step_workspace_bytes(b, h, d, window, kc, variant)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (q.data_ptr(), kv.data_ptr(), kv_new.data_ptr(), sink.data_ptr(),
            cidx.data_ptr() if cidx is not None else None, idx_out.data_ptr() if idx_out is not None else None,
            b, h, d, rows, window, kc, start_pos, float(scale), out.data_ptr(), ws_ptr, ws_bytes, _stream(stream),
            k, sp)
    if rope is not None:
        table, rope_dim = rope
        _dev(table, "rope table", torch.float32)
        _check("sa_sparse_attn_decode_step_rope",
               lib().sa_sparse_attn_decode_step_rope(*args, table.data_ptr(), table.shape[0], rope_dim))
        return out
    _check("sa_sparse_attn_decode_step", lib().sa_sparse_attn_decode_step(*args))
    return out


def prefill_step_workspace_bytes(b: int, s: int, h: int, d: int, window: int, kc: int,
                                 variant: tuple | None = None) -> int:
    k, sp = variant if variant is not None else (0, 0)
    return int(lib().sa_sparse_attn_prefill_step_workspace_bytes(b, s, h, d, window, kc, k, sp))


def sparse_attn_prefill_step(q: torch.Tensor, kv: torch.Tensor, sink: torch.Tensor, window: int, scale: float,
                             cidx: torch.Tensor | None = None, out: torch.Tensor | None = None,
                             idx_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                             variant: tuple | None = None, stream=None, rope: tuple | None = None) -> torch.Tensor:
    """Prefill attention with the index list built in the kernel: q [b][s][h][d] at
    positions 0 .. s-1, kv [b][rows][d] (rows [0, s) the chunk, already through its
    fp8 round trip; compressed rows after), the window list (min(s, window)
    columns) + cidx [b][s][kc] (+s) as the index list, built by the pair kernel
    (``variant`` may only name it).  ``idx_out`` ([b][s][min(s, window) + kc]
    int32) receives the list when given.  ``rope`` = (table, rope_dim) un-rotates
    the output's last rope_dim values at each query's position."""
    _dev(q, "q", torch.bfloat16)
    _dev(kv, "kv", torch.bfloat16)
    _dev(sink, "sink", torch.float32)
    b, rows, d = kv.shape
    if q.dim() != 4 or q.shape[0] != b or q.shape[-1] != d:
        raise ValueError(f"q must be [{b}][s][h][{d}], got {tuple(q.shape)}")
    s, h = q.shape[1], q.shape[2]
    if sink.shape != (h,):
        raise ValueError(f"sink must be [{h}]")
    kc = 0
    if cidx is not None:
        _dev(cidx, "cidx", torch.int32)
        kc = cidx.shape[-1]
        if cidx.numel() != b * s * kc:
            raise ValueError(f"cidx must be [{b}][{s}][kc], got {tuple(cidx.shape)}")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", torch.bfloat16)
    if idx_out is not None:
        _dev(idx_out, "idx_out", torch.int32)
        if idx_out.numel() != b * s * (min(s, window) + kc):
            raise ValueError(f"idx_out must hold [{b}][{s}][{min(s, window) + kc}]")
    k, sp = variant if variant is not None else (0, 0)
    need = prefill_step_workspace_bytes(b, s, h, d, window, kc, variant)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (q.data_ptr(), kv.data_ptr(), sink.data_ptr(), cidx.data_ptr() if cidx is not None else None,
            idx_out.data_ptr() if idx_out is not None else None, b, s, h, d, rows, window, kc, float(scale),
            out.data_ptr(), ws_ptr, ws_bytes, _stream(stream), k, sp)
    if rope is not None:
        table, rope_dim = rope
        _dev(table, "rope table", torch.float32)
        _check("sa_sparse_attn_prefill_step_rope",
               lib().sa_sparse_attn_prefill_step_rope(*args, table.data_ptr(), table.shape[0], rope_dim))
        return out
    _check("sa_sparse_attn_prefill_step", lib().sa_sparse_attn_prefill_step(*args))
    return out


def kv8_pack(x: torch.Tensor, codes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
             stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16 rows [..., row_len] -> (uint8 codes [..., row_len], uint8 scales [..., 16])."""
    _dev(x, "x", torch.bfloat16)
    row_len = x.shape[-1]
    n_rows = x.numel() // row_len if row_len else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (KV8_SCALE_BYTES,), dtype=torch.uint8, device=x.device)
    _dev(codes, "codes", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    if codes.numel() != x.numel() or scales.numel() != n_rows * KV8_SCALE_BYTES:
        raise ValueError("codes must match x; scales must be [rows][16]")
    _check("sa_kv8_pack", lib().sa_kv8_pack(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), n_rows, row_len,
                                            _stream(stream)))
    return codes, scales


def kv8_unpack(codes: torch.Tensor, scales: torch.Tensor, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    _dev(codes, "codes", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    row_len = codes.shape[-1]
    n_rows = codes.numel() // row_len if row_len else 0
    if scales.numel() != n_rows * KV8_SCALE_BYTES:
        raise ValueError("scales must be [rows][16]")
    if out is None:
        out = torch.empty(codes.shape, dtype=torch.bfloat16, device=codes.device)
    _dev(out, "out", torch.bfloat16)
    _check("sa_kv8_unpack", lib().sa_kv8_unpack(codes.data_ptr(), scales.data_ptr(), out.data_ptr(), n_rows,
                                                row_len, _stream(stream)))
    return out



def kv8_workspace_bytes(b: int, s: int, h: int, d: int, topk: int, splits: int = 0) -> int:
    return int(lib().sa_sparse_attn_kv8_workspace_bytes(b, s, h, d, topk, splits))


def _kv8_rows(codes: torch.Tensor, scales: torch.Tensor) -> tuple[int, int, int]:
    _dev(codes, "kv_codes", torch.uint8)
    _dev(scales, "kv_scales", torch.uint8)
    if codes.dim() != 3 or scales.shape != codes.shape[:2] + (KV8_SCALE_BYTES,):
        raise ValueError(f"kv_codes must be [b][rows][d] and kv_scales [b][rows][{KV8_SCALE_BYTES}], "
                         f"got {tuple(codes.shape)} and {tuple(scales.shape)}")
    return tuple(codes.shape)


def _workspace(need: int, workspace: torch.Tensor | None, device) -> tuple:
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def sparse_attn_kv8(q: torch.Tensor, kv_codes: torch.Tensor, kv_scales: torch.Tensor, sink: torch.Tensor,
                    idx: torch.Tensor, scale: float, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, splits: int = 0, stream=None) -> torch.Tensor:
    """sparse_attn over kv8 rows: kv_codes [b][rows][d] uint8, kv_scales [b][rows][16] uint8."""
    _dev(q, "q", torch.bfloat16)
    _dev(sink, "sink", torch.float32)
    _dev(idx, "idx", torch.int32)
    b, s, h, d = q.shape
    kb, rows, kd = _kv8_rows(kv_codes, kv_scales)
    if kb != b or kd != d:
        raise ValueError(f"kv_codes must be [{b}][rows][{d}], got {tuple(kv_codes.shape)}")
    if idx.dim() != 3 or idx.shape[0] != b or idx.shape[1] != s:
        raise ValueError(f"idx must be [{b}][{s}][topk], got {tuple(idx.shape)}")
    if sink.shape != (h,):
        raise ValueError(f"sink must be [{h}]")
    topk = idx.shape[2]
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", torch.bfloat16)
    ws_ptr, ws_bytes = _workspace(kv8_workspace_bytes(b, s, h, d, topk, splits), workspace, q.device)
    _check("sa_sparse_attn_kv8",
           lib().sa_sparse_attn_kv8(q.data_ptr(), kv_codes.data_ptr(), kv_scales.data_ptr(), sink.data_ptr(),
                                    idx.data_ptr(), b, s, h, d, rows, topk, float(scale), out.data_ptr(), ws_ptr,
                                    ws_bytes, _stream(stream), splits))
    return out


def sparse_attn_decode_step_kv8(q: torch.Tensor, kv_codes: torch.Tensor, kv_scales: torch.Tensor,
                                kv_new: torch.Tensor, sink: torch.Tensor, window: int, start_pos: int,
                                scale: float, cidx: torch.Tensor | None = None, out: torch.Tensor | None = None,
                                idx_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                splits: int = 0, stream=None) -> torch.Tensor:
    """sparse_attn_decode_step over kv8 rows; the new row's codes and scale record
    go to ring slot start_pos % window of kv_codes / kv_scales."""
    _dev(q, "q", torch.bfloat16)
    _dev(kv_new, "kv_new", torch.bfloat16)
    _dev(sink, "sink", torch.float32)
    b, rows, d = _kv8_rows(kv_codes, kv_scales)
    h = q.shape[-2]
    if q.numel() != b * h * d or q.shape[0] != b or q.shape[-1] != d:
        raise ValueError(f"q must be [{b}][{h}][{d}] (or [{b}][1][{h}][{d}]), got {tuple(q.shape)}")
    if kv_new.numel() != b * d or kv_new.shape[0] != b:
        raise ValueError(f"kv_new must be [{b}][{d}], got {tuple(kv_new.shape)}")
    if sink.shape != (h,):
        raise ValueError(f"sink must be [{h}]")
    kc = 0
    if cidx is not None:
        _dev(cidx, "cidx", torch.int32)
        kc = cidx.shape[-1]
        if cidx.numel() != b * kc:
            raise ValueError(f"cidx must be [{b}][kc], got {tuple(cidx.shape)}")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", torch.bfloat16)
    if idx_out is not None:
        _dev(idx_out, "idx_out", torch.int32)
        if idx_out.numel() != b * (window + kc):
            raise ValueError(f"idx_out must hold [{b}][{window + kc}]")
    ws_ptr, ws_bytes = _workspace(kv8_workspace_bytes(b, 1, h, d, window + kc, splits), workspace, q.device)
    _check("sa_sparse_attn_decode_step_kv8",
           lib().sa_sparse_attn_decode_step_kv8(q.data_ptr(), kv_codes.data_ptr(), kv_scales.data_ptr(),
                                                kv_new.data_ptr(), sink.data_ptr(),
                                                cidx.data_ptr() if cidx is not None else None,
                                                idx_out.data_ptr() if idx_out is not None else None,
                                                b, h, d, rows, window, kc, start_pos, float(scale),
                                                out.data_ptr(), ws_ptr, ws_bytes, _stream(stream), splits))
    return out


def apply_rotary(x: torch.Tensor, table: torch.Tensor, rope_dim: int, start_pos: int = 0, inverse: bool = False,
                 stream=None) -> torch.Tensor:
    """Rotary embedding of the last ``rope_dim`` values of x [b][s][h][row_len] (or
    [b][s][row_len]) bf16, in place; row (b, s, .) at position start_pos + s,
    table [n_pos][rope_dim / 2][2] f32 (cos, sin)."""
    _dev(x, "x", torch.bfloat16)
    _dev(table, "table", torch.float32)
    if x.dim() not in (3, 4):
        raise ValueError("x must be [b][s][h][row_len] or [b][s][row_len]")
    b, s = x.shape[0], x.shape[1]
    h = x.shape[2] if x.dim() == 4 else 1
    _check("sa_apply_rotary", lib().sa_apply_rotary(x.data_ptr(), b, s, h, x.shape[-1], rope_dim, table.data_ptr(),
                                                    table.shape[0], start_pos, int(bool(inverse)), _stream(stream)))
    return x


def indexer_topk(scores: torch.Tensor, start_pos: int, ratio: int, index_topk: int, offset: int,
                 out: torch.Tensor | None = None, col0: int = 0, stream=None) -> torch.Tensor:
    """Indexer selection tail: scores [b][s][T] f32 (T = (start_pos + s) // ratio) ->
    int32 [b][s][min(index_topk, T)] positions + offset in position order, -1 where
    unreachable.  With ``out`` ([b][s][cols] int32) the selection is written into
    columns [col0, col0 + topk) of it (e.g. after the window columns)."""
    _dev(scores, "scores", torch.float32)
    b, s, T = scores.shape
    topk = min(index_topk, T)
    if out is None:
        out = torch.empty((b, s, topk), dtype=torch.int32, device=scores.device)
        col0 = 0
    _dev(out, "out", torch.int32)
    if out.dim() != 3 or out.shape[0] != b or out.shape[1] != s:
        raise ValueError(f"out must be [{b}][{s}][cols]")
    _check("sa_indexer_topk", lib().sa_indexer_topk(scores.data_ptr(), b, s, T, start_pos, ratio, index_topk,
                                                    offset, out.data_ptr(), out.shape[2], col0, _stream(stream)))
    return out
