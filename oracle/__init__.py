"""CPU oracle for sparse latent attention -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper around ``libsa_oracle.so`` (plain C, ``sa_oracle.c``).
Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline leg may import this package; the GPU library and its Python binding
never do.  Every array is a numpy array on the host; bf16 tensors travel as
``uint16`` bit patterns.

Each function follows the page passage cited in ``sa_oracle.c``:
window selection and the sparse_attn kernel from "DeepSeek V4.1 ... attention /
attend"; the index concatenation from "... attention / query-latent"
(Attention.forward, Indexer tail) and the rotary embedding (apply_rotary_emb);
and the Indexer's selection tail; the ring write, fp8 round trip, pow2_ceil and
apply_rotary contract from the "Module attn" rustdoc page.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsa_oracle.so")
_lib = None

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_INDEX = 0, 1, 2, 3, 5


class OracleError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned status {status}")
        self.status = status


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
             "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        L.sao_window_topk_idxs_shape.argtypes = [i32, i32, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.sao_window_topk_idxs.argtypes = [i32, i32, i32, i64, vp, i64]
        L.sao_ring_write.argtypes = [vp, vp, i32, i32, i32, i64, i32]
        L.sao_pow2_ceil.argtypes = [f32]
        L.sao_pow2_ceil.restype = f32
        L.sao_act_quant_fp8_inplace.argtypes = [vp, i64, i32]
        L.sao_kv8_pack.argtypes = [vp, vp, vp, i64, i32]
        L.sao_kv8_unpack.argtypes = [vp, vp, vp, i64, i32]
        L.sao_append_compressed_idxs.argtypes = [vp, i64, i32, vp, i64, i32, i32]
        L.sao_sparse_attn.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i64, i32, f32, vp, vp]
        L.sao_apply_rotary.argtypes = [vp, i64, i64, i32, i32, i32, vp, i64, i64, ctypes.c_int]
        L.sao_indexer_topk.argtypes = [vp, i64, i64, i32, i64, i32, i32, i32, vp, i64, i32]
        L.sao_set_threads.argtypes = [ctypes.c_int]
        for name in ("sao_window_topk_idxs_shape", "sao_window_topk_idxs", "sao_ring_write",
                     "sao_act_quant_fp8_inplace", "sao_append_compressed_idxs", "sao_sparse_attn",
                     "sao_kv8_pack", "sao_kv8_unpack", "sao_apply_rotary", "sao_indexer_topk", "sao_set_threads"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def set_threads(n: int = 0) -> int:
    """Thread count of the oracle's parallel loops (n > 0 sets it); returns the
    count they use from now on."""
    return int(lib().sao_set_threads(int(n)))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(fn: str, st: int):
    if st != OK:
        raise OracleError(fn, st)


def window_topk_idxs_shape(window: int, seqlen: int, start_pos: int) -> tuple[int, int]:
    r, c = ctypes.c_int32(), ctypes.c_int32()
    _check("sao_window_topk_idxs_shape",
           lib().sao_window_topk_idxs_shape(window, seqlen, start_pos, ctypes.byref(r), ctypes.byref(c)))
    return r.value, c.value


def window_topk_idxs(window: int, bsz: int, seqlen: int, start_pos: int) -> np.ndarray:
    """int32 [bsz][rows][cols] slot lists (-1 = empty slot)."""
    rows, cols = window_topk_idxs_shape(window, seqlen, start_pos)
    out = np.full((bsz, rows, cols), -7, dtype=np.int32)
    _check("sao_window_topk_idxs",
           lib().sao_window_topk_idxs(window, bsz, seqlen, start_pos, _ptr(out), cols))
    return out


def window_topk_idxs_into(out: np.ndarray, window: int, bsz: int, seqlen: int, start_pos: int):
    """Writes the window lists into the first columns of ``out`` [bsz][rows][stride]."""
    assert out.dtype == np.int32 and out.flags.c_contiguous
    _check("sao_window_topk_idxs",
           lib().sao_window_topk_idxs(window, bsz, seqlen, start_pos, _ptr(out), out.shape[-1]))


def ring_write(ring: np.ndarray, rows: np.ndarray, start_pos: int) -> None:
    """ring uint16 [bsz][window][d] updated in place with rows uint16 [bsz][seqlen][d]."""
    assert ring.dtype == np.uint16 and rows.dtype == np.uint16
    assert ring.flags.c_contiguous and rows.flags.c_contiguous
    bsz, window, d = ring.shape
    assert rows.shape[0] == bsz and rows.shape[2] == d
    _check("sao_ring_write",
           lib().sao_ring_write(_ptr(ring), _ptr(rows), bsz, window, d, start_pos, rows.shape[1]))


def pow2_ceil(v: float) -> float:
    return float(lib().sao_pow2_ceil(v))


def act_quant_fp8_inplace(x: np.ndarray) -> None:
    """x uint16 (bf16 bits) [..., row_len], row_len % 32 == 0, rounded through fp8 in place."""
    assert x.dtype == np.uint16 and x.flags.c_contiguous
    row_len = x.shape[-1]
    n_rows = x.size // row_len if row_len else 0
    _check("sao_act_quant_fp8_inplace", lib().sao_act_quant_fp8_inplace(_ptr(x), n_rows, row_len))


def act_quant_fp8(x: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(x).copy()
    act_quant_fp8_inplace(y)
    return y


def kv8_pack(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits [..., row_len] -> (e4m3fn codes uint8 [..., row_len], E8M0 scale bytes [..., row_len // 32])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    row_len = x.shape[-1]
    n_rows = x.size // row_len if row_len else 0
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (row_len // 32,), dtype=np.uint8)
    _check("sao_kv8_pack", lib().sao_kv8_pack(_ptr(x), _ptr(codes), _ptr(scales), n_rows, row_len))
    return codes, scales


def kv8_unpack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    row_len = codes.shape[-1]
    n_rows = codes.size // row_len if row_len else 0
    x = np.empty(codes.shape, dtype=np.uint16)
    _check("sao_kv8_unpack", lib().sao_kv8_unpack(_ptr(codes), _ptr(scales), _ptr(x), n_rows, row_len))
    return x


def append_compressed_idxs(out: np.ndarray, col0: int, cidx: np.ndarray, offset: int) -> None:
    """out int32 [..., stride]; writes cidx (+offset, -1 kept) into columns col0.. ."""
    assert out.dtype == np.int32 and cidx.dtype == np.int32
    assert out.flags.c_contiguous and cidx.flags.c_contiguous
    stride = out.shape[-1]
    kc = cidx.shape[-1]
    n_rows = cidx.size // kc if kc else out.size // max(stride, 1)
    assert out.size // stride == n_rows
    _check("sao_append_compressed_idxs",
           lib().sao_append_compressed_idxs(_ptr(out), stride, col0, _ptr(cidx), n_rows, kc, offset))


def sparse_attn(q: np.ndarray, kv: np.ndarray, sink: np.ndarray, idx: np.ndarray, scale: float,
                want_f32: bool = False):
    """q uint16 [b][s][h][d], kv uint16 [b][rows][d], sink f32 [h], idx int32 [b][s][topk].

    Returns out uint16 [b][s][h][d] (bf16 bits), plus the f32 value before rounding when
    ``want_f32``."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    sink = np.ascontiguousarray(sink, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    b, s, h, d = q.shape
    assert kv.shape[0] == b and kv.shape[2] == d, (kv.shape, q.shape)
    assert idx.shape[:2] == (b, s) and sink.shape == (h,)
    rows, topk = kv.shape[1], idx.shape[2]
    out = np.zeros((b, s, h, d), dtype=np.uint16)
    out32 = np.zeros((b, s, h, d), dtype=np.float32) if want_f32 else None
    _check("sao_sparse_attn",
           lib().sao_sparse_attn(_ptr(q), _ptr(kv), _ptr(sink), _ptr(idx), b, s, h, d, rows, topk,
                                 float(scale), _ptr(out), _ptr(out32)))
    return (out, out32) if want_f32 else out


def apply_rotary(x: np.ndarray, table: np.ndarray, rope_dim: int, start_pos: int, inverse: bool) -> np.ndarray:
    """Rotary embedding of the last ``rope_dim`` values of bf16 bits ``x``
    [b][s][h][row_len] (or [b][s][row_len]); row (b, s, .) at position start_pos + s.
    ``table`` [n_pos][rope_dim / 2][2] f32 (cos, sin).  Returns a rotated copy."""
    y = np.ascontiguousarray(x, dtype=np.uint16).copy()
    shp = y.shape
    b, s = shp[0], shp[1]
    h = shp[2] if y.ndim == 4 else 1
    t = np.ascontiguousarray(table, dtype=np.float32)
    _check("sao_apply_rotary", lib().sao_apply_rotary(_ptr(y), b, s, h, shp[-1], rope_dim, _ptr(t), t.shape[0],
                                                       start_pos, int(bool(inverse))))
    return y


def indexer_topk(scores: np.ndarray, start_pos: int, ratio: int, index_topk: int, offset: int) -> np.ndarray:
    """Indexer selection tail: scores [b][s][T] f32 -> int32 [b][s][min(index_topk, T)]
    (positions + offset in position order, -1 where unreachable)."""
    sc = np.ascontiguousarray(scores, dtype=np.float32)
    b, s, T = sc.shape
    topk = min(index_topk, T)
    out = np.full((b, s, topk), -7, dtype=np.int32)
    _check("sao_indexer_topk", lib().sao_indexer_topk(_ptr(sc), b, s, T, start_pos, ratio, index_topk, offset,
                                                       _ptr(out), topk, 0))
    return out
