"""Shared test helpers: bit views, the parity tolerance, GPU guards."""
from __future__ import annotations

import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 numpy view of a bf16 tensor (copied to the host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def bf16_f32(a: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(a).astype(np.uint32) << 16).view(np.float32)


def bf16_ulp(r: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values (8 significant bits) at |r|; 0 where r == 0."""
    a = np.abs(r.astype(np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 7), 0.0)


def parity_tolerance(ref: np.ndarray) -> np.ndarray:
    """Per-element bound: 2 bf16 ulps of the reference, or 1e-2 absolute, whichever is larger."""
    return np.maximum(2.0 * bf16_ulp(ref), 1e-2)


def assert_parity(gpu_bits: np.ndarray, ref_f32: np.ndarray, what: str = "") -> dict:
    """GPU bf16 output vs the oracle's f32 value, element by element."""
    g = bf16_f32(gpu_bits).astype(np.float64)
    r = ref_f32.astype(np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    tol = parity_tolerance(r)
    bad = err > tol
    stats = dict(max_abs=float(err.max(initial=0.0)),
                 max_rel=float((err / np.maximum(np.abs(r), 1e-30)).max(initial=0.0)),
                 mean_abs=float(err.mean()) if err.size else 0.0)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance; "
                           f"worst {float((err - tol).max())} over; {stats}")
    return stats


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU (the HIP path has no CPU fallback)")


def all_finite_bf16() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_f32(b)
    return b[np.isfinite(f)]


def act_quant_blocks() -> np.ndarray:
    """[nblk][32] bf16 bits: every finite bf16 value quantised under many block
    amax values (each power-of-two scale, exact-boundary and just-above amax,
    the 1e-4 floor, the top of the range)."""
    vals = all_finite_bf16()
    fv = bf16_f32(vals).astype(np.float64)
    amaxes = []
    for k in range(-40, 120, 3):
        amaxes.append(448.0 * 2.0 ** k)
        amaxes.append(448.0 * (1 + 2.0 ** -7) * 2.0 ** k)
    amaxes += [5e-5, 1e-4, 3.3e38]
    blocks = []
    for A in amaxes:
        A_bits = bits(torch.tensor([A], dtype=torch.float32).to(torch.bfloat16))[0]
        A_val = float(bf16_f32(np.array([A_bits], dtype=np.uint16))[0])
        if not np.isfinite(A_val):
            continue
        members = vals[np.abs(fv) <= A_val]
        pad = (-len(members)) % 31
        members = np.concatenate([members, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 31)
        blocks.append(np.concatenate([np.full((len(members), 1), A_bits, dtype=np.uint16), members], axis=1))
    return np.ascontiguousarray(np.concatenate(blocks))
