"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fp4_kv_cache_02_amd as csa2


def announce(*parts) -> None:
    """Print (and flush) what the next GPU step is, so a crash names its case."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def dev() -> torch.device:
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch.device("cuda:0")


def t(a: np.ndarray) -> torch.Tensor:
    """numpy -> contiguous device tensor (uint16 arrays are passed as int16 bit patterns)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def h(x: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return x.detach().cpu().numpy()


def empty_u8(*shape) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.uint8, device=dev())


def workspace(nbytes: int) -> torch.Tensor:
    # zero-filled before first use, as the attention and group calls require
    return torch.zeros(max(256, nbytes), dtype=torch.uint8, device=dev())


def gpu_quantize(x: np.ndarray, w_ik: np.ndarray | None = None):
    """Quantise fp32 rows on the GPU; returns device (codes, scales[, ik_codes, ik_scales])."""
    rows, dim = x.shape
    xd = t(x.astype(np.float32))
    codes, scales = empty_u8(rows, dim // 2), empty_u8(rows, dim // 16)
    if w_ik is None:
        csa2.csa2_quantize_fp4(xd, codes, scales)
        return codes, scales
    di = w_ik.shape[1]
    ikc, iks = empty_u8(rows, di // 2), empty_u8(rows, di // 16)
    csa2.csa2_quantize_fp4(xd, codes, scales, w_ik=t(w_ik.astype(np.float32)), ik_codes=ikc, ik_scales=iks)
    return codes, scales, ikc, iks


def assert_sets_equal_modulo_band(gpu_ids, ora_ids, values_of, k, rel=1e-4, what="set"):
    """Equal as sets except inside the near-tie band around the k-th value.

    ``values_of(ids)`` returns the oracle values of ids.  Band = ids whose value
    lies within rel*|theta| of theta, the k-th largest oracle value of the
    oracle's own selection.  Returns the number of band elements involved.
    """
    g = set(int(v) for v in gpu_ids if v >= 0)
    o = set(int(v) for v in ora_ids if v >= 0)
    assert len(g) == len(o), (what, len(g), len(o))
    if g == o:
        return 0
    ov = values_of(np.array(sorted(o)))
    theta = np.sort(ov)[::-1][min(k, len(ov)) - 1]
    tol = rel * abs(theta)
    diff = sorted(g ^ o)
    dv = values_of(np.array(diff))
    bad = [(i, v) for i, v in zip(diff, dv) if abs(v - theta) > tol]
    assert not bad, f"{what}: {len(bad)} differences outside the near-tie band (theta={theta}): {bad[:8]}"
    return len(diff)
