"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fp4_kv_cache_02_amd as csa2
import synth


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
    # no call needs initial workspace contents: fill it with a byte pattern so
    # that a kernel reading what it did not write shows up in the results
    return torch.full((max(256, nbytes),), 0xA5, dtype=torch.uint8, device=dev())


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


def random_group(cfg, lens, n_layers, D=512, H=64, DI=128, HI=8, P=256, K=128, W=64):
    """A Full decode group over raw random FP4 caches (one query per sequence at
    its last entry) with bf16 queries and FP8 windows; returns a function that
    builds a fresh descriptor and fresh output tensors (filled with marker
    values) on each call: (group, [pool, count, topk, score, out..., lse...]).
    """
    M = len(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    n = int(sum(lens))
    rc, rs = synth.fp4_bytes(cfg, 0, n, D)
    ic, is_ = synth.fp4_bytes(cfg, 1, n, DI)
    kv = csa2.fp4_cache(t(rc), t(rs), t(starts), t(np.asarray(lens, np.int32)), D, max(lens), 1)
    idx = csa2.fp4_cache(t(ic), t(is_), t(starts), t(np.asarray(lens, np.int32)), DI, max(lens), 1)
    qs = csa2.queries(t(np.arange(M, dtype=np.int32)), t((np.asarray(lens) - 1).astype(np.int32)))
    qi, wi = synth.q_idx(cfg, 0, M, HI, DI), synth.w_idx(cfg, 0, M, HI)
    q_list, swa_list = [], []
    for layer in range(n_layers):
        q_list.append(t(synth.q_main(cfg, layer, M, H, D, "bf16")).view(torch.bfloat16))
        sc, ss = empty_u8(M * W, D), torch.empty((M * W,), dtype=torch.float32, device=dev())
        csa2.csa2_quantize_fp8_rows(t(synth.swa_rows(cfg, layer, 0, M * W, D)), sc, ss)
        swa_list.append(csa2.swa(sc, ss, t(np.arange(M, dtype=np.int32) * W), t(np.full(M, W, np.int32)), D, W))

    def outputs():
        pool = torch.full((M, P), -7, dtype=torch.int32, device=dev())
        cnt = torch.full((M,), -7, dtype=torch.int32, device=dev())
        topk = torch.full((M, K), -7, dtype=torch.int32, device=dev())
        score = torch.full((M, K), -7.0, dtype=torch.float32, device=dev())
        out = [torch.full((M, H, D), 7.0, dtype=torch.float32, device=dev()) for _ in range(n_layers)]
        lse = [torch.full((M, H), 7.0, dtype=torch.float32, device=dev()) for _ in range(n_layers)]
        g = csa2.Group(csa2.CSA2_MODE_FULL, kv, idx, qs, t(qi).view(torch.bfloat16), t(wi), P, K, pool, cnt, topk,
                       score, q_list, csa2.CSA2_BF16, H, swa_list, out, lse, D ** -0.5)
        return g, [pool, cnt, topk, score] + out + lse

    return outputs
