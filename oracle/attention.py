"""Oracle: per-layer sparse attention over selected FP4 entries plus the FP8 window.

Test infrastructure only (see ``oracle/__init__``).

What the pages fix: every CSA2 layer keeps its own main query and its own
sliding-window KV in all three modes (P1 CSA2 section; P2 section 03; P4
section 二); the window is 128 tokens in every layer (P1 section "Causal
Encoder-Decoder"; P4 section 一); core attention runs over the selected main-KV
entries concatenated with the window KV (P5 figure caption of the attention
diagram: Selection / Top-K / Concatenation); main KV is FP4 and window KV FP8
(P2 section 03; P5 section "缓存精度与持久化分层").

Readings where the pages are silent:

* one joint softmax over [DQ4(main_j) for valid j in the list] ++ [DQ8(window
  row i)], no de-duplication between the two sets, no sink;
* keys and values are the same shared latent row (MQA over the latent);
  entries are stored after RoPE, so no rotation is applied here;
* z_hj = tau * q_h . k_j with tau the caller's softmax scale (D^-1/2 by
  default); o_h = sum_j p_hj k_j; lse_h = log sum_j exp(z_hj) (natural log);
* list entries < 0 or >= the query's visible count are skipped; an empty key
  set gives o = 0 and lse = -inf.

Parity pins (tests/test_oracle_attention.py): with Top-K covering every entry
the result equals dense attention computed by
torch.nn.functional.scaled_dot_product_attention in fp64; merging the
selected-only and window-only results by log-sum-exp equals the joint result;
invariance to the order of the index list; one key gives o = k; a zero query
gives the mean of the keys and lse = log(n).
"""
from __future__ import annotations

import numpy as np

from .codec import fp4_decode, fp8_rows_decode


def gather_keys(main_codes, main_scales, idx, vis, swa_codes=None, swa_scale=None) -> np.ndarray:
    """Key/value rows [n, D] of one query: selected main rows then window rows."""
    idx = np.asarray(idx, dtype=np.int64)
    valid = idx[(idx >= 0) & (idx < vis)]
    parts = []
    if len(valid):
        parts.append(fp4_decode(np.asarray(main_codes)[valid], np.asarray(main_scales)[valid]))
    if swa_codes is not None and len(swa_codes):
        parts.append(fp8_rows_decode(swa_codes, swa_scale))
    if not parts:
        dim = np.asarray(main_codes).shape[1] * 2
        return np.zeros((0, dim), dtype=np.float64)
    return np.concatenate(parts, axis=0)


def attend(q: np.ndarray, keys: np.ndarray, tau: float):
    """Softmax attention of heads q [H, D] over keys = values [n, D], fp64.

    Returns (o [H, D], lse [H]).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    h, d = q.shape
    if len(keys) == 0:
        return np.zeros((h, d)), np.full(h, -np.inf)
    z = tau * (q @ keys.T)                                  # [H, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    return p @ keys, (m + np.log(l))[:, 0]


def sparse_swa_attention(q, main_codes, main_scales, idx, vis, swa_codes, swa_scale, tau):
    """One query's layer attention: selected FP4 entries ++ FP8 window rows."""
    keys = gather_keys(main_codes, main_scales, idx, vis, swa_codes, swa_scale)
    return attend(q, keys, tau)


def lse_merge(parts):
    """Combine [(o_i, lse_i)] of disjoint key sets into the joint (o, lse)."""
    lses = np.stack([p[1] for p in parts])                  # [n, H]
    m = np.max(lses, axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    wts = np.exp(lses - m_safe)                              # exp(-inf) = 0
    tot = wts.sum(axis=0)
    o = sum(w[:, None] * p[0] for w, p in zip(wts, parts))
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(tot[:, None] > 0, o / np.where(tot > 0, tot, 1.0)[:, None], 0.0)
        lse = np.where(tot > 0, m_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    return o, lse
