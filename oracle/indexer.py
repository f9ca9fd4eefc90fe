"""Oracle: Hierarchical Sparse Indexer (Full / Reindex / Reuse, flat prefill).

Test infrastructure only (see ``oracle/__init__``).

What the pages fix:

* three static layer modes (P1 section "Compressed Sparse Attention 2
  (CSA2)"; P4 section 二, mode table; P5 section "CSA2注意力"): Full computes
  its own main KV, projects the indexer key from it and selects a fresh
  Top-512; Reindex reuses the previous Full layer's main KV and indexer keys
  and re-scores them with its own indexer query; Reuse reuses the main KV and
  the latest Top-K list and runs no indexer;
* the decoder's hierarchical indexer (P1 CSA2 section; P2 section 03; P4
  section 二; P5 figure caption "Hierarchical Sparse Indexer"): the first Full
  layer scores every causally visible position, ranks 8-position blocks by
  their maximum score and keeps 2,048 blocks (16,384 positions) as a candidate
  pool; later Reindex layers score only pool positions and take Top-512;
* the encoder uses no pool (flat Top-K per query).

Readings where the pages are silent:

* score of entry j: s_j = sum_h w_h * max(0, q_h . k_j) over indexer heads h,
  with k_j the dequantised FP4 indexer key, q in bf16, w in fp32, all products
  and sums in fp64; no further scale factor;
* entry j (one per r tokens) is visible to token t iff (j+1)*r - 1 <= t, so
  a query sees vis = min(len, floor((t+1)/r)) entries;
* blocks are aligned at multiples of 8; a partial last block takes the max of
  its visible positions; blocks without visible positions do not exist;
* the pool is the min(P, #blocks) blocks ordered by (block max desc, block id
  asc); Top-K is the min(K, #candidates) positions ordered by (score desc,
  position asc); lists are returned ascending and padded with -1;
* the Full layer's Top-K is taken from its own pool (it equals the flat Top-K
  whenever K <= P, see the invariant tests).

Parity pins (tests/test_oracle_indexer.py): brute force over tiny inputs with
explicit Python loops and full sorts; invariants hierarchical == flat when the
pool covers the context, Full-from-pool == flat for K <= P, K >= N selects
every visible position, Reindex with the Full layer's own query == Full,
Reuse == the group's list; planted keys with known winners; a single-head
unit-query case whose scores are the key channel itself.
"""
from __future__ import annotations

import numpy as np

from .codec import fp4_decode

BLOCK = 8


def visible_count(seq_len: int, t: int, ratio: int) -> int:
    """Entries of a length-``seq_len`` cache visible to token ``t`` at ratio ``ratio``."""
    return int(max(0, min(seq_len, (t + 1) // ratio)))


def scores(q_idx: np.ndarray, w_idx: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """s_j = sum_h w_h * relu(q_h . k_j) in fp64.

    q_idx [H_I, d_I] (fp values of the bf16 query), w_idx [H_I], keys [N, d_I]
    (dequantised indexer keys).
    """
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w_idx, dtype=np.float64)
    dots = np.asarray(keys, dtype=np.float64) @ q.T          # [N, H_I]
    return np.maximum(dots, 0.0) @ w


def scores_of_rows(q_idx, w_idx, ik_codes, ik_scales) -> np.ndarray:
    return scores(q_idx, w_idx, fp4_decode(ik_codes, ik_scales))


def order_desc(values: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Permutation of ``ids`` sorted by (value desc, id asc)."""
    return np.lexsort((ids, -np.asarray(values, dtype=np.float64)))


def top_ids(values: np.ndarray, ids: np.ndarray, k: int) -> np.ndarray:
    """The ``k`` ids ranked first by (value desc, id asc), ascending."""
    perm = order_desc(values, ids)
    return np.sort(np.asarray(ids)[perm[:k]])


def pad(ids: np.ndarray, n: int) -> np.ndarray:
    out = np.full(n, -1, dtype=np.int64)
    out[:len(ids)] = ids
    return out


def block_max(s: np.ndarray) -> np.ndarray:
    """Max score of each 8-position block of s (last block may be partial)."""
    n = len(s)
    nb = (n + BLOCK - 1) // BLOCK
    return np.array([s[b * BLOCK:min(n, (b + 1) * BLOCK)].max() for b in range(nb)], dtype=np.float64)


def pool_select(bmax: np.ndarray, pool_blocks: int) -> np.ndarray:
    """Top min(P, #blocks) block ids by (block max desc, block id asc), ascending."""
    return top_ids(bmax, np.arange(len(bmax)), min(pool_blocks, len(bmax)))


def pool_positions(pool: np.ndarray, vis: int) -> np.ndarray:
    """Visible positions of the pool blocks, ascending."""
    pool = np.asarray(pool)
    pool = pool[pool >= 0]
    pos = (pool[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    return np.sort(pos[pos < vis])


def index_full(q_idx, w_idx, keys_vis: np.ndarray, pool_blocks: int, top_k: int):
    """Full layer over the visible keys [vis, d_I].

    Returns (pool ids padded to P, pool count, top-k positions padded to K,
    scores of all visible positions).
    """
    s = scores(q_idx, w_idx, keys_vis)
    vis = len(s)
    if vis == 0:
        return pad(np.zeros(0, np.int64), pool_blocks), 0, pad(np.zeros(0, np.int64), top_k), s
    pool = pool_select(block_max(s), pool_blocks)
    cand = pool_positions(pool, vis)
    sel = top_ids(s[cand], cand, min(top_k, len(cand)))
    return pad(pool, pool_blocks), len(pool), pad(sel, top_k), s


def reindex(q_idx, w_idx, keys_vis: np.ndarray, pool: np.ndarray, top_k: int):
    """Reindex layer: its own (q, w) scored over the given pool's visible positions."""
    vis = len(keys_vis)
    cand = pool_positions(pool, vis)
    if len(cand) == 0:
        return pad(np.zeros(0, np.int64), top_k), np.zeros(0)
    s = scores(q_idx, w_idx, keys_vis[cand])
    sel = top_ids(s, cand, min(top_k, len(cand)))
    return pad(sel, top_k), s


def index_flat(q_idx, w_idx, keys_vis: np.ndarray, top_k: int):
    """No pool: Top-K over every visible position (encoder / prefill)."""
    s = scores(q_idx, w_idx, keys_vis)
    sel = top_ids(s, np.arange(len(s)), min(top_k, len(s)))
    return pad(sel, top_k), s


def reuse(latest_idx: np.ndarray) -> np.ndarray:
    """Reuse layer: the group's latest Top-K list, unchanged."""
    return np.array(latest_idx, copy=True)


def tie_band(values: np.ndarray, k: int, rel: float = 1e-4):
    """Near-tie band around the k-th largest value: (theta, mask of |v - theta| <= rel*|theta|)."""
    v = np.asarray(values, dtype=np.float64)
    if k <= 0 or len(v) == 0:
        return None, np.zeros(len(v), bool)
    k = min(k, len(v))
    theta = np.sort(v)[::-1][k - 1]
    return theta, np.abs(v - theta) <= rel * abs(theta)
