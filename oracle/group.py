"""Oracle: one CSA2 layer group for one query, composed from the steps.

Test infrastructure only (see ``oracle/__init__``).

Group layouts (P1 CSA2 section; P4 section 二; P5 section "CSA2注意力"): the
decoder's 20 CSA2 layers form 5 groups of 4 at ratio 1 - the first group is
Full + 3 Reuse, the others Reindex + 3 Reuse - and the encoder's 18 CSA2
layers form 3 groups of 6 at ratio 2, each Full + 5 Reuse.  Every layer of a
group attends with its own query and window rows over the group's single
Top-K list (Reuse copies it, P1 CSA2 section).

Parity pins (tests/test_oracle_group.py): planted indexer keys whose scores
are known by construction fix the selected lists of both functions at tokens
before the cache's last entry and at ratio 2 inside a two-token entry
(planted winners the token may not see yet must stay out); every layer's
output equals torch's scaled_dot_product_attention in fp64 over the rows of
the known list plus the layer's window (tests/test_oracle_attention.py adds
the Reuse-list and per-layer composition checks).
"""
from __future__ import annotations

import numpy as np

from . import attention, indexer
from .codec import fp4_decode


def decoder_group(first_mode: str, main_codes, main_scales, ik_codes, ik_scales, t: int, ratio: int,
                  q_idx, w_idx, pool_in, pool_blocks: int, top_k: int, layers, tau: float):
    """One decoder group for one query at token ``t``.

    ``main_*`` / ``ik_*`` are the sequence's whole caches (rows = entries);
    ``layers`` is a list of (q [H, D], swa_codes [n, D], swa_scale [n]);
    ``first_mode`` is "full" (builds the pool) or "reindex" (uses ``pool_in``).
    Returns dict(pool, pool_count, idx, scores, out=[(o, lse), ...]).
    """
    vis = indexer.visible_count(len(ik_codes), t, ratio)
    keys = fp4_decode(ik_codes[:vis], ik_scales[:vis])
    if first_mode == "full":
        pool, count, idx, s = indexer.index_full(q_idx, w_idx, keys, pool_blocks, top_k)
    elif first_mode == "reindex":
        pool = np.asarray(pool_in)
        count = int((pool >= 0).sum())
        idx, s = indexer.reindex(q_idx, w_idx, keys, pool, top_k)
    else:
        raise ValueError(first_mode)
    outs = []
    group_idx = idx
    for q, swa_codes, swa_scale in layers:
        layer_idx = indexer.reuse(group_idx)
        outs.append(attention.sparse_swa_attention(q, main_codes, main_scales, layer_idx, vis,
                                                   swa_codes, swa_scale, tau))
    return dict(pool=pool, pool_count=count, idx=idx, scores=s, out=outs)


def encoder_group_query(main_codes, main_scales, ik_codes, ik_scales, t: int, ratio: int,
                        q_idx, w_idx, top_k: int, layers, tau: float):
    """One encoder group (Full + Reuse layers, flat Top-K) for one prefill query."""
    vis = indexer.visible_count(len(ik_codes), t, ratio)
    keys = fp4_decode(ik_codes[:vis], ik_scales[:vis])
    idx, s = indexer.index_flat(q_idx, w_idx, keys, top_k)
    outs = [attention.sparse_swa_attention(q, main_codes, main_scales, indexer.reuse(idx), vis,
                                           swa_codes, swa_scale, tau)
            for q, swa_codes, swa_scale in layers]
    return dict(idx=idx, scores=s, out=outs)
