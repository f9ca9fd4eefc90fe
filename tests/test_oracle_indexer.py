"""Pins of the oracle's hierarchical sparse indexer (CPU only)."""
import math
import os

import numpy as np
import pytest

import synth
from oracle import codec, indexer


def _dyadic_keys(rng, n, d):
    """Dequantised FP4 keys with small scales: every score below is exact in fp64."""
    x = rng.standard_normal((n, d)).astype(np.float32)
    codes, scales = codec.fp4_encode(x)
    scales = np.clip(scales, 0x30, 0x40).astype(np.uint8)      # scales in [0.5, 2]
    return codec.fp4_decode(codes, scales)


def _small_query(rng, h, d):
    q = rng.integers(-4, 5, size=(h, d)).astype(np.float64) / 2
    w = rng.integers(-3, 4, size=h).astype(np.float64)
    w[0] = abs(w[0]) + 1
    return q, w


def _bf_scores(q, w, keys):
    out = []
    for k in keys.tolist():
        tot = 0.0
        for h in range(len(w)):
            dot = 0.0
            for c in range(len(k)):
                dot += q[h][c] * k[c]
            tot += w[h] * max(0.0, dot)
        out.append(tot)
    return out


def _bf_full(q, w, keys, P, K):
    s = _bf_scores(q.tolist(), w.tolist(), keys)
    n = len(s)
    nb = (n + 7) // 8
    bm = [max(s[8 * b:min(n, 8 * b + 8)]) for b in range(nb)]
    pool = sorted(sorted(range(nb), key=lambda b: (-bm[b], b))[:P])
    cand = [j for b in pool for j in range(8 * b, min(n, 8 * b + 8))]
    sel = sorted(sorted(cand, key=lambda j: (-s[j], j))[:K])
    return pool, sel


@pytest.mark.parametrize("n", [1, 7, 8, 9, 63, 64, 65, 513])
@pytest.mark.parametrize("P,K", [(1, 1), (2, 8), (4, 5), (8, 64), (64, 16)])
def test_full_bruteforce_tiny(n, P, K):
    rng = np.random.default_rng(n * 1000 + P * 10 + K)
    keys = _dyadic_keys(rng, n, 16)
    q, w = _small_query(rng, 3, 16)
    pool, cnt, sel, s = indexer.index_full(q, w, keys, P, K)
    bp, bs = _bf_full(q, w, keys, P, K)
    assert pool[:cnt].tolist() == bp and np.all(pool[cnt:] == -1)
    got = sel[sel >= 0].tolist()
    assert got == bs and np.all(sel[len(got):] == -1) and len(sel) == K


def test_scores_exact_against_bruteforce():
    rng = np.random.default_rng(11)
    keys = _dyadic_keys(rng, 50, 32)
    q, w = _small_query(rng, 4, 32)
    assert indexer.scores(q, w, keys).tolist() == _bf_scores(q.tolist(), w.tolist(), keys)


def test_score_unit_query_is_key_channel():
    rng = np.random.default_rng(12)
    keys = _dyadic_keys(rng, 40, 16)
    q = np.zeros((1, 16))
    q[0, 5] = 1.0
    assert np.array_equal(indexer.scores(q, np.array([1.0]), keys), np.maximum(keys[:, 5], 0))
    # a negative head weight flips the sign of that head's contribution
    assert np.array_equal(indexer.scores(q, np.array([-2.0]), keys), -2 * np.maximum(keys[:, 5], 0))


def test_all_equal_scores_pick_lowest_ids():
    keys = np.ones((100, 8))
    q = np.ones((2, 8)) / 8
    w = np.array([1.0, 1.0])
    pool, cnt, sel, _ = indexer.index_full(q, w, keys, 3, 10)
    assert pool[:cnt].tolist() == [0, 1, 2]
    assert sel.tolist() == list(range(10))


def test_planted_winners():
    rng = np.random.default_rng(13)
    n, d = 4096, 64
    keys = _dyadic_keys(rng, n, d) * 0.01
    q, w = np.zeros((2, d)), np.array([1.0, 0.5])
    q[0, :] = 1.0
    planted = np.sort(rng.choice(n, 40, replace=False))
    keys[planted, :] = np.linspace(2, 3, 40)[:, None]
    pool, cnt, sel, _ = indexer.index_full(q, w, keys, 64, 40)
    assert sel.tolist() == planted.tolist()
    assert set((planted // 8).tolist()) <= set(pool[:cnt].tolist())


def test_hierarchical_equals_flat_when_pool_covers_context():
    rng = np.random.default_rng(14)
    for n, P, K in [(4096, 512, 64), (1000, 125, 300), (4096, 600, 64)]:
        keys = rng.standard_normal((n, 32))
        q, w = rng.standard_normal((4, 32)), np.abs(rng.standard_normal(4))
        _, cnt, sel, _ = indexer.index_full(q, w, keys, P, K)
        flat, _ = indexer.index_flat(q, w, keys, K)
        assert cnt == min(P, (n + 7) // 8)
        assert np.array_equal(sel, flat)


def test_full_from_pool_equals_flat_when_k_le_p():
    # the <= K blocks holding the flat top-K all have block max >= the K-th score,
    # so they rank among the top K <= P blocks
    rng = np.random.default_rng(15)
    for n, P, K in [(4096, 64, 64), (4096, 64, 17), (20000, 100, 90), (777, 9, 9)]:
        keys = rng.standard_normal((n, 32))
        q, w = rng.standard_normal((4, 32)), rng.standard_normal(4)
        _, _, sel, _ = indexer.index_full(q, w, keys, P, K)
        flat, _ = indexer.index_flat(q, w, keys, K)
        assert np.array_equal(sel, flat)


def test_k_ge_visible_selects_everything():
    rng = np.random.default_rng(16)
    keys = rng.standard_normal((37, 8))
    q, w = rng.standard_normal((2, 8)), rng.standard_normal(2)
    _, _, sel, _ = indexer.index_full(q, w, keys, 100, 64)
    assert sel[:37].tolist() == list(range(37)) and np.all(sel[37:] == -1)
    flat, _ = indexer.index_flat(q, w, keys, 40)
    assert flat[:37].tolist() == list(range(37))


def test_reindex_with_full_query_reproduces_full():
    rng = np.random.default_rng(17)
    keys = rng.standard_normal((6000, 32))
    q, w = rng.standard_normal((4, 32)), rng.standard_normal(4)
    pool, cnt, sel, _ = indexer.index_full(q, w, keys, 64, 48)
    again, _ = indexer.reindex(q, w, keys, pool, 48)
    assert np.array_equal(again, sel)
    # another query selects only inside the pool
    q2, w2 = rng.standard_normal((4, 32)), rng.standard_normal(4)
    other, _ = indexer.reindex(q2, w2, keys, pool, 48)
    assert set((other[other >= 0] // 8).tolist()) <= set(pool[:cnt].tolist())


def test_reuse_copies_the_list():
    lst = np.array([3, 9, 11, -1])
    out = indexer.reuse(lst)
    assert np.array_equal(out, lst) and out is not lst


def test_visibility_rule():
    assert indexer.visible_count(100, 99, 1) == 100
    assert indexer.visible_count(100, 50, 1) == 51
    # ratio 2: entry j covers tokens 2j, 2j+1 and is visible once token 2j+1 is seen
    assert indexer.visible_count(65536, 131071, 2) == 65536
    assert indexer.visible_count(65536, 126976, 2) == 63488
    assert indexer.visible_count(65536, 126977, 2) == 63489
    assert indexer.visible_count(10, -1, 1) == 0


def test_partial_last_block():
    s_keys = np.zeros((11, 1))
    s_keys[10, 0] = 5.0     # only visible position of block 1 above zero
    q, w = np.ones((1, 1)), np.ones(1)
    pool, cnt, sel, s = indexer.index_full(q, w, s_keys, 1, 1)
    assert pool[:cnt].tolist() == [1] and sel.tolist() == [10]
    assert indexer.block_max(s).tolist() == [0.0, 5.0]


def test_tie_band():
    v = np.array([5.0, 4.0, 3.00001, 3.0, 2.99999, 1.0])
    theta, band = indexer.tie_band(v, 4, 1e-4)
    assert theta == 3.0 and band.tolist() == [False, False, True, True, True, False]


def test_method_constants_golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "method_constants.txt")
    kv = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            kv[k] = v
    assert indexer.BLOCK == int(kv["block_positions"])
    assert codec.GROUP == int(kv["fp4_group"])
    assert int(kv["pool_blocks"]) * int(kv["block_positions"]) == int(kv["pool_positions"])
    to_modes = {"F": "full", "R": "reindex", "U": "reuse"}
    dec = [[to_modes[m] for m in g.split(",")] for g in kv["decoder_groups"].split("|")]
    enc = [[to_modes[m] for m in g.split(",")] for g in kv["encoder_groups"].split("|")]
    for cfg in (1, 3, 4):
        wl = synth.workload(cfg)
        assert wl.groups == dec and wl.ratio == int(kv["decoder_ratio"]) and wl.n_layers == 20
        assert wl.pool_blocks == int(kv["pool_blocks"]) and wl.top_k == int(kv["top_k"])
        assert wl.window == int(kv["window"])
    wl = synth.workload(2)
    assert wl.groups == enc and wl.ratio == int(kv["encoder_ratio"]) and wl.n_layers == 18
    assert wl.top_k == int(kv["top_k"]) and wl.pool_blocks == 0 and wl.window == int(kv["window"])
