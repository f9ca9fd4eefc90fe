"""Pins of the oracle's sparse + window attention (CPU only)."""
import numpy as np
import torch

from oracle import attention, codec, group, indexer


def _cache(rng, n, d):
    codes, scales = codec.fp4_encode(rng.standard_normal((n, d)).astype(np.float32))
    return codes, scales


def _swa(rng, n, d):
    return codec.fp8_rows_encode(rng.standard_normal((n, d)).astype(np.float32))


def test_full_topk_equals_dense_sdpa():
    rng = np.random.default_rng(21)
    n, d, h, w = 200, 64, 8, 16
    codes, scales = _cache(rng, n, d)
    sc, ss = _swa(rng, w, d)
    q = rng.standard_normal((h, d))
    tau = d ** -0.5
    idx = np.arange(n)
    o, lse = attention.sparse_swa_attention(q, codes, scales, idx, n, sc, ss, tau)
    keys = np.concatenate([codec.fp4_decode(codes, scales), codec.fp8_rows_decode(sc, ss)])
    qt = torch.from_numpy(q)[None, :, None, :]                     # [1, H, 1, D]
    kt = torch.from_numpy(keys)[None, None].expand(1, h, -1, -1)   # [1, H, n, D]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=tau)[0, :, 0].numpy()
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)
    z = tau * (q @ keys.T)
    assert np.allclose(lse, np.log(np.exp(z).sum(axis=1)), rtol=1e-12)


def test_lse_merge_of_selected_and_window_equals_joint():
    rng = np.random.default_rng(22)
    n, d, h = 300, 32, 4
    codes, scales = _cache(rng, n, d)
    sc, ss = _swa(rng, 20, d)
    q = rng.standard_normal((h, d)) * 3
    idx = np.sort(rng.choice(n, 40, replace=False))
    joint = attention.sparse_swa_attention(q, codes, scales, idx, n, sc, ss, 0.2)
    a = attention.sparse_swa_attention(q, codes, scales, idx, n, None, None, 0.2)
    b = attention.attend(q, codec.fp8_rows_decode(sc, ss), 0.2)
    o, lse = attention.lse_merge([a, b])
    assert np.allclose(o, joint[0], rtol=1e-12, atol=1e-13) and np.allclose(lse, joint[1], rtol=1e-13)


def test_index_order_invariance_and_skipped_entries():
    rng = np.random.default_rng(23)
    n, d, h = 100, 32, 3
    codes, scales = _cache(rng, n, d)
    sc, ss = _swa(rng, 5, d)
    q = rng.standard_normal((h, d))
    idx = np.array([5, 17, 50, 99])
    a = attention.sparse_swa_attention(q, codes, scales, idx, n, sc, ss, 0.3)
    b = attention.sparse_swa_attention(q, codes, scales, idx[::-1], n, sc, ss, 0.3)
    c = attention.sparse_swa_attention(q, codes, scales, np.array([-1, 5, 17, 120, 50, 99, -1]), n, sc, ss, 0.3)
    for x in (b, c):
        assert np.allclose(a[0], x[0], rtol=1e-13, atol=1e-14) and np.allclose(a[1], x[1], rtol=1e-13)
    # entries at or beyond the visible count are skipped
    d_ = attention.sparse_swa_attention(q, codes, scales, idx, 60, sc, ss, 0.3)
    e = attention.sparse_swa_attention(q, codes, scales, idx[:3], 100, sc, ss, 0.3)
    assert np.allclose(d_[0], e[0], rtol=1e-13, atol=1e-14)


def test_single_key_and_zero_query_and_empty():
    rng = np.random.default_rng(24)
    codes, scales = _cache(rng, 10, 16)
    q = rng.standard_normal((2, 16))
    o, lse = attention.sparse_swa_attention(q, codes, scales, [4], 10, None, None, 0.5)
    k = codec.fp4_decode(codes[4:5], scales[4:5])[0]
    assert np.array_equal(o, np.stack([k, k])) and np.allclose(lse, 0.5 * (q @ k))
    o, lse = attention.sparse_swa_attention(np.zeros((2, 16)), codes, scales, np.arange(10), 10, None, None, 0.5)
    assert np.allclose(o, codec.fp4_decode(codes, scales).mean(axis=0)[None, :].repeat(2, 0), rtol=1e-13)
    assert np.allclose(lse, np.log(10.0))
    o, lse = attention.sparse_swa_attention(q, codes, scales, [-1, -1], 10, None, None, 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_decoder_group_reuse_layers_share_list():
    rng = np.random.default_rng(25)
    n, d, di = 700, 64, 32
    codes, scales = _cache(rng, n, d)
    w_ik = (rng.standard_normal((d, di)) / np.sqrt(d)).astype(np.float32)
    ikc, iks = codec.indexer_key(codes, scales, w_ik)
    qi, wi = rng.standard_normal((2, di)), rng.standard_normal(2)
    layers = [(rng.standard_normal((4, d)),) + _swa(rng, 8, d) for _ in range(4)]
    res = group.decoder_group("full", codes, scales, ikc, iks, n - 1, 1, qi, wi, None, 16, 32, layers, d ** -0.5)
    keys = codec.fp4_decode(ikc, iks)
    pool, cnt, idx, _ = indexer.index_full(qi, wi, keys, 16, 32)
    assert np.array_equal(res["idx"], idx) and np.array_equal(res["pool"], pool)
    for (q, sc, ss), (o, lse) in zip(layers, res["out"]):
        ro, rl = attention.sparse_swa_attention(q, codes, scales, idx, n, sc, ss, d ** -0.5)
        assert np.array_equal(o, ro) and np.array_equal(lse, rl)
    res2 = group.decoder_group("reindex", codes, scales, ikc, iks, n - 1, 1, qi, wi, res["pool"], 16, 32, layers,
                               d ** -0.5)
    assert np.array_equal(res2["idx"], res["idx"])          # same query re-scored over its own pool
