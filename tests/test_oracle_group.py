"""Pins of the oracle's group composition (CPU only).

The indexer keys below are planted: every entry's key is zero except a few
entries whose channel 0 holds a chosen E2M1 value at unit scale, and the
indexer query is the unit vector of channel 0 with weight 1.  The score of an
entry is then the planted value itself (0 elsewhere), so the selected lists
are known by construction: the planted visible entries in value order, then
the lowest visible positions of the pool (ties go to the lower position).
Planted entries that the query token may not see yet carry the largest
values, so a visibility slip in the composition selects them.

The attention outputs of every layer are compared with torch's
scaled_dot_product_attention in fp64 over the rows the known list names plus
the layer's window rows.
"""
import numpy as np
import torch

from oracle import codec, group

E4M3_ONE = 0x38                       # E4M3FN code of 1.0
E2M1 = {6.0: 0x7, 4.0: 0x6, 3.0: 0x5, 2.0: 0x4}


def _planted_keys(n, di, planted):
    codes = np.zeros((n, di // 2), np.uint8)
    scales = np.full((n, di // 16), E4M3_ONE, np.uint8)
    for j, v in planted.items():
        codes[j, 0] = E2M1[v]         # channel 0 = low nibble of byte 0
    return codes, scales


def _unit_query(di):
    q = np.zeros((1, di))
    q[0, 0] = 1.0
    return q, np.array([1.0])


def _layers(rng, n_layers, h, d, w):
    out = []
    for _ in range(n_layers):
        q = rng.standard_normal((h, d))
        sc, ss = codec.fp8_rows_encode(rng.standard_normal((w, d)).astype(np.float32))
        out.append((q, sc, ss))
    return out


def _sdpa(q, rows, tau):
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.from_numpy(np.asarray(rows, np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=tau)[0, :, 0].numpy()


def _check_layers(res_out, layers, main_codes, main_scales, known_idx, tau):
    valid = [j for j in known_idx if j >= 0]
    main = codec.fp4_decode(main_codes[valid], main_scales[valid]) if valid else np.zeros((0, main_codes.shape[1] * 2))
    for (q, sc, ss), (o, lse) in zip(layers, res_out):
        rows = np.concatenate([main, codec.fp8_rows_decode(sc, ss)])
        assert np.allclose(o, _sdpa(q, rows, tau), rtol=1e-12, atol=1e-13)
        z = tau * (q @ rows.T)
        assert np.allclose(lse, np.log(np.exp(z).sum(axis=1)), rtol=1e-12)


def _main(rng, n, d):
    return codec.fp4_encode(rng.standard_normal((n, d)).astype(np.float32))


def test_decoder_group_full_before_last_token():
    """Full group at token t = 120 of a 200-entry cache (ratio 1): entries
    0..120 are visible; entries 121 and 199 score highest but lie ahead."""
    rng = np.random.default_rng(41)
    n, d, di, t, P, K = 200, 32, 16, 120, 4, 8
    ikc, iks = _planted_keys(n, di, {5: 4.0, 50: 3.0, 120: 2.0, 121: 6.0, 199: 6.0})
    mc, ms = _main(rng, n, d)
    layers = _layers(rng, 4, 4, d, 8)
    qi, wi = _unit_query(di)
    res = group.decoder_group("full", mc, ms, ikc, iks, t, 1, qi, wi, None, P, K, layers, d ** -0.5)
    # block maxima of the visible entries: block 0 -> 4, block 6 -> 3,
    # block 15 (only entry 120 visible) -> 2, every other block 0; the pool's
    # fourth block is the lowest zero block
    assert res["pool"].tolist() == [0, 1, 6, 15] and res["pool_count"] == 4
    known = [0, 1, 2, 3, 4, 5, 50, 120]
    assert res["idx"].tolist() == known
    _check_layers(res["out"], layers, mc, ms, known, d ** -0.5)


def test_decoder_group_reindex_before_last_token():
    """Reindex at t = 120 over a pool that holds a partly visible block (15:
    only entry 120 visible) and an invisible one (20)."""
    rng = np.random.default_rng(42)
    n, d, di, t, K = 200, 32, 16, 120, 3
    ikc, iks = _planted_keys(n, di, {5: 4.0, 120: 2.0, 121: 6.0, 160: 6.0})
    mc, ms = _main(rng, n, d)
    layers = _layers(rng, 2, 4, d, 8)
    qi, wi = _unit_query(di)
    res = group.decoder_group("reindex", mc, ms, ikc, iks, t, 1, qi, wi, np.array([0, 15, 20, -1]), 4, K, layers,
                              d ** -0.5)
    assert res["pool_count"] == 3
    known = [0, 5, 120]
    assert res["idx"].tolist() == known
    _check_layers(res["out"], layers, mc, ms, known, d ** -0.5)


def test_decoder_group_ratio2_token_inside_entry():
    """Ratio 2: token t = 62 sees entries 0..30 (entry 31 holds tokens 62 and
    63 and is not complete yet); token 63 sees entry 31 as well."""
    rng = np.random.default_rng(43)
    n, d, di, P, K = 64, 32, 16, 16, 3
    ikc, iks = _planted_keys(n, di, {31: 6.0, 30: 3.0, 10: 2.0, 40: 6.0})
    mc, ms = _main(rng, n, d)
    layers = _layers(rng, 2, 4, d, 8)
    qi, wi = _unit_query(di)
    for t, known in ((61, [0, 10, 30]), (62, [0, 10, 30]), (63, [10, 30, 31])):
        res = group.decoder_group("full", mc, ms, ikc, iks, t, 2, qi, wi, None, P, K, layers, d ** -0.5)
        assert res["idx"].tolist() == known, t
        _check_layers(res["out"], layers, mc, ms, known, d ** -0.5)


def test_encoder_group_query_ratio2_visibility():
    """Encoder group (Full + 5 Reuse, flat Top-K) at ratio 2 for chunk-internal
    tokens: every layer attends over the flat Top-K of the entries complete at
    its token, including the token-0 case with no visible entry."""
    rng = np.random.default_rng(44)
    n, d, di, K = 64, 32, 16, 3
    ikc, iks = _planted_keys(n, di, {31: 6.0, 30: 3.0, 10: 2.0, 40: 6.0, 63: 6.0})
    mc, ms = _main(rng, n, d)
    layers = _layers(rng, 6, 4, d, 8)
    qi, wi = _unit_query(di)
    cases = ((0, [-1, -1, -1]), (1, [0, -1, -1]), (2, [0, -1, -1]), (21, [0, 1, 10]), (61, [0, 10, 30]),
             (62, [0, 10, 30]), (63, [10, 30, 31]), (64, [10, 30, 31]), (81, [30, 31, 40]))
    for t, known in cases:
        res = group.encoder_group_query(mc, ms, ikc, iks, t, 2, qi, wi, K, layers, d ** -0.5)
        assert res["idx"].tolist() == known, t
        assert len(res["out"]) == 6
        _check_layers(res["out"], layers, mc, ms, known, d ** -0.5)


def test_encoder_group_query_no_entry_gives_window_only():
    rng = np.random.default_rng(45)
    n, d, di = 16, 32, 16
    ikc, iks = _planted_keys(n, di, {})
    mc, ms = _main(rng, n, d)
    layers = _layers(rng, 1, 2, d, 5)
    qi, wi = _unit_query(di)
    res = group.encoder_group_query(mc, ms, ikc, iks, 0, 2, qi, wi, 4, layers, d ** -0.5)
    q, sc, ss = layers[0]
    assert np.allclose(res["out"][0][0], _sdpa(q, codec.fp8_rows_decode(sc, ss), d ** -0.5), rtol=1e-12)
