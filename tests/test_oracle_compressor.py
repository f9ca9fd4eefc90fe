"""Pins of the compressor oracle (CPU only).

The compressor is a linear map of each entry's own r token rows with one
fp32 rounding of an exactly accumulated sum; these tests check it against
special weights with a known answer and against an exact-rational brute force
of the whole fused write (entry, FP4 codes, indexer key).
"""
from fractions import Fraction

import numpy as np

import synth
from oracle import codec, compressor
from tests import _exact


def _bf16_values(bits):
    return synth.bf16_bits_to_f32(bits)


def _tokens(n_tok, d_in, seed):
    x = np.random.default_rng(seed).standard_normal((n_tok, d_in)).astype(np.float32)
    return _bf16_values(synth.f32_to_bf16_bits(x).reshape(n_tok, d_in))


def test_selection_weights_return_even_and_odd_tokens():
    d = 64
    x = _tokens(2 * 9, d, 1)
    eye, zero = np.eye(d, dtype=np.float32), np.zeros((d, d), np.float32)
    even = compressor.compress_entries(x, np.concatenate([eye, zero], axis=1), 2)
    odd = compressor.compress_entries(x, np.concatenate([zero, eye], axis=1), 2)
    assert np.array_equal(even.view(np.uint32), (x[0::2] + np.float32(0)).view(np.uint32))
    assert np.array_equal(odd.view(np.uint32), (x[1::2] + np.float32(0)).view(np.uint32))


def test_half_half_weights_average_the_pair():
    d = 32
    x = _tokens(2 * 40, d, 2)
    x[5, :4] = 0.0           # zero pairs and exact cancellations
    x[4, :4] = 0.0
    x[7, 4:8] = -x[6, 4:8]
    half = np.float32(0.5) * np.eye(d, dtype=np.float32)
    got = compressor.compress_entries(x, np.concatenate([half, half], axis=1), 2)
    a, b = x[0::2].astype(np.float64), x[1::2].astype(np.float64)
    want = ((a + b) / 2).astype(np.float32)      # the sum of two bf16 values is exact in fp64
    assert np.array_equal(got, want)
    assert not np.signbit(got[got == 0]).any()   # zero sums are +0


def test_ratio_one_permutation_permutes_channels():
    d = 48
    x = _tokens(11, d, 3)
    perm = np.random.default_rng(3).permutation(d)
    w = np.zeros((d, d), np.float32)
    w[np.arange(d), perm] = 1.0                  # output c takes input perm[c]
    got = compressor.compress_entries(x, w, 1)
    assert np.array_equal(got, x[:, perm])


def test_entry_depends_only_on_its_own_tokens():
    d, r, n = 32, 2, 8
    x = _tokens(r * n, d, 4)
    w = _bf16_values(synth.w_c(0, 0, d, r, d))
    base = compressor.compress_entries(x, w, r)
    for tok in (0, 5, 2 * n - 1):
        y = x.copy()
        y[tok] = _tokens(1, d, 100 + tok)[0]
        got = compressor.compress_entries(y, w, r)
        j = tok // r
        others = np.arange(n) != j
        assert np.array_equal(got[others], base[others])
        assert not np.array_equal(got[j], base[j])


def _exact_fused(x, w_c, ratio, w_ik):
    """Brute force with exact rationals: entry, its FP4 codes, its indexer key."""
    n = x.shape[0] // ratio
    d_in = x.shape[1]
    dim = w_c.shape[0]
    di = w_ik.shape[1]
    concat = x.reshape(n, ratio * d_in)
    entries, codes, scales, kcodes, kscales = [], [], [], [], []
    for j in range(n):
        xf = [Fraction(float(v)) for v in concat[j]]
        c = [_exact.fraction_to_f32(sum(xf[k] * Fraction(float(w_c[o, k])) for k in range(ratio * d_in)))
             for o in range(dim)]
        entries.append(c)
        row_codes, row_scales, dq = [], [], []
        for g in range(dim // 16):
            cs, sc = _exact.fp4_group(c[16 * g:16 * g + 16])
            row_codes += cs
            row_scales.append(sc)
            s = _exact.E4M3_POS_FR[sc]
            dq += [(-1 if cc & 8 else 1) * _exact.E2M1_POS_FR[cc & 7] * s for cc in cs]
        codes.append(row_codes)
        scales.append(row_scales)
        key = [_exact.fraction_to_f32(sum(dq[i] * Fraction(float(w_ik[i, o])) for i in range(dim)))
               for o in range(di)]
        krow, kscale = [], []
        for g in range(di // 16):
            cs, sc = _exact.fp4_group(key[16 * g:16 * g + 16])
            krow += cs
            kscale.append(sc)
        kcodes.append(krow)
        kscales.append(kscale)

    def pack(rows):
        a = np.array(rows, dtype=np.uint8)
        return (a[:, 0::2] | (a[:, 1::2] << 4)).astype(np.uint8)

    return (np.array(entries, np.float32), pack(codes), np.array(scales, np.uint8), pack(kcodes),
            np.array(kscales, np.uint8))


def test_fused_write_against_exact_bruteforce():
    ratio, d_in, dim, di, n = 2, 16, 32, 16, 4
    x = _tokens(ratio * n, d_in, 5)
    x[3] = -x[2]                     # with identity-like weights this row would cancel
    x[6, :8] = 0.0
    w_c = _bf16_values(synth.w_c(0, 1, dim, ratio, d_in))
    w_c[:, :4] *= np.float32(64.0)   # a wide spread of magnitudes inside each sum
    w_ik = synth.w_ik(0, dim, di)
    e, c, s, kc, ks = _exact_fused(x, w_c, ratio, w_ik)
    got_e = compressor.compress_entries(x, w_c, ratio)
    assert np.array_equal(got_e.view(np.uint32), e.view(np.uint32))
    gc, gs, gkc, gks = compressor.compress_write(x, w_c, ratio, w_ik)
    assert np.array_equal(gc, c) and np.array_equal(gs, s)
    assert np.array_equal(gkc, kc) and np.array_equal(gks, ks)


def test_cancelling_pair_gives_positive_zero_codes():
    d = 32
    x = _tokens(2 * 3, d, 6)
    x[1::2] = -x[0::2]
    eye = np.eye(d, dtype=np.float32)
    w_ik = np.ones((d, 16), np.float32)
    codes, scales, kc, ks = compressor.compress_write(x, np.concatenate([eye, eye], axis=1), 2, w_ik)
    assert not codes.any() and not scales.any()   # +0 everywhere: no sign bits
    assert not kc.any() and not ks.any()
    assert np.array_equal(codec.fp4_decode(codes, scales), np.zeros((3, d)))
