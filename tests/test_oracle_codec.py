"""Pins of the oracle codec against the format definitions (CPU only)."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codec
from tests import _exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    raw = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = raw.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codec.E4M3_VALUES
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], ours[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(ours[ok]))


def test_e4m3_special_golden():
    for code, val in _read_table("e4m3_special.txt"):
        v = codec.E4M3_VALUES[int(code, 16)]
        if val == "nan":
            assert np.isnan(v)
        else:
            assert v == float(val) and np.signbit(v) == val.startswith("-")


def test_e2m1_grid_golden():
    table = _read_table("e2m1_grid.txt")
    assert len(table) == 16
    for code, val in table:
        v = codec.E2M1_VALUES[int(code, 16)]
        assert v == float(val) and np.signbit(v) == val.startswith("-")


def _interesting_f32(rng, n):
    parts = [
        rng.standard_normal(n).astype(np.float32),
        (rng.standard_normal(n) * 1e-3).astype(np.float32),
        (rng.standard_normal(n) * 300).astype(np.float32),
        (rng.standard_normal(n) * 1e4).astype(np.float32),
        np.ldexp(rng.random(n), rng.integers(-16, 12, n)).astype(np.float32),
        # far beyond the grid: saturation
        np.ldexp(rng.random(n) + 0.5, rng.integers(12, 127, n)).astype(np.float32),
        np.array([np.finfo(np.float32).max, 2.0 ** 100, 449.0, 464.0, 465.0], np.float32),
    ]
    mids = (codec.E4M3_POS[:-1] + codec.E4M3_POS[1:]) / 2
    m32 = mids.astype(np.float32)
    parts += [m32, np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(0))]
    return np.concatenate(parts).astype(np.float32)


def test_e4m3_encode_against_exact_bruteforce():
    rng = np.random.default_rng(1)
    x = _interesting_f32(rng, 300)
    x = np.concatenate([x, -x[:200]])
    for den in (1, 6):
        ours = codec.e4m3_nearest(x, float(den))
        for xi, oi in zip(x, ours):
            ref = _exact.e4m3_code(abs(Fraction(float(xi))) / den, bool(np.signbit(xi)))
            assert oi == ref, (xi, den, hex(oi), hex(ref))


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    x = _interesting_f32(rng, 20000)
    x = x[np.abs(x) <= 448].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codec.e4m3_nearest(x), ref)


def test_fp4_pack_golden():
    with open(os.path.join(GOLDEN, "fp4_pack_example.txt")) as f:
        lines = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(lines) == 6
    for ln in lines:
        name, xs, packed, scale = [p.strip() for p in ln.split("|")]
        x = np.array([float(v) for v in xs.split()], dtype=np.float32)[None, :]
        codes, scales = codec.fp4_encode(x)
        assert codes[0].tolist() == [int(b, 16) for b in packed.split()], name
        assert scales[0].tolist() == [int(scale, 16)], name


def test_fp4_value_roundtrip_every_code_and_scale():
    # groups whose amax is 6*s re-encode to exactly (codes, s)
    all_codes = np.arange(16)
    for sc in range(1, 127):
        s = codec.E4M3_POS[sc]
        for rest in (all_codes[:15], all_codes[1:]):
            codes = np.concatenate([[7], rest]).astype(np.int64)
            x = (codec.E2M1_VALUES[codes] * s).astype(np.float32)[None, :]
            assert np.array_equal(x.astype(np.float64)[0], codec.E2M1_VALUES[codes] * s)  # exact in fp32
            packed, scales = codec.fp4_encode(x)
            assert scales[0, 0] == sc
            assert np.array_equal(codec.fp4_unpack(packed)[0], codes)
            assert np.array_equal(codec.fp4_decode(packed, scales)[0], codec.E2M1_VALUES[codes] * s)


def test_fp4_tie_rule_at_every_midpoint():
    mids = (codec.E2M1_POS[:-1] + codec.E2M1_POS[1:]) / 2        # 0.25 .. 5
    rng = np.random.default_rng(3)
    for sc in rng.choice(np.arange(1, 127), 40, replace=False).tolist() + [1, 8, 56, 126]:
        s = codec.E4M3_POS[sc]
        for m in mids:
            t = np.float32(m * s)
            assert float(t) == m * s                               # midpoint exact in fp32
            for v in (t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(0))):
                row = np.zeros(16, np.float32)
                row[0] = np.float32(6 * s)
                row[1] = v
                row[2] = -v
                packed, scales = codec.fp4_encode(row[None, :])
                got = codec.fp4_unpack(packed)[0][:3].tolist()
                ref, rsc = _exact.fp4_group(row)
                assert rsc == sc and got == ref[:3], (sc, m, v, got, ref[:3])


def test_fp4_random_rows_against_exact_bruteforce():
    rng = np.random.default_rng(4)
    rows = [rng.standard_normal(64).astype(np.float32),
            (rng.standard_normal(64) * 1e-4).astype(np.float32),
            (rng.standard_normal(64) * 5e3).astype(np.float32),
            np.ldexp(rng.standard_normal(64), rng.integers(-20, 10, 64)).astype(np.float32),
            # groups whose amax / 6 is far beyond the largest scale (saturating scale and codes)
            np.ldexp(rng.standard_normal(64), rng.integers(20, 125, 64)).astype(np.float32),
            np.concatenate([np.full(16, np.finfo(np.float32).max), np.full(16, -1e30),
                            (rng.standard_normal(16) * 1e25), (rng.standard_normal(16) * 3000)]).astype(np.float32)]
    x = np.stack(rows)
    x[1, 5] = -0.0
    x[2, 16:32] = 0.0
    packed, scales = codec.fp4_encode(x)
    codes = codec.fp4_unpack(packed)
    for r in range(x.shape[0]):
        for g in range(4):
            ref, rsc = _exact.fp4_group(x[r, 16 * g:16 * g + 16])
            assert scales[r, g] == rsc
            assert codes[r, 16 * g:16 * g + 16].tolist() == ref


def test_fp4_decode_exact_in_fp16_and_bf16():
    # every code x finite scale product is representable in fp16 and bf16
    prod = (codec.E2M1_POS[1:, None] * codec.E4M3_POS[None, 1:]).reshape(-1)
    assert np.array_equal(prod.astype(np.float16).astype(np.float64), prod)
    bf = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf, prod)


def test_byte_accounting():
    assert codec.fp4_row_bytes(512) == 288
    assert codec.fp4_row_bytes(512) * (1 << 20) == 288 * (1 << 20)       # 288 MiB per 1M entries
    assert codec.fp4_row_bytes(128) == 72
    assert codec.fp4_row_bytes(64) == 36


def test_fp8_rows_against_exact_bruteforce():
    rng = np.random.default_rng(5)
    x = np.stack([rng.standard_normal(32).astype(np.float32),
                  (rng.standard_normal(32) * 1e-6).astype(np.float32),
                  (rng.standard_normal(32) * 1e6).astype(np.float32),
                  np.zeros(32, np.float32)])
    x[3, 3] = -0.0
    codes, scale = codec.fp8_rows_encode(x)
    for r in range(x.shape[0]):
        ref_codes, ref_scale = _exact.fp8_row(x[r])
        assert float(scale[r]) == ref_scale
        assert codes[r].tolist() == ref_codes
    dq = codec.fp8_rows_decode(codes, scale)
    assert np.array_equal(dq, codec.E4M3_VALUES[codes] * scale.astype(np.float64)[:, None])
    # row scale maps the row max to (about) 448
    assert np.all(np.abs(dq[:3]).max(axis=1) <= 448 * scale[:3].astype(np.float64) * (1 + 1e-6))


def test_indexer_key_with_channel_selection_matrix():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((20, 128)).astype(np.float32)
    codes, scales = codec.fp4_encode(x)
    sel = rng.permutation(128)[:64]
    w = np.zeros((128, 64), np.float32)
    w[sel, np.arange(64)] = 1.0
    kc, ks = codec.indexer_key(codes, scales, w)
    dq = (codec.fp4_decode(codes, scales)[:, sel] + 0.0).astype(np.float32)   # zero sums are +0
    rc, rs = codec.fp4_encode(dq)
    assert np.array_equal(kc, rc) and np.array_equal(ks, rs)


def test_indexer_projection_single_rounding():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 32)).astype(np.float32)
    codes, scales = codec.fp4_encode(x)
    w = rng.standard_normal((32, 5)).astype(np.float32)
    got = codec.project_indexer_key(codes, scales, w)
    dq = codec.fp4_decode(codes, scales)
    for r in range(3):
        for c in range(5):
            exact = sum(Fraction(float(dq[r, i])) * Fraction(float(w[i, c])) for i in range(32))
            assert float(got[r, c]) == _exact.fraction_to_f32(exact)
