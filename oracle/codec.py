"""Oracle: FP4 main-KV codec, FP8 window rows, indexer-key derivation.

Test infrastructure only (see ``oracle/__init__``).

What the pages fix (P1 section "FP4 KV、Bounded Replay 及其他扩展"; P4 section
三 "FP4 与部署侧的两个数字池"; P5 section "缓存精度与持久化分层"): the main
global KV is stored as E2M1 values with one E4M3 scale for every 16 channels,
the NVFP4 layout minus its second-level (global) scale; the sliding-window KV
stays in FP8.  The pages do not print the grids, the rounding rule, the nibble
order or the window-row scaling; the readings taken here are:

* E4M3 is the OCP "E4M3FN" variant: bias 7, no infinities, 0x7F/0xFF are NaN,
  largest finite 448, smallest subnormal 2^-9.
* E2M1 magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3.
* group scale s = the E4M3 value nearest to the exact quotient amax/6 (ties to
  the even code, finite values only, so it saturates at 448);
* each element code = the E2M1 value nearest to the exact quotient |x|/s
  (ties to the even code, saturating at 6), with the sign bit of x kept
  (-0 encodes as 0x8); s = 0 gives magnitude 0 everywhere;
* byte k of a row holds channel 2k in its low nibble and 2k+1 in its high
  nibble; scale byte g covers channels 16g..16g+15;
* a window row is stored as E4M3 codes of fp32(x / r) with one fp32 scale
  r = fp32(amax / 448) per row (r = 1 for an all-zero row), both divisions
  correctly rounded in fp32, codes ties-to-even and saturating;
* the indexer key of an entry is the FP4 encoding of fp32(W_ik^T DQ4(row)),
  the product taken in fp64 and rounded once to fp32 (P4 section 二 and P5
  section "CSA2注意力" say the indexer key is projected from the main-KV
  entry; its format is not given, so it reuses this FP4 codec).

"Nearest to the exact quotient" is evaluated without dividing: below the top
of the grid, |a - 6 v| and ||x| - g s| are exact in fp64 wherever the choice
depends on them (all operands are fp32 numbers and 6 v, g s have at most 7
significant bits); at or beyond the top (a >= 6 * 448, |x| >= 6 s) the
largest grid value is taken directly, since there the fp64 distances of huge
inputs can round to one value.

Parity pins (tests/test_oracle_codec.py): decode table against torch's
float8_e4m3fn; encode against an exact-rational brute force; E2M1 grid and the
packing fixture under tests/golden; value round-trip for every code x scale;
tie rule at every midpoint and its fp32 neighbours; byte accounting.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# E4M3FN
# ---------------------------------------------------------------------------


def _e4m3_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for b in range(256):
        sign = -1.0 if b & 0x80 else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            vals[b] = np.nan
        elif e == 0:
            vals[b] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[b] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()
#: non-negative finite E4M3 values; index == code (0x00 .. 0x7E), ascending
E4M3_POS = E4M3_VALUES[:127].copy()
E4M3_MAX = 448.0

#: E2M1 magnitudes; index == 3-bit magnitude code
E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_VALUES = np.concatenate([E2M1_POS, -E2M1_POS])


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def _nearest_index(num_abs: np.ndarray, den: np.ndarray | float, grid: np.ndarray) -> np.ndarray:
    """Index k of grid[k]*den nearest to num_abs; on a tie the even index.

    ``num_abs`` >= 0 (fp64 holding fp32 values), ``den`` >= 0 broadcastable
    to it, ``grid`` ascending.  Processed in slices to bound memory.
    """
    num_abs = np.asarray(num_abs, dtype=np.float64)
    den = np.broadcast_to(np.asarray(den, dtype=np.float64), num_abs.shape)
    flat_n = num_abs.reshape(-1)
    flat_d = den.reshape(-1)
    out = np.empty(flat_n.shape, dtype=np.int64)
    step = max(1, (1 << 22) // len(grid))
    for lo in range(0, flat_n.size, step):
        n = flat_n[lo:lo + step, None]
        top = flat_d[lo:lo + step] * grid[-1]
        d = np.abs(n - flat_d[lo:lo + step, None] * grid[None, :])
        best = d.min(axis=1, keepdims=True)
        hit = d == best
        first = hit.argmax(axis=1)
        nxt = np.minimum(first + 1, len(grid) - 1)
        tie = hit[np.arange(hit.shape[0]), nxt] & (nxt != first)
        near = np.where(tie & (first % 2 == 1), nxt, first)
        # at or beyond the top of the grid the largest value is nearest
        # (saturation); taken explicitly, since for huge inputs the fp64
        # distances to all candidates round to one value
        out[lo:lo + step] = np.where(n[:, 0] >= top, len(grid) - 1, near)
    return out.reshape(num_abs.shape)


def e4m3_nearest(num: np.ndarray, den: float = 1.0) -> np.ndarray:
    """E4M3FN code of the finite value nearest to num/den, ties to even code.

    ``num`` holds fp32 values (any float dtype), ``den`` > 0 exact.  Values
    beyond 448 saturate to the largest finite code; the sign bit is copied
    from ``num`` (so -0.0 gives 0x80).
    """
    num = np.asarray(num, dtype=np.float64)
    mag = _nearest_index(np.abs(num), den, E4M3_POS).astype(np.uint8)
    return (mag | (np.signbit(num).astype(np.uint8) << 7)).astype(np.uint8)


# ---------------------------------------------------------------------------
# FP4 main-KV rows
# ---------------------------------------------------------------------------

GROUP = 16


def fp4_encode(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Encode fp32 rows [R, D] (D % 16 == 0) into (codes u8 [R, D/2], scales u8 [R, D/16])."""
    x = np.asarray(x, dtype=np.float32)
    assert x.ndim == 2 and x.shape[1] % GROUP == 0
    rows, dim = x.shape
    g = x.reshape(rows, dim // GROUP, GROUP).astype(np.float64)
    amax = np.abs(g).max(axis=2)
    scale_code = e4m3_nearest(amax, 6.0)                 # amax >= 0, sign bit 0
    s = E4M3_VALUES[scale_code]                           # [R, G]
    mag = _nearest_index(np.abs(g), s[:, :, None], E2M1_POS)
    mag = np.where(s[:, :, None] == 0.0, 0, mag)
    code = (mag | (np.signbit(g).astype(np.int64) << 3)).reshape(rows, dim)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale_code.astype(np.uint8)


def fp4_unpack(codes: np.ndarray) -> np.ndarray:
    """Packed bytes [R, D/2] -> 4-bit codes [R, D] (channel 2k = low nibble)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def fp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """DQ4: exact fp64 values e2m1(code) * e4m3(scale) of rows [R, D]."""
    c = fp4_unpack(codes)
    rows, dim = c.shape
    s = e4m3_decode(scales)                               # [R, D/16]
    v = E2M1_VALUES[c].reshape(rows, dim // GROUP, GROUP) * s[:, :, None]
    return v.reshape(rows, dim)


def fp4_row_bytes(dim: int) -> int:
    return dim // 2 + dim // GROUP


# ---------------------------------------------------------------------------
# FP8 sliding-window rows
# ---------------------------------------------------------------------------


def fp8_rows_encode(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Encode fp32 rows [R, D] into (E4M3 codes u8 [R, D], fp32 row scale [R])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    r = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    r = np.where(amax == 0, np.float32(1.0), r).astype(np.float32)
    y = (x / r[:, None]).astype(np.float32)               # fp32 division, correctly rounded
    return e4m3_nearest(y), r


def fp8_rows_decode(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """DQ8: fp64 values e4m3(code) * row_scale."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[:, None]


# ---------------------------------------------------------------------------
# indexer key derived from the main-KV entry
# ---------------------------------------------------------------------------


def project_indexer_key(codes: np.ndarray, scales: np.ndarray, w_ik: np.ndarray) -> np.ndarray:
    """fp32(DQ4(row) @ W_ik), product in fp64, one rounding to fp32.

    A sum that is exactly zero is +0 (the sum starts from +0), so a -0 input
    channel never yields a -0 key channel.
    """
    dq = fp4_decode(codes, scales)
    return ((dq @ np.asarray(w_ik, dtype=np.float64)) + 0.0).astype(np.float32)


def indexer_key(codes: np.ndarray, scales: np.ndarray, w_ik: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """FP4-encoded indexer key of main-KV rows: Q4(fp32(W_ik^T DQ4(row)))."""
    return fp4_encode(project_indexer_key(codes, scales, w_ik))
