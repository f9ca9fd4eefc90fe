"""GPU parity of the FP4 / FP8 codec and the indexer-key derivation (bit-exact)."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_02_amd as csa2
import synth
from oracle import codec
from tests._gpu_util import announce, dev, empty_u8, gpu_quantize, h, t

pytestmark = pytest.mark.gpu


def test_dequant_exhaustive_codes_and_scales():
    announce("dequant exhaustive")
    scale_bytes = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
    rows = len(scale_bytes)
    codes = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))          # dim 512: every code byte
    scales = np.repeat(scale_bytes[:, None], 32, axis=1)
    out = torch.empty((rows, 512), dtype=torch.float32, device=dev())
    csa2.csa2_dequant_fp4(t(codes), t(scales), out)
    got = h(out).astype(np.float64)
    ref = codec.fp4_decode(codes, scales)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def _adversarial_rows(dim=128):
    rng = np.random.default_rng(31)
    rows = []
    mids = (codec.E2M1_POS[:-1] + codec.E2M1_POS[1:]) / 2
    for sc in list(range(1, 127, 3)) + [1, 2, 7, 8, 9, 56, 125, 126]:
        s = codec.E4M3_POS[sc]
        g = []
        for _ in range(dim // 16):
            grp = np.zeros(16, np.float32)
            grp[0] = np.float32(6 * s)
            vals = np.float32(mids * s)
            pick = rng.permutation(np.concatenate([vals, np.nextafter(vals, np.float32(np.inf)),
                                                   np.nextafter(vals, np.float32(0))]))[:15]
            grp[1:] = pick * rng.choice([-1, 1], 15)
            g.append(grp)
        rows.append(np.concatenate(g))
    # scale ties: amax/6 exactly on an E4M3 midpoint, and just around it
    emids = (codec.E4M3_POS[:-1] + codec.E4M3_POS[1:]) / 2
    for i in range(0, 126, 5):
        a = np.float32(6 * emids[i])
        for v in (a, np.nextafter(a, np.float32(np.inf)), np.nextafter(a, np.float32(0))):
            r = (rng.standard_normal(dim) * float(v) / 8).astype(np.float32)
            r[::16] = v
            rows.append(r)
    special = np.zeros((8, dim), np.float32)
    special[1, 3] = -0.0
    special[2] = -0.0
    special[3] = np.float32(6 * 2.0 ** -10)              # scale rounds to 0
    special[4] = (rng.standard_normal(dim) * 1e5).astype(np.float32)   # scale saturates
    special[5] = (rng.standard_normal(dim) * 1e-8).astype(np.float32)
    special[6] = np.ldexp(rng.standard_normal(dim), rng.integers(20, 125, dim)).astype(np.float32)  # far beyond
    special[7, ::2] = np.finfo(np.float32).max
    special[7, 1::2] = -np.finfo(np.float32).max
    return np.concatenate([np.stack(rows), special]).astype(np.float32)


@pytest.mark.parametrize("dim", [128, 512])
def test_quantize_bit_exact_random_and_adversarial(dim):
    announce("quantize fp4", dim)
    rng = np.random.default_rng(32)
    x = np.concatenate([rng.standard_normal((3000, dim)).astype(np.float32), _adversarial_rows(dim)])
    codes, scales = gpu_quantize(x)
    rc, rs = codec.fp4_encode(x)
    assert np.array_equal(h(scales), rs)
    assert np.array_equal(h(codes), rc)


def test_quantize_bf16_input_and_scattered_rows():
    announce("quantize fp4 bf16 + dst_row")
    rng = np.random.default_rng(33)
    bits = synth.f32_to_bf16_bits(rng.standard_normal((257, 128)).astype(np.float32))
    xf = synth.bf16_bits_to_f32(bits)
    dst = rng.permutation(400)[:257].astype(np.int64)
    codes, scales = empty_u8(400, 64), empty_u8(400, 8)
    codes.zero_()
    scales.zero_()
    csa2.csa2_quantize_fp4(t(bits).view(torch.bfloat16), codes, scales, dst_row=t(dst))
    rc, rs = codec.fp4_encode(xf)
    gc, gs = h(codes), h(scales)
    assert np.array_equal(gc[dst], rc) and np.array_equal(gs[dst], rs)
    untouched = np.setdiff1d(np.arange(400), dst)
    assert np.all(gc[untouched] == 0) and np.all(gs[untouched] == 0)


@pytest.mark.parametrize("dim,di,rows", [(128, 64, 2000), (512, 128, 2000), (256, 256, 2000), (512, 128, 5),
                                         (512, 128, 1024), (128, 64, 3),
                                         (512, 32, 1500), (512, 64, 1500), (96, 32, 1100),
                                         (256, 256, 7), (512, 32, 9), (64, 32, 200), (192, 64, 333),
                                         (512, 128, 65), (512, 128, 4096)])
def test_derive_indexer_key_bit_exact(dim, di, rows):
    # dim <= 512 runs the fp64 matrix-core kernels: up to 64 rows with the
    # channels split over 8 waves per 16-column tile; more rows (dim a
    # multiple of 64) with 64 rows and one key group per workgroup, else
    # 16 rows and 1, 2, 4 or 8 key groups per workgroup (96 channels).
    # Every row count here leaves a ragged last tile or row quad.
    announce("derive indexer key", dim, di, rows)
    x = synth.main_kv_rows(0, 0, 0, rows, dim)
    w = synth.w_ik(0, dim, di)
    codes, scales, ikc, iks = gpu_quantize(x, w)
    rc, rs = codec.fp4_encode(x)
    assert np.array_equal(h(codes), rc) and np.array_equal(h(scales), rs)
    kc, ks = codec.indexer_key(rc, rs, w)
    assert np.array_equal(h(iks), ks)
    assert np.array_equal(h(ikc), kc)


def test_fp8_rows_bit_exact():
    announce("fp8 rows")
    rng = np.random.default_rng(34)
    x = np.concatenate([rng.standard_normal((300, 512)),
                        rng.standard_normal((5, 512)) * 1e-7,
                        rng.standard_normal((5, 512)) * 1e7,
                        np.zeros((2, 512))]).astype(np.float32)
    x[-1, 7] = -0.0
    codes = empty_u8(len(x), 512)
    scale = torch.empty(len(x), dtype=torch.float32, device=dev())
    csa2.csa2_quantize_fp8_rows(t(x), codes, scale)
    rc, rs = codec.fp8_rows_encode(x)
    assert np.array_equal(h(scale), rs)
    assert np.array_equal(h(codes), rc)


def test_quantize_full_cache_shape_sample():
    # 65,536 rows of the 512-channel latent (one 64K decoder cache), every row checked
    announce("quantize 64K x 512")
    x = synth.main_kv_rows(1, 0, 0, 65536, 512)
    codes, scales = gpu_quantize(x)
    rc, rs = codec.fp4_encode(x)
    assert np.array_equal(h(scales), rs)
    assert np.array_equal(h(codes), rc)


def test_derive_bf16_scattered_and_adversarial_rows():
    # the 64-row tiles with bf16 input, scattered destination rows and the
    # adversarial groups (saturating, subnormal-scale, exact-midpoint values)
    announce("derive bf16 + dst_row + adversarial")
    rng = np.random.default_rng(34)
    dim, di = 512, 128
    xf = np.concatenate([rng.standard_normal((300, dim)).astype(np.float32), _adversarial_rows(dim)])
    xf = np.clip(xf, -3.0e38, 3.0e38)          # finite in bf16
    bits = synth.f32_to_bf16_bits(xf).reshape(xf.shape)
    xb = synth.bf16_bits_to_f32(bits)
    n = xb.shape[0]
    dst = rng.permutation(2 * n)[:n].astype(np.int64)
    w = synth.w_ik(1, dim, di)
    codes, scales = empty_u8(2 * n, dim // 2), empty_u8(2 * n, dim // 16)
    ikc, iks = empty_u8(2 * n, di // 2), empty_u8(2 * n, di // 16)
    for z in (codes, scales, ikc, iks):
        z.fill_(0x5A)
    csa2.csa2_quantize_fp4(t(bits).view(torch.bfloat16), codes, scales, dst_row=t(dst),
                           w_ik=t(w.astype(np.float32)), ik_codes=ikc, ik_scales=iks)
    rc, rs = codec.fp4_encode(xb)
    kc, ks = codec.indexer_key(rc, rs, w)
    untouched = np.setdiff1d(np.arange(2 * n), dst)
    for got, want in ((codes, rc), (scales, rs), (ikc, kc), (iks, ks)):
        g = h(got)
        assert np.array_equal(g[dst], want)
        assert np.all(g[untouched] == 0x5A)
