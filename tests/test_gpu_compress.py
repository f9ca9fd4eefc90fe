"""GPU parity of the compressor fused with the FP4 write and the indexer keys (bit-exact)."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_02_amd as csa2
import synth
from oracle import compressor
from tests._gpu_util import announce, dev, empty_u8, h, t

pytestmark = pytest.mark.gpu


def _inputs(cfg, entries, ratio, d_in, dim, di):
    tok_bits = synth.token_rows(cfg, 0, 0, 0, entries * ratio, d_in)
    wc_bits = synth.w_c(cfg, 0, dim, ratio, d_in)
    w_ik = synth.w_ik(cfg, dim, di) if di else None
    return tok_bits, wc_bits, w_ik


def _gpu(tok_bits, wc_bits, ratio, w_ik, rows=None, dst=None, fill=None):
    entries = tok_bits.shape[0] // ratio
    dim = wc_bits.shape[0]
    rows = entries if rows is None else rows
    codes, scales = empty_u8(rows, dim // 2), empty_u8(rows, dim // 16)
    ikc = iks = None
    if w_ik is not None:
        di = w_ik.shape[1]
        ikc, iks = empty_u8(rows, di // 2), empty_u8(rows, di // 16)
    if fill is not None:
        for x in (codes, scales, ikc, iks):
            if x is not None:
                x.fill_(fill)
    csa2.csa2_compress_fp4(t(tok_bits), ratio, t(wc_bits), codes, scales,
                           dst_row=None if dst is None else t(dst.astype(np.int64)),
                           w_ik=None if w_ik is None else t(w_ik.astype(np.float32)), ik_codes=ikc, ik_scales=iks)
    return codes, scales, ikc, iks


def _oracle(tok_bits, wc_bits, ratio, w_ik):
    x = synth.bf16_bits_to_f32(tok_bits)
    w = synth.bf16_bits_to_f32(wc_bits)
    if w_ik is None:
        from oracle import codec
        return codec.fp4_encode(compressor.compress_entries(x, w, ratio)) + (None, None)
    return compressor.compress_write(x, w, ratio, w_ik)


# entries, ratio, d_in, dim, idx_dim
CASES = [
    (2048, 2, 512, 512, 128),    # the 4,096-token prefill chunk's entries at ratio 2
    (4, 2, 512, 512, 128),       # a decode step's completed entries (few-entry schedule)
    (37, 2, 512, 512, 128),      # ragged 16-entry tile, few-entry schedule
    (100, 2, 512, 512, 128),     # ragged tile, many-entry schedule
    (65, 1, 512, 512, 128),      # ratio 1 (a per-token linear map)
    (50, 3, 96, 96, 32),         # 6 FP4 groups (2 per workgroup), K = 288: one wave per workgroup
    (16, 2, 32, 32, 32),         # K = 64: two waves
    (300, 4, 128, 256, 64),      # K = 512
    (3, 16, 1024, 512, 256),     # K = 16384, the largest
]


@pytest.mark.parametrize("entries,ratio,d_in,dim,di", CASES)
def test_compress_write_bit_exact(entries, ratio, d_in, dim, di):
    announce("compress", entries, ratio, d_in, dim, di)
    tok, wc, w_ik = _inputs(0, entries, ratio, d_in, dim, di)
    codes, scales, ikc, iks = _gpu(tok, wc, ratio, w_ik)
    rc, rs, rkc, rks = _oracle(tok, wc, ratio, w_ik)
    assert np.array_equal(h(scales), rs)
    assert np.array_equal(h(codes), rc)
    assert np.array_equal(h(iks), rks)
    assert np.array_equal(h(ikc), rkc)


def test_compress_without_keys_and_scattered_rows():
    announce("compress scattered rows")
    entries, ratio, d_in, dim, di = 45, 2, 256, 512, 128
    tok, wc, w_ik = _inputs(1, entries, ratio, d_in, dim, di)
    dst = np.random.default_rng(9).permutation(300)[:entries]
    codes, scales, ikc, iks = _gpu(tok, wc, ratio, w_ik, rows=300, dst=dst, fill=0xA5)
    rc, rs, rkc, rks = _oracle(tok, wc, ratio, w_ik)
    for got, want in ((codes, rc), (scales, rs), (ikc, rkc), (iks, rks)):
        g = h(got)
        assert np.array_equal(g[dst], want)
        untouched = np.setdiff1d(np.arange(300), dst)
        assert np.all(g[untouched] == 0xA5)
    codes, scales, ikc, iks = _gpu(tok, wc, ratio, None)
    assert ikc is None
    rc, rs, _, _ = _oracle(tok, wc, ratio, None)
    assert np.array_equal(h(codes), rc) and np.array_equal(h(scales), rs)


def test_compress_special_weights_and_cancelling_pairs():
    # selection weights return the token rows themselves; a pair that cancels
    # under [I I] writes +0 codes; a huge weight column saturates the scales
    announce("compress special weights")
    d = 128
    tok = synth.token_rows(2, 0, 0, 0, 2 * 40, d)
    x = synth.bf16_bits_to_f32(tok)
    x[1::2][:10] = -x[0::2][:10]
    tok = synth.f32_to_bf16_bits(x).reshape(x.shape)
    eye = np.eye(d, dtype=np.float32)
    for w in (np.concatenate([eye, 0 * eye], axis=1), np.concatenate([eye, eye], axis=1),
              np.concatenate([eye * np.float32(2.0 ** 100), eye], axis=1)):
        wc = synth.f32_to_bf16_bits(w).reshape(w.shape)
        w_ik = synth.w_ik(2, d, 64)
        codes, scales, ikc, iks = _gpu(tok, wc, 2, w_ik)
        rc, rs, rkc, rks = _oracle(tok, wc, 2, w_ik)
        assert np.array_equal(h(codes), rc) and np.array_equal(h(scales), rs)
        assert np.array_equal(h(ikc), rkc) and np.array_equal(h(iks), rks)


def test_compress_deterministic_and_stream_ordered():
    announce("compress determinism")
    tok, wc, w_ik = _inputs(3, 512, 2, 512, 512, 128)
    a = [h(x) for x in _gpu(tok, wc, 2, w_ik)]
    s = torch.cuda.Stream(device=dev())
    with torch.cuda.stream(s):
        b = [x for x in _gpu(tok, wc, 2, w_ik)]
    s.synchronize()
    for x, y in zip(a, b):
        assert np.array_equal(x, h(y))
