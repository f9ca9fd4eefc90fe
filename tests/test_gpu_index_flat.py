"""GPU parity of the flat (prefill) Top-K indexer, csa2_index_full with pool_blocks = 0, against the oracle."""
import numpy as np
import pytest
import torch

import fp4_kv_cache_02_amd as csa2
import synth
from oracle import codec, indexer
from tests._gpu_util import announce, assert_sets_equal_modulo_band, dev, gpu_quantize, h, t, workspace

pytestmark = pytest.mark.gpu


def _quantized_cache(cfg, lens, di):
    """Ragged cache: GPU and oracle each quantise the same raw rows (bytes compared)."""
    x = np.concatenate([synth.gaussian_rows(cfg, synth.TAG_IDX_KEY, 0, s, 0, n, di) for s, n in enumerate(lens)])
    codes, scales = gpu_quantize(x)
    rc, rs = codec.fp4_encode(x)
    assert np.array_equal(h(codes), rc) and np.array_equal(h(scales), rs)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return codes, scales, rc, rs, starts


def _run_flat(codes, scales, starts, lens, di, q_seq, q_pos, qi, wi, K, ratio):
    M = len(q_seq)
    cache = csa2.fp4_cache(codes, scales, t(starts), t(np.asarray(lens, np.int32)), di, max(lens), ratio)
    qs = csa2.queries(t(np.asarray(q_seq, np.int32)), t(np.asarray(q_pos, np.int32)))
    ws = workspace(csa2.csa2_index_workspace_size(cache, M, 0, K))
    topk = torch.full((M, K), -7, dtype=torch.int32, device=dev())
    sc = torch.full((M, K), -7.0, dtype=torch.float32, device=dev())
    csa2.csa2_index_full(cache, qs, t(qi).view(torch.bfloat16), t(wi), 0, K, None, None, topk, sc, ws)
    return h(topk), h(sc)


def _check_flat(keys_vis, qf, w, K, gtopk, gscore):
    """One query: the GPU list against the oracle's flat Top-K over every visible position."""
    otopk, s = indexer.index_flat(qf, w, keys_vis, K)
    sel = gtopk[gtopk >= 0]
    nsel = int((otopk >= 0).sum())
    assert nsel == min(K, len(s))
    assert len(sel) == nsel and np.all(gtopk[nsel:] == -1) and np.all(np.diff(sel) > 0)
    assert_sets_equal_modulo_band(sel, otopk[otopk >= 0], lambda j: s[j], K, what="flat")
    if nsel:
        tol = 1e-5 * max(1.0, np.abs(s).max())
        err = np.abs(gscore[:nsel] - s[sel])
        assert np.all(err <= tol), err.max()
    assert np.all(np.isnan(gscore[nsel:]))


CASES = {
    # name: (lens, di, H, K, ratio, q_seq, q_pos)
    # a chunk of 40 causal queries at the end of a 4K context (not a multiple of the 16-query tile)
    "c0_chunk": ([4096], 64, 4, 64, 1, [0] * 40, list(range(4056, 4096))),
    # ratio 2: query t sees floor((t + 1) / 2) entries
    "c2_small": ([3000], 128, 8, 100, 2, [0] * 50, list(range(5950, 6000))),
    # queries of several sequences in one workgroup, one query that sees nothing
    "mixed_seqs": ([1, 7, 64, 513, 2000, 9], 128, 8, 32, 2,
                   [4, 0, 3, 4, 2, 1, 5, 4, 3, 0, 4, 2, 3, 4, 1, 5, 4, 4],
                   [3999, 0, 1025, 2500, 127, 13, 17, 3998, 600, 1, 77, 100, 1024, 3, 5, 2, 1999, 4000]),
    # 12 heads: queries take 16 rows
    "wide_heads": ([2500], 128, 12, 64, 1, [0] * 20, list(range(2480, 2500))),
    "di256_h8": ([1500], 256, 8, 50, 1, [0] * 12, list(range(1400, 1500, 9))[:12]),
    "di256_h16": ([1500], 256, 16, 50, 1, [0] * 6, [1499, 1200, 999, 700, 33, 8]),
    "di64_h16": ([900], 64, 16, 40, 1, [0] * 9, [899, 898, 500, 300, 200, 100, 64, 15, 0]),
    # K above the visible counts: every visible position is selected
    "k_exceeds": ([300], 128, 8, 512, 1, [0] * 17, list(range(0, 300, 18))[:17]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_index_flat_matches_oracle(case):
    lens, di, H, K, ratio, q_seq, q_pos = CASES[case]
    announce("index_flat", case)
    cfg = 300 + list(CASES).index(case)
    codes, scales, rc, rs, starts = _quantized_cache(cfg, lens, di)
    M = len(q_seq)
    qi, wi = synth.q_idx(cfg, 0, M, H, di), synth.w_idx(cfg, 0, M, H)
    gtopk, gsc = _run_flat(codes, scales, starts, lens, di, q_seq, q_pos, qi, wi, K, ratio)
    qf = synth.bf16_bits_to_f32(qi)
    for i in range(M):
        s_ = q_seq[i]
        vis = indexer.visible_count(lens[s_], q_pos[i], ratio)
        keys = codec.fp4_decode(rc[starts[s_]:starts[s_] + vis], rs[starts[s_]:starts[s_] + vis])
        _check_flat(keys, qf[i], wi[i], K, gtopk[i], gsc[i])


def test_index_flat_ties_take_lowest_positions():
    announce("index_flat ties")
    lens, di, H, K = [1000], 128, 8, 64
    codes, scales, rc, rs, starts = _quantized_cache(320, lens, di)
    M = 20
    qi = synth.q_idx(320, 0, M, H, di)
    wi = np.zeros((M, H), np.float32)  # every score is exactly 0
    q_pos = list(range(980, 1000))
    gtopk, gsc = _run_flat(codes, scales, starts, lens, di, [0] * M, q_pos, qi, wi, K, 1)
    for i in range(M):
        assert gtopk[i].tolist() == list(range(K))
        assert np.all(gsc[i] == 0)


def test_index_flat_prefill_chunk_full_size_sampled():
    """A 4,096-query prefill chunk over 65,536 entries at ratio 2 (tokens
    126,976 .. 131,071 of a 131,072-token prompt), 8 heads x 128 dims, Top-512,
    in one call.  Raw cache bytes come from the seeded byte generator; 256
    queries (the first, the last and 254 drawn at random, spanning the chunk's
    visible counts 63,488 .. 65,536) are checked against the oracle's flat
    Top-K over every visible entry, every query against the structural
    properties."""
    announce("index_flat prefill 4096 x 65536")
    cfg, n, di, H, K, ratio, M = 330, 65536, 128, 8, 512, 2, 4096
    rc, rs = synth.fp4_bytes(cfg, 0, n, di)
    starts = np.zeros(1, np.int64)
    q_pos = np.arange(131072 - M, 131072, dtype=np.int32)
    qi, wi = synth.q_idx(cfg, 0, M, H, di), synth.w_idx(cfg, 0, M, H)
    gtopk, gsc = _run_flat(t(rc), t(rs), starts, [n], di, [0] * M, q_pos.tolist(), qi, wi, K, ratio)
    vis = np.minimum(n, (q_pos.astype(np.int64) + 1) // ratio)
    sel_ok = gtopk >= 0
    assert np.all(sel_ok.sum(1) == K)
    assert np.all(np.diff(gtopk, axis=1) > 0)
    assert np.all(gtopk < vis[:, None])
    assert not np.isnan(gsc).any()
    keys = codec.fp4_decode(rc, rs)
    qf = synth.bf16_bits_to_f32(qi)
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 254, replace=False)]))
    assert len(sample) == 256
    for i in sample.tolist():
        _check_flat(keys[:vis[i]], qf[i], wi[i], K, gtopk[i], gsc[i])
