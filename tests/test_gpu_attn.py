"""GPU parity of the sparse + window attention against the oracle.

Tolerance (from the method's requirement): per (query, head) row,
max|o_gpu - o_ref| / max|o_ref| <= 2e-3 and |lse_gpu - lse_ref| <= 1e-3.
"""
import numpy as np
import pytest
import torch

import fp4_kv_cache_02_amd as csa2
import synth
from oracle import attention, codec
from tests._gpu_util import announce, dev, empty_u8, gpu_quantize, h, t, workspace

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL = 2e-3, 1e-3


def _lists(cfg, M, K, n_valid, vis, n_pad, n_invalid):
    """Ascending Top-K-style lists: n_valid distinct positions < vis, then
    n_invalid entries >= vis (skipped by contract), then -1 padding."""
    g = synth.rng(cfg, synth.TAG_IDX_LIST)
    out = np.full((M, K), -1, np.int32)
    for m in range(M):
        nv = min(n_valid[m], vis[m])
        pos = np.sort(g.choice(vis[m], nv, replace=False)) if nv else np.zeros(0, np.int64)
        bad = vis[m] + np.arange(n_invalid[m])
        row = np.concatenate([pos, bad])[:K - n_pad[m]] if K - n_pad[m] > 0 else np.zeros(0)
        out[m, :len(row)] = row
    return out


def _run(cfg, n_rows, D, H, qdt, K, W, M, q_pos, n_valid, n_pad, n_invalid, counts, q_mult=1.0, sample=None):
    announce("attention", cfg, n_rows, D, H, qdt, K, W, M)
    x = synth.main_kv_rows(cfg, 0, 0, n_rows, D)
    codes, scales = gpu_quantize(x)
    rc, rs = codec.fp4_encode(x)
    assert np.array_equal(h(codes), rc) and np.array_equal(h(scales), rs)
    vis = [min(n_rows, p + 1) for p in q_pos]
    idx = _lists(cfg, M, K, n_valid, vis, n_pad, n_invalid) if K > 0 else np.zeros((M, 0), np.int32)
    swx = synth.swa_rows(cfg, 0, 0, max(1, M * W), D)
    sc8 = empty_u8(max(1, M * W), D)
    ss8 = torch.empty(max(1, M * W), dtype=torch.float32, device=dev())
    csa2.csa2_quantize_fp8_rows(t(swx), sc8, ss8)
    rc8, rs8 = codec.fp8_rows_encode(swx)
    assert np.array_equal(h(sc8), rc8) and np.array_equal(h(ss8), rs8)
    q = synth.q_main(cfg, 0, M, H, D, qdt)
    if qdt == "f32":
        q = (q * q_mult).astype(np.float32)
        qd = t(q)
        qf = q.astype(np.float64)
    else:
        if q_mult != 1.0:
            q = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(q) * np.float32(q_mult))
        qd = t(q).view(torch.bfloat16)
        qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    tau = D ** -0.5
    kv = csa2.fp4_cache(codes, scales, t(np.zeros(1, np.int64)), t(np.array([n_rows], np.int32)), D, n_rows, 1)
    qs = csa2.queries(t(np.zeros(M, np.int32)), t(np.asarray(q_pos, np.int32)))
    starts = (np.arange(M) * W).astype(np.int32)
    sw = csa2.swa(sc8, ss8, t(starts), t(np.asarray(counts, np.int32)), D, W)
    out = torch.full((M, H, D), 7.0, dtype=torch.float32, device=dev())
    lse = torch.full((M, H), 7.0, dtype=torch.float32, device=dev())
    ws = workspace(csa2.csa2_attn_workspace_size(M, H, D, K, W))
    csa2.csa2_sparse_swa_attn(kv, qs, qd, t(idx) if K > 0 else None, K, sw, tau, out, lse, ws)
    go, gl = h(out), h(lse)
    worst = 0.0
    for m in (range(M) if sample is None else sample):
        lo = m * W
        ro, rl = attention.sparse_swa_attention(qf[m], rc, rs, idx[m], vis[m], rc8[lo:lo + counts[m]],
                                                rs8[lo:lo + counts[m]], tau)
        for hh in range(H):
            ref = ro[hh]
            den = np.abs(ref).max()
            if den == 0:
                assert np.all(go[m, hh] == 0) and np.isneginf(gl[m, hh]) == np.isneginf(rl[hh])
                continue
            err = np.abs(go[m, hh] - ref).max() / den
            worst = max(worst, err)
            assert err <= O_TOL, (m, hh, err)
            assert abs(gl[m, hh] - rl[hh]) <= LSE_TOL, (m, hh, gl[m, hh], rl[hh])
    print(f"[attention] worst row-relative error {worst:.3e}")
    return worst


def test_attn_tiny_config_fp32_queries():
    _run(200, 4096, 128, 8, "f32", 64, 128, 1, [4095], [64], [0], [0], [128])


def test_attn_decoder_shape_bf16_batch():
    _run(201, 16384, 512, 64, "bf16", 512, 128, 4, [16383, 16383, 9000, 16383], [512, 300, 512, 1],
         [0, 200, 0, 500], [0, 12, 0, 11], [128, 77, 1, 0])


def test_attn_edge_cases():
    # query 0: no valid entry and an empty window -> o = 0, lse = -inf
    # query 1: invalid entries beyond the visible count, 5 window rows
    # query 2: large logits
    _run(202, 3000, 512, 64, "bf16", 128, 16, 3, [2999, 1000, 2999], [0, 90, 128], [128, 10, 0], [0, 28, 0],
         [0, 5, 16], q_mult=30.0)


def test_attn_many_queries_single_range():
    # enough queries that each (query, head group) handles all keys in one workgroup
    _run(203, 8192, 512, 64, "bf16", 512, 128, 160, [8191] * 160, [512] * 160, [0] * 160, [0] * 160, [128] * 160)


def test_attn_fp32_d256_partial_head_group_mixed_chunk():
    _run(204, 5000, 256, 20, "f32", 100, 50, 2, [4999, 4999], [100, 60], [0, 40], [0, 0], [50, 13])


def test_attn_window_only_and_small_dim():
    _run(205, 100, 64, 3, "bf16", 0, 128, 2, [99, 99], [0, 0], [0, 0], [0, 0], [128, 3])


def test_attn_decode_odd_topk_chunks():
    # K = 80: three 32-slot Top-K chunks, so one logits workgroup holds the
    # last Top-K chunk and the first window chunk (the mixed path), another
    # two Top-K chunks (the straight path); padding, invalid entries and a
    # one-row window on the other queries
    _run(207, 4000, 512, 64, "bf16", 80, 128, 3, [3999, 3999, 2000], [80, 50, 60], [0, 30, 10], [0, 0, 10],
         [128, 40, 1])


def test_attn_no_window_padded_slots():
    # K = 100 is not a multiple of the 64-slot chunk and there is no window:
    # the padding slots past K must contribute nothing
    _run(206, 3000, 128, 16, "bf16", 100, 0, 2, [2999, 1500], [100, 50], [0, 30], [0, 5], [0, 0])


def test_attn_prefill_schedule_sampled():
    # 320 queries x 64 heads: the one-workgroup-per-query (flash) schedule;
    # every query runs on the GPU, 64 sampled queries are checked
    M = 320
    rng = np.random.default_rng(207)
    _run(207, 6000, 512, 64, "bf16", 512, 128, M, [5999] * M, [512] * M, [0] * M, [0] * M,
         rng.integers(1, 129, M).tolist(), sample=sorted(rng.choice(M, 64, replace=False).tolist()))


def _run_prefill(cfg, n_rows, H, K, W, M, q_pos, n_valid, n_pad, n_invalid, counts, sample, q_mult=1.0):
    """Prefill-shaped call (512 channels, bf16 queries): query i's window is
    rows i .. i+counts[i]-1 of one shared buffer of M + W - 1 rows, as in a
    prefill chunk whose consecutive tokens slide the window by one row."""
    D = 512
    announce("attention prefill", cfg, n_rows, H, K, W, M)
    x = synth.main_kv_rows(cfg, 0, 0, n_rows, D)
    codes, scales = gpu_quantize(x)
    rc, rs = codec.fp4_encode(x)
    assert np.array_equal(h(codes), rc) and np.array_equal(h(scales), rs)
    vis = [min(n_rows, p + 1) for p in q_pos]
    idx = _lists(cfg, M, K, n_valid, vis, n_pad, n_invalid) if K > 0 else np.zeros((M, 0), np.int32)
    nsw = max(1, M + W - 1)
    swx = synth.swa_rows(cfg, 0, 0, nsw, D)
    sc8 = empty_u8(nsw, D)
    ss8 = torch.empty(nsw, dtype=torch.float32, device=dev())
    csa2.csa2_quantize_fp8_rows(t(swx), sc8, ss8)
    rows = sorted(set(r for m in sample for r in range(m, m + counts[m])))
    rc8, rs8 = codec.fp8_rows_encode(swx[rows]) if rows else (np.zeros((0, D), np.uint8), np.zeros(0, np.float32))
    where = {r: i for i, r in enumerate(rows)}
    g8, gs8 = h(sc8), h(ss8)
    assert np.array_equal(g8[rows], rc8) and np.array_equal(gs8[rows], rs8)
    q = synth.q_main(cfg, 0, M, H, D, "bf16")
    if q_mult != 1.0:
        q = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(q) * np.float32(q_mult))
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    tau = D ** -0.5
    kv = csa2.fp4_cache(codes, scales, t(np.zeros(1, np.int64)), t(np.array([n_rows], np.int32)), D, n_rows, 1)
    qs = csa2.queries(t(np.zeros(M, np.int32)), t(np.asarray(q_pos, np.int32)))
    sw = csa2.swa(sc8, ss8, t(np.arange(M, dtype=np.int32)), t(np.asarray(counts, np.int32)), D, W)
    out = torch.full((M, H, D), 7.0, dtype=torch.float32, device=dev())
    lse = torch.full((M, H), 7.0, dtype=torch.float32, device=dev())
    ws = workspace(csa2.csa2_attn_workspace_size(M, H, D, K, W))
    csa2.csa2_sparse_swa_attn(kv, qs, t(q).view(torch.bfloat16), t(idx) if K > 0 else None, K, sw, tau, out, lse, ws)
    go, gl = h(out), h(lse)
    assert not np.isnan(go).any() and not np.isnan(gl).any()
    worst = 0.0
    for m in sample:
        wr = [where[r] for r in range(m, m + counts[m])]
        ro, rl = attention.sparse_swa_attention(qf[m], rc, rs, idx[m], vis[m], rc8[wr], rs8[wr], tau)
        for hh in range(H):
            ref = ro[hh]
            den = np.abs(ref).max()
            if den == 0:
                assert np.all(go[m, hh] == 0) and np.isneginf(gl[m, hh]) == np.isneginf(rl[hh])
                continue
            err = np.abs(go[m, hh] - ref).max() / den
            worst = max(worst, err)
            assert err <= O_TOL, (m, hh, err)
            assert abs(gl[m, hh] - rl[hh]) <= LSE_TOL, (m, hh, gl[m, hh], rl[hh])
    print(f"[attention prefill] worst row-relative error {worst:.3e}")


def test_attn_prefill_chunk_4096_queries_sampled():
    # a 4,096-query chunk (tokens 4096 .. 8191 of an 8,192-entry cache), Top-512
    # lists and 128-row sliding windows; 256 queries checked (the first, the
    # last and 254 drawn at random)
    M, n = 4096, 8192
    rng = np.random.default_rng(208)
    sample = sorted(set([0, M - 1] + rng.choice(np.arange(1, M - 1), 254, replace=False).tolist()))
    assert len(sample) == 256
    _run_prefill(208, n, 64, 512, 128, M, list(range(n - M, n)), [512] * M, [0] * M, [0] * M, [128] * M, sample)


def test_attn_prefill_edges():
    # K = 80: the second chunk holds one wave's main entries and three waves'
    # window rows; lists with padding and entries past the visible count;
    # window counts from 0 to 128; short causal prefixes; queries that see
    # nothing (o = 0, lse = -inf); large logits
    M = 300
    rng = np.random.default_rng(209)
    q_pos = rng.integers(0, 3000, M)
    q_pos[:5] = [0, 3, 7, 2999, 2999]
    n_valid = rng.integers(0, 81, M)
    n_pad = rng.integers(0, 30, M)
    n_invalid = rng.integers(0, 6, M)
    counts = rng.integers(0, 129, M)
    n_valid[0], n_pad[0], n_invalid[0], counts[0] = 0, 80, 0, 0
    n_valid[4], n_pad[4], n_invalid[4], counts[4] = 80, 0, 0, 128
    sample = sorted(set([0, 1, 2, 3, 4] + rng.choice(M, 7, replace=False).tolist()))
    _run_prefill(209, 3000, 64, 80, 128, M, q_pos.tolist(), n_valid.tolist(), n_pad.tolist(), n_invalid.tolist(),
                 counts.tolist(), sample, q_mult=12.0)


def test_attn_prefill_two_head_blocks_and_window_only():
    # 80 heads: a full and a partial block of 64; then no Top-K list at all
    M = 200
    rng = np.random.default_rng(210)
    sample = sorted(rng.choice(M, 5, replace=False).tolist())
    _run_prefill(210, 2000, 80, 64, 32, M, [1999] * M, [60] * M, [4] * M, [0] * M,
                 rng.integers(1, 33, M).tolist(), sample)
    M = 260
    sample = sorted(rng.choice(M, 5, replace=False).tolist())
    _run_prefill(211, 500, 64, 0, 128, M, [499] * M, [0] * M, [0] * M, [0] * M,
                 rng.integers(0, 129, M).tolist(), sample)
