#!/usr/bin/env python3
"""Benchmark of the CSA2 decode hot path on one MI355X.

Workload (default): 4 sequences x 1,048,576 visible entries, one decode token
per sequence through the 20-layer decoder (group 1 = Full + 3 Reuse, groups
2-5 = Reindex + 3 Reuse), 512-channel FP4 latent, 64 bf16 query heads,
indexer 8 x 128, pool 2,048 blocks, Top-512, FP8 window 128.  A step is one
pass of the whole hot path for the batch: write the new token's FP4 entry and
its indexer key, the Full layer's first scan + pool + Top-K, four Reindex
selections and twenty attention layers.  Inputs are seeded synthetic tensors
already resident in HBM when timing starts.

--workload 2 times the encoder prefill chunk instead: 4,096 query tokens
(tokens 126,976 .. 131,072 of a 131,072-token prompt, ratio 2, 65,536
compressed entries) through the 18 encoder layers (3 groups of Full + 5
Reuse, flat Top-512), each Full group re-writing the chunk's 2,048 entries.

Prints one JSON line (see the `result` dict below).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA2 decode query-tokens/s + achieved HBM GB/s vs peak, 20-layer decoder @1M ctx"
METRIC_PREFILL = "CSA2 encoder prefill query-tokens/s, 18 layers, 4,096-token chunk @128K tokens"
HBM_PEAK_GBS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0   # dense f16/bf16 MFMA, MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4,
                    help="workload index (4 = 4 x 1M decode; 2 = encoder prefill chunk)")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph",
                    help="graph: the timed steps replay one captured HIP graph; eager: launched one by one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after timing, copy a buffer of this size once (counter calibration under --pmc)")
    return ap.parse_args()


def scan_source_sha256() -> str:
    """Digest of the sources the first-scan kernel is compiled from (its traffic
    record is only reported while they are unchanged)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("csa2_index.hip", "csa2_indexer.hpp", "csa2_device.hpp"):
        h.update(open(os.path.join(ROOT, "fp4_kv_cache_02_amd", "csrc", f), "rb").read())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# GPU workload (HIP path only)
# ---------------------------------------------------------------------------

class DecodeWorkload:
    def __init__(self, wl, torch, csa2, synth):
        self.wl, self.torch, self.csa2 = wl, torch, csa2
        dev = torch.device("cuda:0")
        S, D, DI = len(wl.seq_lens), wl.dim, wl.idx_dim
        lens = np.asarray(wl.seq_lens, np.int64)
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        R = int(lens.sum())
        u8 = dict(dtype=torch.uint8, device=dev)
        self.kv_codes = torch.empty((R, D // 2), **u8)
        self.kv_scales = torch.empty((R, D // 16), **u8)
        self.ik_codes = torch.empty((R, DI // 2), **u8)
        self.ik_scales = torch.empty((R, DI // 16), **u8)
        w_ik = torch.from_numpy(synth.w_ik(wl.cfg, D, DI)).to(dev)
        chunk = 1 << 20
        for s in range(S):
            for c0 in range(0, int(lens[s]), chunk):
                n = min(chunk, int(lens[s]) - c0)
                x = torch.from_numpy(synth.main_kv_rows(wl.cfg, s, c0, n, D)).to(dev)
                r0 = int(starts[s]) + c0
                csa2.csa2_quantize_fp4(x, self.kv_codes[r0:r0 + n], self.kv_scales[r0:r0 + n], w_ik=w_ik,
                                       ik_codes=self.ik_codes[r0:r0 + n], ik_scales=self.ik_scales[r0:r0 + n])
                del x
        torch.cuda.synchronize()
        seq_start = torch.from_numpy(starts).to(dev)
        seq_len = torch.from_numpy(lens.astype(np.int32)).to(dev)
        max_len = int(lens.max())
        self.kv = csa2.fp4_cache(self.kv_codes, self.kv_scales, seq_start, seq_len, D, max_len, wl.ratio)
        self.idx = csa2.fp4_cache(self.ik_codes, self.ik_scales, seq_start, seq_len, DI, max_len, wl.ratio)
        M = S
        self.M = M
        self.q_pos_host = (lens - 1).astype(np.int32)
        self.qs = csa2.queries(torch.arange(M, dtype=torch.int32, device=dev),
                               torch.from_numpy(self.q_pos_host).to(dev))
        # the decode token's own entry (position len-1) is (re)written by the Full group
        new = np.stack([synth.main_kv_rows(wl.cfg, s, int(lens[s]) - 1, 1, D)[0] for s in range(S)])
        self.new_kv = torch.from_numpy(new).to(dev)
        self.new_dst = torch.from_numpy(starts + lens - 1).to(dev)
        self.w_ik = w_ik
        # per-layer queries, window rows and outputs
        L, H, W = wl.n_layers, wl.heads, wl.window
        self.q, self.swa, self.out, self.lse = [], [], [], []
        swa_start = torch.from_numpy((np.arange(M) * W).astype(np.int32)).to(dev)
        swa_count = torch.from_numpy(np.minimum(W, lens).astype(np.int32)).to(dev)
        for layer in range(L):
            qb = synth.q_main(wl.cfg, layer, M, H, D, "bf16")
            self.q.append(torch.from_numpy(qb.view(np.int16)).to(dev).view(torch.bfloat16))
            rows = np.concatenate([synth.swa_rows(wl.cfg, layer, s, W, D) for s in range(M)])
            sc = torch.empty((M * W, D), **u8)
            ss = torch.empty((M * W,), dtype=torch.float32, device=dev)
            csa2.csa2_quantize_fp8_rows(torch.from_numpy(rows).to(dev), sc, ss)
            self.swa.append(csa2.swa(sc, ss, swa_start, swa_count, D, W))
            self.out.append(torch.empty((M, H, D), dtype=torch.float32, device=dev))
            self.lse.append(torch.empty((M, H), dtype=torch.float32, device=dev))
        P, K = wl.pool_blocks, wl.top_k
        self.pool = torch.empty((M, P), dtype=torch.int32, device=dev)
        self.pool_count = torch.empty((M,), dtype=torch.int32, device=dev)
        self.groups = []
        layer = 0
        for gi, modes in enumerate(wl.groups):
            n = len(modes)
            qi = synth.q_idx(wl.cfg, layer, M, wl.idx_heads, DI)
            wi = synth.w_idx(wl.cfg, layer, M, wl.idx_heads)
            qi_t = torch.from_numpy(qi.view(np.int16)).to(dev).view(torch.bfloat16)
            wi_t = torch.from_numpy(wi).to(dev)
            topk = torch.empty((M, K), dtype=torch.int32, device=dev)
            full = modes[0] == "full"
            g = csa2.Group(csa2.CSA2_MODE_FULL if full else csa2.CSA2_MODE_REINDEX, self.kv, self.idx, self.qs,
                           qi_t, wi_t, P, K, self.pool, self.pool_count, topk, None,
                           self.q[layer:layer + n], csa2.CSA2_BF16, H, self.swa[layer:layer + n],
                           self.out[layer:layer + n], self.lse[layer:layer + n], D ** -0.5,
                           new_kv=self.new_kv if full else None, new_dst_row=self.new_dst if full else None,
                           w_ik=self.w_ik if full else None)
            g.topk_tensor = topk
            self.groups.append(g)
            layer += n
        ws_bytes = max(csa2.csa2_group_workspace_size(g) for g in self.groups)
        self.ws = torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev)  # zero before first use
        torch.cuda.synchronize()

    def step(self):
        for g in self.groups:
            self.csa2.csa2_group_step(g, self.ws)

    def snapshot(self):
        t = self.torch
        t.cuda.synchronize()
        return ([g.topk_tensor.clone() for g in self.groups], self.pool.clone(),
                [o.clone() for o in self.out], [l.clone() for l in self.lse])

    # algorithmic bytes
    def scan_bytes_per_launch(self) -> int:
        wl = self.wl
        row = wl.idx_dim // 2 + wl.idx_dim // 16
        vis = np.minimum(np.asarray(wl.seq_lens), (self.q_pos_host + 1) // wl.ratio)
        return int(vis.sum()) * row

    def attn_bytes_per_launch(self) -> int:
        # one layer's attention: selected main rows, window rows, bf16 queries, fp32 outputs and lse
        wl = self.wl
        D, H, W, K = wl.dim, wl.heads, wl.window, wl.top_k
        kv_row = D // 2 + D // 16
        return self.M * (K * kv_row + W * (D + 4) + H * D * 2 + H * D * 4 + H * 4)

    def step_bytes(self) -> int:
        wl = self.wl
        D, H, W, K, P = wl.dim, wl.heads, wl.window, wl.top_k, wl.pool_blocks
        idx_row = wl.idx_dim // 2 + wl.idx_dim // 16
        kv_row = D // 2 + D // 16
        vis = np.minimum(np.asarray(wl.seq_lens), (self.q_pos_host + 1) // wl.ratio)
        n_sel = sum(1 for g in wl.groups)                                # Full + Reindex selections
        pool_pos = np.minimum(vis, 8 * P)
        sel = int(n_sel * pool_pos.sum()) * idx_row
        attn_per_q = K * kv_row + W * (D + 4) + H * D * 2 + H * D * 4 + H * 4
        attn = wl.n_layers * self.M * attn_per_q
        write = self.M * (D * 4 + kv_row + idx_row)
        return self.scan_bytes_per_launch() + sel + attn + write


class PrefillWorkload:
    """Encoder prefill chunk: every Full group writes the chunk's entries,
    selects flat Top-K lists for all its queries and runs its layers."""

    def __init__(self, wl, torch, csa2, synth):
        self.wl, self.torch, self.csa2 = wl, torch, csa2
        dev = torch.device("cuda:0")
        E, D, DI, ratio = int(wl.seq_lens[0]), wl.dim, wl.idx_dim, wl.ratio
        M, t0 = wl.n_queries, wl.first_query_token
        R = M // ratio                                    # entries completed by the chunk's tokens
        u8 = dict(dtype=torch.uint8, device=dev)
        self.kv_codes = torch.empty((E, D // 2), **u8)
        self.kv_scales = torch.empty((E, D // 16), **u8)
        self.ik_codes = torch.empty((E, DI // 2), **u8)
        self.ik_scales = torch.empty((E, DI // 16), **u8)
        w_ik = torch.from_numpy(synth.w_ik(wl.cfg, D, DI)).to(dev)
        x = torch.from_numpy(synth.main_kv_rows(wl.cfg, 0, 0, E, D)).to(dev)
        csa2.csa2_quantize_fp4(x, self.kv_codes, self.kv_scales, w_ik=w_ik, ik_codes=self.ik_codes,
                               ik_scales=self.ik_scales)
        self.new_kv = x[E - R:].clone()
        del x
        self.new_dst = torch.arange(E - R, E, dtype=torch.int64, device=dev)
        self.w_ik = w_ik
        seq_start = torch.zeros(1, dtype=torch.int64, device=dev)
        seq_len = torch.tensor([E], dtype=torch.int32, device=dev)
        self.kv = csa2.fp4_cache(self.kv_codes, self.kv_scales, seq_start, seq_len, D, E, ratio)
        self.idx = csa2.fp4_cache(self.ik_codes, self.ik_scales, seq_start, seq_len, DI, E, ratio)
        self.M = M
        self.q_pos_host = np.arange(t0, t0 + M, dtype=np.int64)
        self.qs = csa2.queries(torch.zeros(M, dtype=torch.int32, device=dev),
                               torch.from_numpy(self.q_pos_host.astype(np.int32)).to(dev))
        L, H, W, K = wl.n_layers, wl.heads, wl.window, wl.top_k
        nsw = M + W - 1                                   # the chunk's token rows and the W-1 before them
        swa_start = torch.arange(M, dtype=torch.int32, device=dev)
        swa_count = torch.full((M,), W, dtype=torch.int32, device=dev)
        self.q, self.swa, self.out, self.lse = [], [], [], []
        for layer in range(L):
            qb = synth.q_main(wl.cfg, layer, M, H, D, "bf16")
            self.q.append(torch.from_numpy(qb.view(np.int16)).to(dev).view(torch.bfloat16))
            sc = torch.empty((nsw, D), **u8)
            ss = torch.empty((nsw,), dtype=torch.float32, device=dev)
            csa2.csa2_quantize_fp8_rows(torch.from_numpy(synth.swa_rows(wl.cfg, layer, 0, nsw, D)).to(dev), sc, ss)
            self.swa.append(csa2.swa(sc, ss, swa_start, swa_count, D, W))
            self.out.append(torch.empty((M, H, D), dtype=torch.float32, device=dev))
            self.lse.append(torch.empty((M, H), dtype=torch.float32, device=dev))
        self.groups = []
        layer = 0
        for modes in wl.groups:
            n = len(modes)
            qi = synth.q_idx(wl.cfg, layer, M, wl.idx_heads, DI)
            wi = synth.w_idx(wl.cfg, layer, M, wl.idx_heads)
            topk = torch.empty((M, K), dtype=torch.int32, device=dev)
            g = csa2.Group(csa2.CSA2_MODE_FULL, self.kv, self.idx, self.qs,
                           torch.from_numpy(qi.view(np.int16)).to(dev).view(torch.bfloat16),
                           torch.from_numpy(wi).to(dev), 0, K, None, None, topk, None,
                           self.q[layer:layer + n], csa2.CSA2_BF16, H, self.swa[layer:layer + n],
                           self.out[layer:layer + n], self.lse[layer:layer + n], D ** -0.5,
                           new_kv=self.new_kv, new_dst_row=self.new_dst, w_ik=self.w_ik)
            g.topk_tensor = topk
            self.groups.append(g)
            layer += n
        ws_bytes = max(csa2.csa2_group_workspace_size(g) for g in self.groups)
        self.ws = torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev)  # zero before first use
        torch.cuda.synchronize()

    def step(self):
        for g in self.groups:
            self.csa2.csa2_group_step(g, self.ws)

    def snapshot(self):
        t = self.torch
        t.cuda.synchronize()
        last = [self.out[i] for i in range(len(self.out)) if (i + 1) % len(self.wl.groups[0]) == 0]
        return ([g.topk_tensor.clone() for g in self.groups], self.new_dst.clone(),
                [o.clone() for o in last], [l.clone() for l in self.lse])

    def visible(self) -> np.ndarray:
        return np.minimum(self.wl.seq_lens[0], (self.q_pos_host + 1) // self.wl.ratio)

    # algorithmic work
    def scoring_flops_per_launch(self) -> float:
        return 2.0 * self.wl.idx_heads * self.wl.idx_dim * float(self.visible().sum())

    def attn_flops_per_launch(self) -> float:
        wl = self.wl
        return 4.0 * self.M * wl.heads * wl.dim * (wl.top_k + wl.window)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def cpu_baseline(wl, synth) -> dict:
    from oracle import attention, codec, indexer
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    ns = 65536                                   # prefix of sequence 0 used by the sample
    D, DI = wl.dim, wl.idx_dim
    x = synth.main_kv_rows(wl.cfg, 0, 0, ns, D)
    kc, ks = codec.fp4_encode(x)
    ikc, iks = codec.indexer_key(kc, ks, synth.w_ik(wl.cfg, D, DI))
    del x
    W, H = wl.window, wl.heads
    q_layers = [synth.bf16_bits_to_f32(synth.q_main(wl.cfg, l, 1, H, D, "bf16"))[0] for l in range(wl.n_layers)]
    swa = [codec.fp8_rows_encode(synth.swa_rows(wl.cfg, l, 0, W, D)) for l in range(wl.n_layers)]
    tau = D ** -0.5

    def one_token():
        t0 = time.perf_counter()
        keys = codec.fp4_decode(ikc, iks)
        layer = 0
        pool = None
        t_scan = 0.0
        for modes in wl.groups:
            qi = synth.bf16_bits_to_f32(synth.q_idx(wl.cfg, layer, 1, wl.idx_heads, DI))[0]
            wi = synth.w_idx(wl.cfg, layer, 1, wl.idx_heads)[0]
            if modes[0] == "full":
                ts = time.perf_counter()
                s = indexer.scores(qi, wi, keys)
                t_scan += time.perf_counter() - ts
                pool = indexer.pool_select(indexer.block_max(s), wl.pool_blocks)
                cand = indexer.pool_positions(pool, ns)
                sel = indexer.top_ids(s[cand], cand, min(wl.top_k, len(cand)))
            else:
                sel, _ = indexer.reindex(qi, wi, keys, pool, wl.top_k)
            for _ in modes:
                attention.sparse_swa_attention(q_layers[layer], kc, ks, sel, ns, swa[layer][0], swa[layer][1], tau)
                layer += 1
        return time.perf_counter() - t0, t_scan

    one_token()
    runs = [one_token() for _ in range(3)]
    t_tok, t_scan = sorted(runs)[1]
    # the first scan (decode of all visible keys + their scores) grows linearly with
    # the context; everything else is bounded by the pool, the Top-K and the window
    n_full = max(wl.seq_lens)
    t_full_ctx = t_tok + t_scan * (n_full / ns - 1.0)
    return {"value": 1.0 / t_full_ctx, "unit": "query-tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"NumPy fp64 oracle, one decode token of sequence 0 through all {wl.n_layers} layers "
                       f"over its first {ns} entries (median of 3: {t_tok * 1e3:.0f} ms, first scan "
                       f"{t_scan * 1e3:.0f} ms); the first scan scaled linearly to {n_full} entries")}


def cpu_baseline_prefill(wl, synth) -> dict:
    from oracle import attention, codec, indexer
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    ns = 8192                                    # prefix of the prompt's entries used by the sample
    D, DI, W, H, K = wl.dim, wl.idx_dim, wl.window, wl.heads, wl.top_k
    x = synth.main_kv_rows(wl.cfg, 0, 0, ns, D)
    kc, ks = codec.fp4_encode(x)
    ikc, iks = codec.indexer_key(kc, ks, synth.w_ik(wl.cfg, D, DI))
    del x
    q_layers = [synth.bf16_bits_to_f32(synth.q_main(wl.cfg, l, 1, H, D, "bf16"))[0] for l in range(wl.n_layers)]
    swa = [codec.fp8_rows_encode(synth.swa_rows(wl.cfg, l, 0, W, D)) for l in range(wl.n_layers)]
    tau = D ** -0.5

    def one_token():
        t0 = time.perf_counter()
        t_scan = 0.0
        layer = 0
        for modes in wl.groups:
            qi = synth.bf16_bits_to_f32(synth.q_idx(wl.cfg, layer, 1, wl.idx_heads, DI))[0]
            wi = synth.w_idx(wl.cfg, layer, 1, wl.idx_heads)[0]
            ts = time.perf_counter()
            sel, _ = indexer.index_flat(qi, wi, codec.fp4_decode(ikc, iks), K)
            t_scan += time.perf_counter() - ts
            for _ in modes:
                attention.sparse_swa_attention(q_layers[layer], kc, ks, sel, ns, swa[layer][0], swa[layer][1], tau)
                layer += 1
        return time.perf_counter() - t0, t_scan

    one_token()
    runs = [one_token() for _ in range(3)]
    t_tok, t_scan = sorted(runs)[1]
    n_full = int(wl.seq_lens[0])
    t_full_ctx = t_tok + t_scan * (n_full / ns - 1.0)
    return {"value": 1.0 / t_full_ctx, "unit": "query-tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"NumPy fp64 oracle, one prefill query through all {wl.n_layers} encoder layers over the "
                       f"first {ns} entries (median of 3: {t_tok * 1e3:.0f} ms, flat Top-K {t_scan * 1e3:.0f} ms); "
                       f"the flat Top-K scaled linearly to {n_full} entries")}


def run_prefill(args, wl, torch, csa2, synth):
    t0 = time.time()
    W = PrefillWorkload(wl, torch, csa2, synth)
    setup_s = time.time() - t0
    print(f"[bench] setup {setup_s:.1f}s: {wl.name}, {W.M} queries over {wl.seq_lens[0]} entries",
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        W.step()
    torch.cuda.synchronize()
    ref = W.snapshot()

    def same(a, b):
        return all(torch.equal(x, y) for x, y in zip(a[0] + [a[1]] + a[2] + a[3], b[0] + [b[1]] + b[2] + b[3]))

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        W.step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    if not same(ref, W.snapshot()):
        raise RuntimeError("timed steps differ from the warm-up step")
    # kernel durations: HIP events stamped by each scoring / attention dispatch, same steps again
    csa2.csa2_profile_scan(True)
    csa2.csa2_profile_attn(True)
    for _ in range(args.steps):
        W.step()
    torch.cuda.synchronize()
    sc_ms, sc_n = csa2.csa2_profile_scan_read()
    at_ms, at_n = csa2.csa2_profile_attn_read()
    csa2.csa2_profile_scan(False)
    csa2.csa2_profile_attn(False)
    assert sc_n == args.steps * len(wl.groups) and at_n == args.steps * wl.n_layers, (sc_n, at_n)
    ms_per_step = ms_total / args.steps
    at_avg, sc_avg = at_ms / at_n, sc_ms / sc_n
    at_tf = W.attn_flops_per_launch() / (at_avg / 1e3) / 1e12
    sc_tf = W.scoring_flops_per_launch() / (sc_avg / 1e3) / 1e12
    result = {
        "metric": METRIC_PREFILL,
        "value": round(W.M / (ms_per_step / 1e3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "queries": W.M, "entries": int(wl.seq_lens[0]), "ratio": wl.ratio,
                   "layers": wl.n_layers, "layout": "3x(Full+5Reuse), flat Top-K", "latent_dim": wl.dim,
                   "heads": wl.heads, "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim, "top_k": wl.top_k,
                   "window": wl.window, "storage": "FP4 E2M1/E4M3x16 main+indexer, FP8 E4M3 window"},
        "roofline": {"bound": "mfma", "kernel": "prefill attention (k_attn_prefill)", "achieved": round(at_tf, 1),
                     "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(at_tf / F16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": None, "avg_launch_ms": round(at_avg, 4),
                     "timing": "HIP events stamped by each attention dispatch (same steps run again)",
                     "algorithmic_flops_per_launch": W.attn_flops_per_launch()},
        "indexer_scoring": {"bound": "mfma", "kernel": "k_score_mq", "achieved": round(sc_tf, 1),
                            "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(sc_tf / F16_MFMA_PEAK_TFLOPS, 4), "avg_launch_ms": round(sc_avg, 4),
                            "algorithmic_flops_per_launch": W.scoring_flops_per_launch()},
        "wall_s_timed": round(wall, 4),
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        t0 = time.time()
        result["cpu_baseline"] = cpu_baseline_prefill(wl, synth)
        print(f"[bench] cpu baseline {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
              "sequences shard across GPUs with no exchange, see DESIGN.md", file=sys.stderr)
        sys.exit(2)
    import torch
    import fp4_kv_cache_02_amd as csa2
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    csa2.lib()
    wl = synth.workload(args.workload)
    if wl.phase == "prefill":
        run_prefill(args, wl, torch, csa2, synth)
        return
    assert wl.phase == "decode", wl.phase
    t0 = time.time()
    W = DecodeWorkload(wl, torch, csa2, synth)
    setup_s = time.time() - t0
    print(f"[bench] setup {setup_s:.1f}s: {wl.name}, {len(wl.seq_lens)} seqs, {sum(wl.seq_lens)} entries",
          file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        W.step()
    torch.cuda.synchronize()
    ref = W.snapshot()

    def same(a, b):
        return all(torch.equal(x, y) for x, y in zip(a[0] + [a[1]] + a[2] + a[3], b[0] + [b[1]] + b[2] + b[3]))

    graph = None
    if args.mode == "graph":
        # all timed steps in one captured graph (kernel launches only)
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for _ in range(args.steps):
                    W.step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph.replay()                     # untimed replay, checked against eager
        torch.cuda.synchronize()
        if not same(ref, W.snapshot()):
            raise RuntimeError("graph replay differs from eager execution")
    else:
        csa2.csa2_profile_scan(True)
        csa2.csa2_profile_attn(True)

    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            W.step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    if not same(ref, W.snapshot()):
        raise RuntimeError("timed steps differ from the eager reference")
    if graph is not None:
        # events cannot be timed inside a graph replay: the first scan's launch
        # duration comes from HIP events stamped by its dispatch in the same steps run eagerly
        csa2.csa2_profile_scan(True)
        csa2.csa2_profile_attn(True)
        for _ in range(args.steps):
            W.step()
        torch.cuda.synchronize()
    scan_ms_total, scan_launches = csa2.csa2_profile_scan_read()
    attn_ms_total, attn_launches = csa2.csa2_profile_attn_read()
    csa2.csa2_profile_scan(False)
    csa2.csa2_profile_attn(False)
    assert scan_launches == args.steps, (scan_launches, args.steps)
    assert attn_launches == args.steps * wl.n_layers, (attn_launches, args.steps)

    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    ms_per_step = ms_total / args.steps
    tokens_per_step = W.M
    value = tokens_per_step / (ms_per_step / 1e3)
    scan_avg_ms = scan_ms_total / max(1, scan_launches)
    scan_bytes = W.scan_bytes_per_launch()
    achieved = scan_bytes / (scan_avg_ms / 1e3) / 1e9
    step_bytes = W.step_bytes()
    attn_avg_ms = attn_ms_total / max(1, attn_launches)
    attn_bytes = W.attn_bytes_per_launch()
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "scan_traffic.json")
    if os.path.exists(tpath):
        import hashlib
        rec = json.load(open(tpath))
        if rec.get("source_sha256") == scan_source_sha256() and rec.get("workload") == wl.name:
            traffic = rec.get("bytes_per_launch")
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "sequences": len(wl.seq_lens), "context": max(wl.seq_lens),
                   "layers": wl.n_layers, "layout": "Full+3Reuse, 4x(Reindex+3Reuse)", "latent_dim": wl.dim,
                   "heads": wl.heads, "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim,
                   "pool_blocks": wl.pool_blocks, "top_k": wl.top_k, "window": wl.window,
                   "storage": "FP4 E2M1/E4M3x16 main+indexer, FP8 E4M3 window", "mode": args.mode},
        "roofline": {"bound": "hbm", "kernel": "first scan (k_scan)", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "avg_launch_ms": round(scan_avg_ms, 5),
                     "timing": "HIP events stamped by each first-scan dispatch" + (
                         " (same steps run eagerly after the timed graph replay)" if graph is not None else ""),
                     "algorithmic_bytes_per_launch": scan_bytes},
        "attention": {"kernel": "k_attn_decode", "avg_launch_ms": round(attn_avg_ms, 5),
                      "algorithmic_bytes_per_launch": attn_bytes,
                      "achieved_gbs": round(attn_bytes / (attn_avg_ms / 1e3) / 1e9, 1),
                      "bound": "latency (one layer's reads are ~1.6 MB)"},
        "step_algorithmic_bytes": step_bytes,
        "step_algorithmic_gbs": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "wall_s_timed": round(wall, 4),
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        t0 = time.time()
        result["cpu_baseline"] = cpu_baseline(wl, synth)
        print(f"[bench] cpu baseline {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
