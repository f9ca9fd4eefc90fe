#!/usr/bin/env python3
"""Benchmark of the CSA2 hot path on one MI355X.

Headline (default): 4 sequences x 1,048,576 visible entries, one decode token
per sequence through the 20-layer decoder (group 1 = Full + 3 Reuse, groups
2-5 = Reindex + 3 Reuse), 512-channel FP4 latent, 64 bf16 query heads,
indexer 8 x 128, pool 2,048 blocks, Top-512, FP8 window 128.  A step is one
pass of the whole hot path for the batch: write the new token's FP4 entry and
its indexer key, the Full layer's first scan + pool + Top-K, four Reindex
selections and twenty attention layers.  Inputs are seeded synthetic tensors
already resident in HBM when timing starts.

The same JSON line carries, under "workloads", the other configurations:
the 4 x 1M decode timed eagerly and cold (a 1 GiB scratch write before each
step evicts the caches), the 64K decoder (graph and eager), the ragged batch
of 32 sequences (32K..256K entries) and the encoder prefill chunk (4,096
query tokens of a 131,072-token prompt at ratio 2 through 18 layers, each
Full group writing its 2,048 new entries into its own caches).  Each carries
its step time, query-tokens/s, the roofline fraction of its dominant kernel
and the oracle's CPU baseline.  --no-extras times the headline only;
--workload 2 makes the prefill chunk the headline.

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
F64_MFMA_PEAK_TFLOPS = 78.6     # fp64 MFMA, MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4,
                    help="headline workload index (4 = 4 x 1M decode; 2 = encoder prefill chunk)")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph",
                    help="graph: the timed steps replay one captured HIP graph; eager: launched one by one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="time the headline workload only")
    ap.add_argument("--cold-reps", type=int, default=10, help="steps of the cold-cache variant")
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
    """One decode step of the decoder: every group's write path and index,
    and every layer's attention.  Schedules:
      "steps"  - one csa2_group_steps call over all groups: their indexers in
                 group order, then every layer's attention batched across
                 groups (the queries of all layers are inputs here);
      "groups" - one csa2_group_step per group (its layers' attention batched);
      "layers" - what a model running layer by layer would issue: the group
                 step of each group's first layer, then one
                 csa2_sparse_swa_attn call per Reuse layer."""

    def __init__(self, wl, torch, csa2, synth, schedule="steps"):
        self.wl, self.torch, self.csa2 = wl, torch, csa2
        assert schedule in ("steps", "groups", "layers"), schedule
        self.schedule = schedule
        layer_sequential = schedule == "layers"
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
        # T tokens per sequence (the last T of each), one query each, in runs per sequence
        T = int(wl.extra.get("tokens_per_seq", 1))
        self.T = T
        M = S * T
        self.M = M
        q_seq = np.repeat(np.arange(S), T).astype(np.int32)
        self.q_seq_host = q_seq
        self.q_pos_host = (np.repeat(lens, T) - T + np.tile(np.arange(T), S)).astype(np.int32)
        self.qs = csa2.queries(torch.from_numpy(q_seq).to(dev), torch.from_numpy(self.q_pos_host).to(dev), run=T)
        # the tokens' own entries (positions len-T .. len-1) are (re)written by the Full group
        new = np.concatenate([synth.main_kv_rows(wl.cfg, s, int(lens[s]) - T, T, D) for s in range(S)])
        self.new_kv = torch.from_numpy(new).to(dev)
        self.new_dst = torch.from_numpy(np.repeat(starts + lens, T) - T + np.tile(np.arange(T), S)).to(dev)
        self.w_ik = w_ik
        # per-layer queries, window rows and outputs
        L, H, W = wl.n_layers, wl.heads, wl.window
        self.q, self.swa, self.out, self.lse = [], [], [], []
        # window rows: per sequence the W + T - 1 rows ending at its last token; token k of a
        # run sees the W rows ending at itself
        NW = W + T - 1
        swa_start = torch.from_numpy((np.repeat(np.arange(S) * NW, T) + np.tile(np.arange(T), S)).astype(np.int32)).to(dev)
        swa_count = torch.from_numpy(np.minimum(W, self.q_pos_host.astype(np.int64) + 1).astype(np.int32)).to(dev)
        for layer in range(L):
            qb = synth.q_main(wl.cfg, layer, M, H, D, "bf16")
            self.q.append(torch.from_numpy(qb.view(np.int16)).to(dev).view(torch.bfloat16))
            rows = np.concatenate([synth.swa_rows(wl.cfg, layer, s, NW, D) for s in range(S)])
            sc = torch.empty((S * NW, D), **u8)
            ss = torch.empty((S * NW,), dtype=torch.float32, device=dev)
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
            ng = 1 if layer_sequential else n
            g = csa2.Group(csa2.CSA2_MODE_FULL if full else csa2.CSA2_MODE_REINDEX, self.kv, self.idx, self.qs,
                           qi_t, wi_t, P, K, self.pool, self.pool_count, topk, None,
                           self.q[layer:layer + ng], csa2.CSA2_BF16, H, self.swa[layer:layer + ng],
                           self.out[layer:layer + ng], self.lse[layer:layer + ng], D ** -0.5,
                           new_kv=self.new_kv if full else None, new_dst_row=self.new_dst if full else None,
                           w_ik=self.w_ik if full else None)
            g.topk_tensor = topk
            g.reuse_layers = list(range(layer + 1, layer + n)) if layer_sequential else []
            self.groups.append(g)
            layer += n
        ws_bytes = max(csa2.csa2_group_workspace_size(g) for g in self.groups)
        if layer_sequential:
            ws_bytes = max(ws_bytes, csa2.csa2_attn_workspace_size(M, H, D, K, W))
        if schedule == "steps":
            ws_bytes = max(ws_bytes, csa2.csa2_group_steps_workspace_size(self.groups))
        self.ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)   # no initial contents needed
        torch.cuda.synchronize()

    def step(self):
        c = self.csa2
        if self.schedule == "steps":
            c.csa2_group_steps(self.groups, self.ws)
            return
        for g in self.groups:
            c.csa2_group_step(g, self.ws)
            for layer in g.reuse_layers:
                c.csa2_sparse_swa_attn(self.kv, self.qs, self.q[layer], g.topk_tensor, self.wl.top_k,
                                       self.swa[layer], self.wl.dim ** -0.5, self.out[layer], self.lse[layer],
                                       self.ws)

    def snapshot(self):
        t = self.torch
        t.cuda.synchronize()
        return ([g.topk_tensor.clone() for g in self.groups], self.pool.clone(),
                [o.clone() for o in self.out], [l.clone() for l in self.lse])

    # algorithmic bytes
    def scan_bytes_per_launch(self) -> int:
        # each sequence's visible indexer rows once (the tokens of a run share them)
        wl = self.wl
        row = wl.idx_dim // 2 + wl.idx_dim // 16
        lens = np.asarray(wl.seq_lens)
        vis = np.minimum(lens[self.q_seq_host], (self.q_pos_host.astype(np.int64) + 1) // wl.ratio)
        per_seq = np.zeros(len(lens), np.int64)
        np.maximum.at(per_seq, self.q_seq_host, vis)
        return int(per_seq.sum()) * row

    @property
    def attn_layers(self) -> int:
        return self.wl.n_layers

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
        lens = np.asarray(wl.seq_lens)
        vis = np.minimum(lens[self.q_seq_host], (self.q_pos_host.astype(np.int64) + 1) // wl.ratio)
        n_sel = sum(1 for g in wl.groups)                                # Full + Reindex selections
        pool_pos = np.minimum(vis, 8 * P)
        sel = int(n_sel * pool_pos.sum()) * idx_row
        attn_per_q = K * kv_row + W * (D + 4) + H * D * 2 + H * D * 4 + H * 4
        attn = wl.n_layers * self.M * attn_per_q
        write = self.M * (D * 4 + kv_row + idx_row)
        return self.scan_bytes_per_launch() + sel + attn + write


class CedDecodeWorkload:
    """One decode token per sequence through the whole encoder-decoder: the
    encoder's 2 window-only layers, its 3 CSA2 groups (Full + 5 Reuse) at
    ratio 2 over the tokens' compressed entries (each Full layer with its own
    caches, writing the entry the token completes; the flat Top-K is taken
    from a pool of K blocks, which holds every flat Top-K position), then the
    20-layer decoder."""

    def __init__(self, wl, torch, csa2, synth):
        self.wl, self.torch, self.csa2 = wl, torch, csa2
        dev = torch.device("cuda:0")
        self.dec = DecodeWorkload(wl, torch, csa2, synth)
        ex = wl.extra
        S, D, DI, H, W, K = len(wl.seq_lens), wl.dim, wl.idx_dim, wl.heads, wl.window, wl.top_k
        r = ex["encoder_ratio"]
        tokens = np.asarray(wl.seq_lens, np.int64)          # the decode token is token len-1
        elens = tokens // r                                 # entries complete at that token
        self.elens = elens
        starts = np.concatenate([[0], np.cumsum(elens)[:-1]]).astype(np.int64)
        R = int(elens.sum())
        u8 = dict(dtype=torch.uint8, device=dev)
        w_ik = torch.from_numpy(synth.w_ik(wl.cfg + 100, D, DI)).to(dev)
        seq_start = torch.from_numpy(starts).to(dev)
        seq_len = torch.from_numpy(elens.astype(np.int32)).to(dev)
        qs = self.dec.qs                                    # same tokens: pos = len - 1
        M = self.dec.M
        P = ex["encoder_pool_blocks"]
        self.enc_groups, self.enc_tensors = [], []
        swa_start = torch.from_numpy((np.arange(M) * W).astype(np.int32)).to(dev)
        swa_count = torch.from_numpy(np.minimum(W, tokens).astype(np.int32)).to(dev)

        def layer_tensors(layer):
            qb = synth.q_main(wl.cfg, layer, M, H, D, "bf16")
            q = torch.from_numpy(qb.view(np.int16)).to(dev).view(torch.bfloat16)
            rows = np.concatenate([synth.swa_rows(wl.cfg, layer, s, W, D) for s in range(M)])
            sc = torch.empty((M * W, D), **u8)
            ss = torch.empty((M * W,), dtype=torch.float32, device=dev)
            csa2.csa2_quantize_fp8_rows(torch.from_numpy(rows).to(dev), sc, ss)
            sw = csa2.swa(sc, ss, swa_start, swa_count, D, W)
            return q, sw, torch.empty((M, H, D), dtype=torch.float32, device=dev), \
                torch.empty((M, H), dtype=torch.float32, device=dev)

        # encoder layers 0-1: window only
        self.swa_only = [layer_tensors(100 + l) for l in range(ex["swa_only_layers"])]
        layer = 100 + ex["swa_only_layers"]
        for gi, modes in enumerate(ex["encoder_groups"]):
            kc, ks = torch.empty((R, D // 2), **u8), torch.empty((R, D // 16), **u8)
            ic, is_ = torch.empty((R, DI // 2), **u8), torch.empty((R, DI // 16), **u8)
            chunk = 1 << 20
            for s in range(S):
                for c0 in range(0, int(elens[s]), chunk):
                    n = min(chunk, int(elens[s]) - c0)
                    x = torch.from_numpy(synth.main_kv_rows(wl.cfg + 100 + gi, s, c0, n, D)).to(dev)
                    r0 = int(starts[s]) + c0
                    csa2.csa2_quantize_fp4(x, kc[r0:r0 + n], ks[r0:r0 + n], w_ik=w_ik, ik_codes=ic[r0:r0 + n],
                                           ik_scales=is_[r0:r0 + n])
                    del x
            kv = csa2.fp4_cache(kc, ks, seq_start, seq_len, D, int(elens.max()), r)
            idx = csa2.fp4_cache(ic, is_, seq_start, seq_len, DI, int(elens.max()), r)
            # the entry each token completes comes from the compressor: the
            # sequence's last r token rows (bf16) times this group's W_c
            tok = np.concatenate([synth.token_rows(wl.cfg + 100 + gi, 0, s, r * (int(elens[s]) - 1), r, D)
                                  for s in range(S)])
            tok = torch.from_numpy(tok.view(np.int16)).to(dev)
            w_c = torch.from_numpy(synth.w_c(wl.cfg + 100, gi, D, r, D).view(np.int16)).to(dev)
            new_dst = torch.from_numpy(starts + elens - 1).to(dev)
            lt = [layer_tensors(layer + i) for i in range(len(modes))]
            qi = synth.q_idx(wl.cfg, layer, M, wl.idx_heads, DI)
            wi = synth.w_idx(wl.cfg, layer, M, wl.idx_heads)
            topk = torch.empty((M, K), dtype=torch.int32, device=dev)
            pool = torch.empty((M, P), dtype=torch.int32, device=dev)
            cnt = torch.empty((M,), dtype=torch.int32, device=dev)
            g = csa2.Group(csa2.CSA2_MODE_FULL, kv, idx, qs,
                           torch.from_numpy(qi.view(np.int16)).to(dev).view(torch.bfloat16),
                           torch.from_numpy(wi).to(dev), P, K, pool, cnt, topk, None,
                           [t[0] for t in lt], csa2.CSA2_BF16, H, [t[1] for t in lt], [t[2] for t in lt],
                           [t[3] for t in lt], D ** -0.5)
            g.topk_tensor = topk
            self.enc_groups.append(g)
            self.enc_tensors.append((kc, ks, ic, is_, (tok, w_c), new_dst, lt))
            self.w_ik_enc = w_ik
            layer += len(modes)
        ws_bytes = max([csa2.csa2_group_workspace_size(g) for g in self.enc_groups] +
                       [csa2.csa2_attn_workspace_size(M, H, D, 0, W), self.dec.ws.numel(),
                        csa2.csa2_group_steps_workspace_size(self.dec.groups)])
        self.ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)   # no initial contents needed
        self.M = M
        self.q_pos_host = self.dec.q_pos_host
        torch.cuda.synchronize()

    def step(self):
        csa2, dec = self.csa2, self.dec
        for q, sw, out, lse in self.swa_only:
            csa2.csa2_sparse_swa_attn(dec.kv, dec.qs, q, None, 0, sw, self.wl.dim ** -0.5, out, lse, self.ws)
        r = self.wl.extra["encoder_ratio"]
        for g, (kc, ks, ic, is_, (tok, w_c), dst, _) in zip(self.enc_groups, self.enc_tensors):
            csa2.csa2_compress_fp4(tok, r, w_c, kc, ks, dst_row=dst, w_ik=self.w_ik_enc, ik_codes=ic, ik_scales=is_)
            csa2.csa2_group_step(g, self.ws)
        csa2.csa2_group_steps(dec.groups, self.ws)

    def snapshot(self):
        t = self.torch
        a = self.dec.snapshot()
        enc = [g.topk_tensor.clone() for g in self.enc_groups]
        outs = [o.clone() for _, _, o, _ in self.swa_only] + [lt[2].clone() for e in self.enc_tensors for lt in e[6]]
        return (a[0] + enc, a[1], a[2] + outs, a[3])

    def scan_bytes_per_launch(self) -> int:
        # averaged over the step's first scans: the decoder's and the encoder groups'
        wl = self.wl
        idx_row = wl.idx_dim // 2 + wl.idx_dim // 16
        n_enc = len(wl.extra["encoder_groups"])
        return (self.dec.scan_bytes_per_launch() + n_enc * int(self.elens.sum()) * idx_row) // (1 + n_enc)

    @property
    def attn_layers(self) -> int:
        ex = self.wl.extra
        return self.wl.n_layers + sum(len(g) for g in ex["encoder_groups"]) + ex["swa_only_layers"]

    def attn_bytes_per_launch(self) -> int:
        # averaged over the step's layers (the window-only ones read no selected rows)
        wl = self.wl
        ex = wl.extra
        D, H, W = wl.dim, wl.heads, wl.window
        n_sparse = wl.n_layers + sum(len(g) for g in ex["encoder_groups"])
        swa_per_q = W * (D + 4) + H * D * 2 + H * D * 4 + H * 4
        tot = n_sparse * self.dec.attn_bytes_per_launch() + ex["swa_only_layers"] * self.M * swa_per_q
        return tot // (n_sparse + ex["swa_only_layers"])

    def step_bytes(self) -> int:
        wl = self.wl
        D, H, W, K = wl.dim, wl.heads, wl.window, wl.top_k
        ex = wl.extra
        idx_row = wl.idx_dim // 2 + wl.idx_dim // 16
        kv_row = D // 2 + D // 16
        attn_per_q = K * kv_row + W * (D + 4) + H * D * 2 + H * D * 4 + H * 4
        swa_per_q = W * (D + 4) + H * D * 2 + H * D * 4 + H * 4
        n_enc_layers = sum(len(g) for g in ex["encoder_groups"])
        enc = 0
        for _ in ex["encoder_groups"]:
            enc += int(self.elens.sum()) * idx_row                              # first scan
            enc += self.M * 8 * ex["encoder_pool_blocks"] * idx_row             # re-score of the pool
            r = ex["encoder_ratio"]
            enc += self.M * (r * D * 2 + 2 * kv_row + idx_row) + 2 * D * r * D  # compressor + key derivation
        enc += n_enc_layers * self.M * attn_per_q + ex["swa_only_layers"] * self.M * swa_per_q
        return self.dec.step_bytes() + enc

    def cache_bytes_per_token(self) -> float:
        # global (FP4) entries per token: the decoder's at ratio 1, each encoder Full layer's at its ratio
        wl = self.wl
        row = wl.dim // 2 + wl.dim // 16 + wl.idx_dim // 2 + wl.idx_dim // 16
        ex = wl.extra
        return row + len(ex["encoder_groups"]) * row / ex["encoder_ratio"]


class PrefillWorkload:
    """Encoder prefill chunk: each Full group has its own main-KV and indexer
    caches (a Full layer computes its own main KV), writes the chunk's new
    entries into them, selects flat Top-K lists for all its queries and runs
    its layers."""

    def __init__(self, wl, torch, csa2, synth):
        self.wl, self.torch, self.csa2 = wl, torch, csa2
        dev = torch.device("cuda:0")
        E, D, DI, ratio = int(wl.seq_lens[0]), wl.dim, wl.idx_dim, wl.ratio
        M, t0 = wl.n_queries, wl.first_query_token
        R = M // ratio                                    # entries completed by the chunk's tokens
        self.R = R
        u8 = dict(dtype=torch.uint8, device=dev)
        w_ik = torch.from_numpy(synth.w_ik(wl.cfg, D, DI)).to(dev)
        self.w_ik = w_ik
        self.new_dst = torch.arange(E - R, E, dtype=torch.int64, device=dev)
        seq_start = torch.zeros(1, dtype=torch.int64, device=dev)
        seq_len = torch.tensor([E], dtype=torch.int32, device=dev)
        # per Full group: its caches (the earlier entries written once at set-up)
        # and its compressor: the chunk's M token rows (bf16) and W_c, whose
        # R = M / ratio entries the step writes with their indexer keys
        self.caches = []
        for gi in range(len(wl.groups)):
            kc, ks = torch.empty((E, D // 2), **u8), torch.empty((E, D // 16), **u8)
            ic, is_ = torch.empty((E, DI // 2), **u8), torch.empty((E, DI // 16), **u8)
            x = torch.from_numpy(synth.main_kv_rows(wl.cfg, gi, 0, E - R, D)).to(dev)
            csa2.csa2_quantize_fp4(x, kc[:E - R], ks[:E - R], w_ik=w_ik, ik_codes=ic[:E - R], ik_scales=is_[:E - R])
            del x
            tok = torch.from_numpy(synth.token_rows(wl.cfg, gi, 0, t0, M, D).view(np.int16)).to(dev)
            w_c = torch.from_numpy(synth.w_c(wl.cfg, gi, D, ratio, D).view(np.int16)).to(dev)
            kv = csa2.fp4_cache(kc, ks, seq_start, seq_len, D, E, ratio)
            idx = csa2.fp4_cache(ic, is_, seq_start, seq_len, DI, E, ratio)
            self.caches.append((kv, idx, (tok, w_c), (kc, ks, ic, is_)))
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
            del qb
            sc = torch.empty((nsw, D), **u8)
            ss = torch.empty((nsw,), dtype=torch.float32, device=dev)
            csa2.csa2_quantize_fp8_rows(torch.from_numpy(synth.swa_rows(wl.cfg, layer, 0, nsw, D)).to(dev), sc, ss)
            self.swa.append(csa2.swa(sc, ss, swa_start, swa_count, D, W))
            self.out.append(torch.empty((M, H, D), dtype=torch.float32, device=dev))
            self.lse.append(torch.empty((M, H), dtype=torch.float32, device=dev))
        self.groups = []
        layer = 0
        for gi, modes in enumerate(wl.groups):
            n = len(modes)
            kv, idx, _, _ = self.caches[gi]
            qi = synth.q_idx(wl.cfg, layer, M, wl.idx_heads, DI)
            wi = synth.w_idx(wl.cfg, layer, M, wl.idx_heads)
            topk = torch.empty((M, K), dtype=torch.int32, device=dev)
            g = csa2.Group(csa2.CSA2_MODE_FULL, kv, idx, self.qs,
                           torch.from_numpy(qi.view(np.int16)).to(dev).view(torch.bfloat16),
                           torch.from_numpy(wi).to(dev), 0, K, None, None, topk, None,
                           self.q[layer:layer + n], csa2.CSA2_BF16, H, self.swa[layer:layer + n],
                           self.out[layer:layer + n], self.lse[layer:layer + n], D ** -0.5)
            g.topk_tensor = topk
            self.groups.append(g)
            layer += n
        ws_bytes = max(csa2.csa2_group_workspace_size(g) for g in self.groups)
        self.ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)   # no initial contents needed
        torch.cuda.synchronize()

    def step(self):
        csa2 = self.csa2
        for g, (_, _, (tok, w_c), (kc, ks, ic, is_)) in zip(self.groups, self.caches):
            csa2.csa2_compress_fp4(tok, self.wl.ratio, w_c, kc, ks, dst_row=self.new_dst, w_ik=self.w_ik,
                                   ik_codes=ic, ik_scales=is_)
            csa2.csa2_group_step(g, self.ws)

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

    def write_bytes_per_launch(self) -> int:
        # the key derivation: the written FP4 rows read back, their FP4 indexer keys, the destination rows, W_ik
        wl = self.wl
        D, DI = wl.dim, wl.idx_dim
        return self.R * (D // 2 + D // 16 + DI // 2 + DI // 16 + 8) + 4 * D * DI

    def compress_flops_per_launch(self) -> float:
        wl = self.wl
        return 2.0 * self.R * (wl.ratio * wl.dim) * wl.dim

    def compress_bytes_per_launch(self) -> int:
        # bf16 token rows and W_c, the FP4 entries written, the destination rows
        wl = self.wl
        D, K = wl.dim, wl.ratio * wl.dim
        return self.R * (2 * K + D // 2 + D // 16 + 8) + 2 * D * K


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def _blas_cores() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


class CpuDecodeModel:
    """The oracle's cost of one decode token through the 20-layer decoder,
    measured on the first 65,536 entries of a sequence and split into the part
    that grows with the visible context (FP4 decode of every indexer key, its
    scores, the block maxima and the pool ranking) and the part bounded by the
    pool, the Top-K and the window (re-scoring, Top-K, attention)."""

    NS = 65536

    def __init__(self, wl, synth):
        from oracle import attention, codec, indexer
        ns, D, DI = self.NS, wl.dim, wl.idx_dim
        x = synth.main_kv_rows(wl.cfg, 0, 0, ns, D)
        kc, ks = codec.fp4_encode(x)
        ikc, iks = codec.indexer_key(kc, ks, synth.w_ik(wl.cfg, D, DI))
        del x
        W, H = wl.window, wl.heads
        q_layers = [synth.bf16_bits_to_f32(synth.q_main(wl.cfg, l, 1, H, D, "bf16"))[0]
                    for l in range(wl.n_layers)]
        swa = [codec.fp8_rows_encode(synth.swa_rows(wl.cfg, l, 0, W, D)) for l in range(wl.n_layers)]
        tau = D ** -0.5

        def one_token():
            t0 = time.perf_counter()
            t_ctx = 0.0
            layer = 0
            pool = keys = None
            for modes in wl.groups:
                qi = synth.bf16_bits_to_f32(synth.q_idx(wl.cfg, layer, 1, wl.idx_heads, DI))[0]
                wi = synth.w_idx(wl.cfg, layer, 1, wl.idx_heads)[0]
                if modes[0] == "full":
                    ts = time.perf_counter()
                    keys = codec.fp4_decode(ikc, iks)
                    s = indexer.scores(qi, wi, keys)
                    pool = indexer.pool_select(indexer.block_max(s), wl.pool_blocks)
                    t_ctx += time.perf_counter() - ts
                    cand = indexer.pool_positions(pool, ns)
                    sel = indexer.top_ids(s[cand], cand, min(wl.top_k, len(cand)))
                else:
                    sel, _ = indexer.reindex(qi, wi, keys, pool, wl.top_k)
                for _ in modes:
                    attention.sparse_swa_attention(q_layers[layer], kc, ks, sel, ns, swa[layer][0], swa[layer][1],
                                                   tau)
                    layer += 1
            return time.perf_counter() - t0, t_ctx

        one_token()
        runs = sorted(one_token() for _ in range(3))
        self.t_tok, self.t_ctx = runs[1]
        self.t_fixed = self.t_tok - self.t_ctx
        self.per_entry = self.t_ctx / ns
        self.cores = _blas_cores()

    def baseline(self, wl) -> dict:
        lens = np.asarray(wl.seq_lens, np.float64)
        t = float(np.sum(self.t_fixed + self.per_entry * lens))
        return {"value": len(lens) / t, "unit": "query-tokens/s", "cores": int(self.cores), "kind": "oracle",
                "sample": (f"NumPy fp64 oracle, one decode token through all {wl.n_layers} layers over the first "
                           f"{self.NS} entries of a sequence (median of 3: {self.t_tok * 1e3:.0f} ms, of which "
                           f"{self.t_ctx * 1e3:.0f} ms grow with the context: FP4 decode of the indexer keys, "
                           f"scores, block maxima and pool ranking); that part scaled linearly to each of the "
                           f"{len(lens)} sequences' visible entries ({int(lens.sum())} in all), the rest counted "
                           f"once per token")}


def cpu_baseline_prefill(wl, synth) -> dict:
    from oracle import attention, codec, indexer
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
    # the write path: the compressor with FP4 write and key derivation for 64
    # entries, counted as 1/ratio entry per query token and Full group
    from oracle import compressor
    ne = 64
    tok = synth.bf16_bits_to_f32(synth.token_rows(wl.cfg, 0, 0, 0, ne * wl.ratio, D))
    w_c = synth.bf16_bits_to_f32(synth.w_c(wl.cfg, 0, D, wl.ratio, D))
    w_ik = synth.w_ik(wl.cfg, D, DI)
    tw = []
    for _ in range(3):
        ts = time.perf_counter()
        compressor.compress_write(tok, w_c, wl.ratio, w_ik)
        tw.append(time.perf_counter() - ts)
    t_write = sorted(tw)[1] / ne / wl.ratio * len(wl.groups)
    t_full_ctx = t_tok + t_scan * (n_full / ns - 1.0) + t_write
    return {"value": 1.0 / t_full_ctx, "unit": "query-tokens/s", "cores": int(_blas_cores()), "kind": "oracle",
            "sample": (f"NumPy fp64 oracle, one prefill query through all {wl.n_layers} encoder layers over the "
                       f"first {ns} entries (median of 3: {t_tok * 1e3:.0f} ms, flat Top-K incl. FP4 decode of the "
                       f"keys {t_scan * 1e3:.0f} ms); the flat Top-K scaled linearly to {n_full} entries; plus "
                       f"the compressor write of {ne} entries scaled to 1/{wl.ratio} entry per token and Full "
                       f"group ({t_write * 1e3:.2f} ms)")}


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def same_snapshot(torch, a, b):
    return all(torch.equal(x, y) for x, y in zip(a[0] + [a[1]] + a[2] + a[3], b[0] + [b[1]] + b[2] + b[3]))


def capture(torch, W, steps):
    """One HIP graph holding `steps` steps of W (kernel launches only)."""
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for _ in range(steps):
                W.step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return graph


def time_steps(torch, W, steps, warmup, mode):
    """Milliseconds per step over `steps` timed steps (graph replay or eager
    launches), checked equal to an eager reference step."""
    for _ in range(warmup):
        W.step()
    torch.cuda.synchronize()
    ref = W.snapshot()
    graph = None
    if mode == "graph":
        graph = capture(torch, W, steps)
        graph.replay()                     # untimed replay, checked against eager
        torch.cuda.synchronize()
        if not same_snapshot(torch, ref, W.snapshot()):
            raise RuntimeError("graph replay differs from eager execution")
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    if graph is not None:
        graph.replay()
    else:
        for _ in range(steps):
            W.step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if not same_snapshot(torch, ref, W.snapshot()):
        raise RuntimeError("timed steps differ from the eager reference")
    del graph
    return t0.elapsed_time(t1) / steps, wall


def kernel_times(torch, csa2, W, steps):
    """Average launch durations of the first scan, the attention, the
    quantise-on-write and the compressor kernels from HIP events stamped by their own dispatches,
    over `steps` eager steps (events cannot be timed inside a graph replay)."""
    csa2.csa2_profile_scan(True)
    csa2.csa2_profile_attn(True)
    csa2.csa2_profile_write(True)
    csa2.csa2_profile_compress(True)
    try:
        for _ in range(steps):
            W.step()
        torch.cuda.synchronize()
        sc = csa2.csa2_profile_scan_read()
        at = csa2.csa2_profile_attn_read()
        wr = csa2.csa2_profile_write_read()
        cp = csa2.csa2_profile_compress_read()
    finally:
        csa2.csa2_profile_scan(False)
        csa2.csa2_profile_attn(False)
        csa2.csa2_profile_write(False)
        csa2.csa2_profile_compress(False)
    return {"scan": sc, "attn": at, "write": wr, "compress": cp, "steps": steps}


def time_cold(torch, W, reps):
    """Median milliseconds of one step (a one-step graph replay) when a 1 GiB
    scratch write just before it has evicted the L2s and the 256 MB Infinity
    Cache."""
    graph = capture(torch, W, 1)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    times = []
    for r in range(reps):
        scratch.fill_(r & 0xFF)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1))
    del scratch, graph
    return float(np.median(times)), float(np.min(times)), float(np.max(times))


def avg_ms(rec):
    ms, n = rec
    return ms / n if n else float("nan")


def decode_record(wl, W, ms_per_step, kt, mode) -> dict:
    """Step time, query-tokens/s and the first scan's roofline for a decode workload."""
    scan_ms = avg_ms(kt["scan"])
    scan_bytes = W.scan_bytes_per_launch()
    achieved = scan_bytes / (scan_ms / 1e3) / 1e9
    # attention time per layer: every attention kernel of the step (decode:
    # a logits and a P V kernel per group of layers) over the step's layers
    attn_ms = kt["attn"][0] / (kt["steps"] * W.attn_layers)
    attn_bytes = W.attn_bytes_per_launch()
    step_bytes = W.step_bytes()
    return {
        "workload": wl.name, "mode": mode, "ms_per_step": round(ms_per_step, 4),
        "value": round(W.M / (ms_per_step / 1e3), 1), "unit": "query-tokens/s",
        "sequences": len(wl.seq_lens), "visible_entries": int(np.sum(wl.seq_lens)),
        "roofline": {"bound": "hbm", "kernel": "first scan (k_scan)", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "avg_launch_ms": round(scan_ms, 5), "algorithmic_bytes_per_launch": scan_bytes},
        "attention": {"kernels": "k_attn_logits + k_attn_pv per batch of up to 24 layers across groups",
                      "launches_per_step": kt["attn"][1] // kt["steps"],
                      "ms_per_layer": round(attn_ms, 5),
                      "algorithmic_bytes_per_layer": attn_bytes,
                      "achieved_gbs": round(attn_bytes / (attn_ms / 1e3) / 1e9, 1)},
        "write_path_avg_launch_ms": round(avg_ms(kt["write"]), 5),
        "step_algorithmic_bytes": step_bytes,
        "step_algorithmic_gbs": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "step_frac_of_hbm_peak": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
    }


def run_prefill(args, wl, torch, csa2, synth) -> dict:
    t0 = time.time()
    W = PrefillWorkload(wl, torch, csa2, synth)
    setup_s = time.time() - t0
    print(f"[bench] setup {setup_s:.1f}s: {wl.name}, {W.M} queries over {wl.seq_lens[0]} entries",
          file=sys.stderr, flush=True)
    ms_per_step, wall = time_steps(torch, W, args.steps, args.warmup, "eager")
    kt = kernel_times(torch, csa2, W, args.steps)
    assert kt["scan"][1] == args.steps * len(wl.groups) and kt["attn"][1] == args.steps * wl.n_layers, kt
    assert kt["write"][1] == args.steps * len(wl.groups) and kt["compress"][1] == args.steps * len(wl.groups), kt
    at_avg, sc_avg, wr_avg = avg_ms(kt["attn"]), avg_ms(kt["scan"]), avg_ms(kt["write"])
    cp_avg = avg_ms(kt["compress"])
    cp_tf = W.compress_flops_per_launch() / (cp_avg / 1e3) / 1e12
    at_tf = W.attn_flops_per_launch() / (at_avg / 1e3) / 1e12
    sc_tf = W.scoring_flops_per_launch() / (sc_avg / 1e3) / 1e12
    wr_b = W.write_bytes_per_launch()
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
                   "layers": wl.n_layers, "layout": "3x(Full+5Reuse), flat Top-K, caches per Full group",
                   "write_path": "compressor over the chunk's token rows (ratio 2) + FP4 + derived keys",
                   "latent_dim": wl.dim, "heads": wl.heads, "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim,
                   "top_k": wl.top_k, "window": wl.window,
                   "storage": "FP4 E2M1/E4M3x16 main+indexer, FP8 E4M3 window"},
        "roofline": {"bound": "mfma", "kernel": "prefill attention (k_attn_prefill)", "achieved": round(at_tf, 1),
                     "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(at_tf / F16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": None, "avg_launch_ms": round(at_avg, 4),
                     "timing": "HIP events stamped by each attention dispatch (same steps run again)",
                     "algorithmic_flops_per_launch": W.attn_flops_per_launch()},
        "indexer_scoring": {"bound": "mfma", "kernel": "k_score_mq", "achieved": round(sc_tf, 1),
                            "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(sc_tf / F16_MFMA_PEAK_TFLOPS, 4), "avg_launch_ms": round(sc_avg, 4),
                            "algorithmic_flops_per_launch": W.scoring_flops_per_launch()},
        "compressor": {"bound": "mfma", "kernel": "k_compress_fp4 (fp64 matrix cores, FP4 write fused)",
                       "entries_per_launch": W.R, "k": wl.ratio * wl.dim, "achieved": round(cp_tf, 2),
                       "peak": F64_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(cp_tf / F64_MFMA_PEAK_TFLOPS, 4),
                       "avg_launch_ms": round(cp_avg, 5),
                       "algorithmic_flops_per_launch": W.compress_flops_per_launch(),
                       "algorithmic_bytes_per_launch": W.compress_bytes_per_launch()},
        "quantize_on_write": {"bound": "hbm", "kernel": "k_quantize_fp4_derive_mfma (keys of the rows just written)",
                              "rows_per_launch": W.R,
                              "avg_launch_ms": round(wr_avg, 5), "algorithmic_bytes_per_launch": wr_b,
                              "achieved_gbs": round(wr_b / (wr_avg / 1e3) / 1e9, 1),
                              "frac": round(wr_b / (wr_avg / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "wall_s_timed": round(wall, 4),
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        t0 = time.time()
        result["cpu_baseline"] = cpu_baseline_prefill(wl, synth)
        print(f"[bench] prefill cpu baseline {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    del W
    torch.cuda.empty_cache()
    return result


def setup_decode(wl, torch, csa2, synth, schedule="steps"):
    t0 = time.time()
    W = DecodeWorkload(wl, torch, csa2, synth, schedule=schedule)
    setup_s = time.time() - t0
    print(f"[bench] setup {setup_s:.1f}s: {wl.name}, {len(wl.seq_lens)} seqs, {sum(wl.seq_lens)} entries",
          file=sys.stderr, flush=True)
    return W, setup_s


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
        result = run_prefill(args, wl, torch, csa2, synth)
        print(json.dumps(result), flush=True)
        return
    assert wl.phase == "decode", wl.phase
    W, setup_s = setup_decode(wl, torch, csa2, synth)
    ms_per_step, wall = time_steps(torch, W, args.steps, args.warmup, args.mode)
    kt = kernel_times(torch, csa2, W, args.steps)
    assert kt["scan"][1] == args.steps and kt["attn"][1] > 0, kt

    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    rec = decode_record(wl, W, ms_per_step, kt, args.mode)
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "scan_traffic.json")
    if os.path.exists(tpath):
        trec = json.load(open(tpath))
        if trec.get("source_sha256") == scan_source_sha256() and trec.get("workload") == wl.name:
            traffic = trec.get("bytes_per_launch")
    roofline = dict(rec["roofline"])
    roofline["traffic"] = traffic
    roofline["timing"] = "HIP events stamped by each first-scan dispatch" + (
        " (same steps run eagerly after the timed graph replay)" if args.mode == "graph" else "")
    result = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "sequences": len(wl.seq_lens), "context": max(wl.seq_lens),
                   "layers": wl.n_layers, "layout": "Full+3Reuse, 4x(Reindex+3Reuse)", "latent_dim": wl.dim,
                   "schedule": "csa2_group_steps: indexers in group order, then attention batched across groups",
                   "heads": wl.heads, "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim,
                   "pool_blocks": wl.pool_blocks, "top_k": wl.top_k, "window": wl.window,
                   "storage": "FP4 E2M1/E4M3x16 main+indexer, FP8 E4M3 window", "mode": args.mode},
        "roofline": roofline,
        "attention": dict(rec["attention"], bound="latency (one layer's reads are ~1.6 MB)"),
        "write_path_avg_launch_ms": rec["write_path_avg_launch_ms"],
        "step_algorithmic_bytes": rec["step_algorithmic_bytes"],
        "step_algorithmic_gbs": rec["step_algorithmic_gbs"],
        "step_frac_of_hbm_peak": rec["step_frac_of_hbm_peak"],
        "wall_s_timed": round(wall, 4),
        "setup_s": round(setup_s, 1),
    }
    model = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        model = CpuDecodeModel(wl, synth)
        result["cpu_baseline"] = model.baseline(wl)
        print(f"[bench] cpu baseline {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    if not args.no_extras:
        extras = {}
        # the headline workload: the other launch mode, and cold caches
        other = "eager" if args.mode == "graph" else "graph"
        ms_o, _ = time_steps(torch, W, args.steps, 1, other)
        extras[f"{wl.name}/{other}"] = decode_record(wl, W, ms_o, kt, other)
        med, lo, hi = time_cold(torch, W, args.cold_reps)
        cold = decode_record(wl, W, med, kt, "graph, cold caches")
        cold["cold"] = {"reps": args.cold_reps, "median_ms": round(med, 4), "min_ms": round(lo, 4),
                        "max_ms": round(hi, 4),
                        "method": "1 GiB scratch written before each one-step graph replay"}
        extras[f"{wl.name}/cold"] = cold
        del W
        torch.cuda.empty_cache()
        # the same step group by group (csa2_group_step per group), and issued
        # layer by layer (a group step for each group's first layer, one
        # attention call per Reuse layer), as a model would
        for sched, label, kern in (("groups", "group-by-group", "k_attn_logits + k_attn_pv per group"),
                                   ("layers", "layer-sequential", "k_attn_logits + k_attn_pv per layer")):
            Ws, _ = setup_decode(wl, torch, csa2, synth, schedule=sched)
            kts = kernel_times(torch, csa2, Ws, args.steps)
            mss, _ = time_steps(torch, Ws, args.steps, args.warmup, "graph")
            rs = decode_record(wl, Ws, mss, kts, f"graph, {label}")
            rs["attention"]["kernels"] = kern
            extras[f"{wl.name}/{label}"] = rs
            del Ws
            torch.cuda.empty_cache()
        for cfg in (1, 3):
            wx = synth.workload(cfg)
            Wx, _ = setup_decode(wx, torch, csa2, synth)
            ktx = kernel_times(torch, csa2, Wx, args.steps)
            for mode in (("graph", "eager") if cfg == 1 else ("graph",)):
                msx, _ = time_steps(torch, Wx, args.steps, args.warmup, mode)
                r = decode_record(wx, Wx, msx, ktx, mode)
                if model is not None:
                    r["cpu_baseline"] = model.baseline(wx)
                extras[f"{wx.name}/{mode}"] = r
            del Wx
            torch.cuda.empty_cache()
        for cfg in (6, 7):
            wx = synth.workload(cfg)
            Wx, _ = setup_decode(wx, torch, csa2, synth)
            ktx = kernel_times(torch, csa2, Wx, args.steps)
            msx, _ = time_steps(torch, Wx, args.steps, args.warmup, "graph")
            r = decode_record(wx, Wx, msx, ktx, "graph")
            r["tokens_per_sequence"] = Wx.T
            r["scan_bytes_per_token"] = Wx.scan_bytes_per_launch() / Wx.M
            r["roofline"]["kernel"] = ("first scan (k_scan_run: the run's tokens share each streamed tile)"
                                       if Wx.T in (2, 4) else
                                       "first scan (k_score_mq: every row scored against the run's tokens)")
            extras[f"{wx.name}/graph"] = r
            del Wx
            torch.cuda.empty_cache()
        wc = synth.workload(5)
        t0 = time.time()
        Wc = CedDecodeWorkload(wc, torch, csa2, synth)
        print(f"[bench] setup {time.time() - t0:.1f}s: {wc.name}", file=sys.stderr, flush=True)
        ktc = kernel_times(torch, csa2, Wc, args.steps)
        msc, _ = time_steps(torch, Wc, args.steps, args.warmup, "graph")
        rc = decode_record(wc, Wc, msc, ktc, "graph")
        rc["layers"] = "2 window-only + 3x(Full+5Reuse) at ratio 2 + decoder 20"
        rc["global_cache_bytes_per_token"] = Wc.cache_bytes_per_token()
        rc["compressor_avg_launch_ms"] = round(avg_ms(ktc["compress"]), 5)
        rc["write_path"] = ("encoder groups: k_compress_fp4 (ratio 2, one entry per sequence) + key derivation; "
                            "decoder: quantise-on-write of given rows")
        extras[f"{wc.name}/graph"] = rc
        del Wc
        torch.cuda.empty_cache()
        wp = synth.workload(2)
        pre = run_prefill(args, wp, torch, csa2, synth)
        extras[wp.name] = {k: pre[k] for k in ("metric", "value", "unit", "ms_per_step", "config", "roofline",
                                                "indexer_scoring", "compressor", "quantize_on_write",
                                                "cpu_baseline")
                           if k in pre}
        result["workloads"] = extras
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
