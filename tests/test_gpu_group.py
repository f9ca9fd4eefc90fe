"""GPU parity of csa2_group_step (write path + indexer + per-layer attention).

Downstream steps are checked teacher-forced: a pool that differs from the
oracle's inside the near-tie band is accepted, and the oracle then takes the
Top-K from the GPU's pool; a Reindex group re-scores the GPU's pool; every
layer's attention is compared with the oracle's attention over the GPU's own
Top-K list, so no group is left unchecked when its list differs legally.
"""
import numpy as np
import pytest
import torch

import fp4_kv_cache_02_amd as csa2
import synth
from oracle import attention, codec, group as ogroup, indexer
from tests._gpu_util import announce, assert_sets_equal_modulo_band, dev, empty_u8, h, random_group, t, workspace

pytestmark = pytest.mark.gpu


def _check_attn_one(o_ref, l_ref, go, gl):
    for hh in range(o_ref.shape[0]):
        den = np.abs(o_ref[hh]).max()
        assert np.abs(go[hh] - o_ref[hh]).max() <= 2e-3 * den, hh
        assert abs(gl[hh] - l_ref[hh]) <= 1e-3, hh


class _Decoder:
    """A decode batch (one token per sequence) and its caches, on the GPU and
    as the oracle's arrays (the state after the Full group's write)."""

    def __init__(self, cfg, lens, D, H, qdt, DI, HI, P, K, W, raw):
        self.cfg, self.lens, self.D, self.H, self.qdt = cfg, list(lens), D, H, qdt
        self.DI, self.HI, self.P, self.K, self.W = DI, HI, P, K, W
        M = self.M = len(lens)
        self.starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        n_tot = int(sum(lens))
        self.dst = (self.starts + np.asarray(lens) - 1).astype(np.int64)   # the decode token's entry
        self.w_ik = synth.w_ik(cfg, D, DI)
        # the new latent rows the Full group writes (one per sequence)
        self.new_x = synth.gaussian_rows(cfg, synth.TAG_MAIN_KV, 1, 0, 0, M, D)
        nc, ns = codec.fp4_encode(self.new_x)
        nic, nis = codec.indexer_key(nc, ns, self.w_ik)
        if raw:
            # caches drawn as raw FP4 bytes (no quantisation pass needed)
            rc, rs = synth.fp4_bytes(cfg, 0, n_tot, D)
            ikc, iks = synth.fp4_bytes(cfg, 1, n_tot, DI)
        else:
            x = np.concatenate([synth.main_kv_rows(cfg, s, 0, n, D) for s, n in enumerate(lens)])
            rc, rs = codec.fp4_encode(x)
            ikc, iks = codec.indexer_key(rc, rs, self.w_ik)
            del x
        # device caches hold the state before the step (rows dst not yet written: zero)
        kv_c, kv_s, ik_c, ik_s = (t(a.copy()) for a in (rc, rs, ikc, iks))
        for z in (kv_c, kv_s, ik_c, ik_s):
            z[t(self.dst)] = 0
        rc[self.dst], rs[self.dst], ikc[self.dst], iks[self.dst] = nc, ns, nic, nis
        self.ref = (rc, rs, ikc, iks)
        self.dev = (kv_c, kv_s, ik_c, ik_s)
        self.keys = [codec.fp4_decode(ikc[s0:s0 + n], iks[s0:s0 + n]).astype(np.float32)
                     for s0, n in zip(self.starts, lens)]
        st, ln = t(self.starts), t(np.asarray(lens, np.int32))
        self.kv = csa2.fp4_cache(kv_c, kv_s, st, ln, D, max(lens), 1)
        self.idx = csa2.fp4_cache(ik_c, ik_s, st, ln, DI, max(lens), 1)
        self.q_pos = (np.asarray(lens) - 1).astype(np.int32)
        self.qs = csa2.queries(t(np.arange(M, dtype=np.int32)), t(self.q_pos))
        self.pool = torch.full((M, P), -7, dtype=torch.int32, device=dev())
        self.cnt = torch.full((M,), -7, dtype=torch.int32, device=dev())

    def layers(self, layer0, n_layers):
        M, H, D, W = self.M, self.H, self.D, self.W
        q_list, swa_list, out_list, lse_list, ref = [], [], [], [], []
        for layer in range(layer0, layer0 + n_layers):
            q = synth.q_main(self.cfg, layer, M, H, D, self.qdt)
            sw = synth.swa_rows(self.cfg, layer, 0, M * W, D)
            sc, ss = empty_u8(M * W, D), torch.empty((M * W,), dtype=torch.float32, device=dev())
            csa2.csa2_quantize_fp8_rows(t(sw), sc, ss)
            swa_list.append(csa2.swa(sc, ss, t(np.arange(M, dtype=np.int32) * W), t(np.full(M, W, np.int32)), D, W))
            if self.qdt == "f32":
                q_list.append(t(q))
                qf = q.astype(np.float64)
            else:
                q_list.append(t(q).view(torch.bfloat16))
                qf = synth.bf16_bits_to_f32(q).astype(np.float64)
            out_list.append(torch.empty((M, H, D), dtype=torch.float32, device=dev()))
            lse_list.append(torch.empty((M, H), dtype=torch.float32, device=dev()))
            sc8, ss8 = codec.fp8_rows_encode(sw)
            assert np.array_equal(h(sc), sc8) and np.array_equal(h(ss), ss8)
            ref.append((qf, sc8, ss8))
        return q_list, swa_list, out_list, lse_list, ref

    def run_group(self, mode, layer0, n_layers):
        full = mode == "full"
        qi, wi = synth.q_idx(self.cfg, layer0, self.M, self.HI, self.DI), synth.w_idx(self.cfg, layer0, self.M, self.HI)
        q_list, swa_list, out_list, lse_list, ref_layers = self.layers(layer0, n_layers)
        topk = torch.full((self.M, self.K), -7, dtype=torch.int32, device=dev())
        g = csa2.Group(csa2.CSA2_MODE_FULL if full else csa2.CSA2_MODE_REINDEX, self.kv, self.idx, self.qs,
                       t(qi).view(torch.bfloat16), t(wi), self.P, self.K, self.pool, self.cnt, topk, None, q_list,
                       csa2.CSA2_F32 if self.qdt == "f32" else csa2.CSA2_BF16, self.H, swa_list, out_list, lse_list,
                       self.D ** -0.5, new_kv=t(self.new_x) if full else None,
                       new_dst_row=t(self.dst) if full else None, w_ik=t(self.w_ik) if full else None)
        ws = workspace(csa2.csa2_group_workspace_size(g))
        csa2.csa2_group_step(g, ws)
        rc, rs, ikc, iks = self.ref
        if full:
            kv_c, kv_s, ik_c, ik_s = self.dev
            assert np.array_equal(h(kv_c), rc) and np.array_equal(h(kv_s), rs), "main cache after the write"
            assert np.array_equal(h(ik_c), ikc) and np.array_equal(h(ik_s), iks), "indexer keys after the write"
        qf = synth.bf16_bits_to_f32(qi)
        gpool, gcnt, gtopk = h(self.pool), h(self.cnt), h(topk)
        outs = [(h(o), h(l)) for o, l in zip(out_list, lse_list)]
        n_band = 0
        for i in range(self.M):
            s0, vis = int(self.starts[i]), int(self.lens[i])
            keys = self.keys[i][:vis]
            pool_i = gpool[i][:gcnt[i]]
            if full:
                opool, ocnt, _, s = indexer.index_full(qf[i], wi[i], keys, self.P, self.K)
                assert gcnt[i] == ocnt and np.all(gpool[i][ocnt:] == -1) and np.all(np.diff(pool_i) > 0)
                bm = indexer.block_max(s)
                n_band += assert_sets_equal_modulo_band(pool_i, opool[:ocnt], lambda b: bm[b], self.P, what="pool")
            # the list from the GPU's pool (a Full layer takes its Top-K from its own pool)
            otopk, s_c = indexer.reindex(qf[i], wi[i], keys, pool_i, self.K)
            cand = indexer.pool_positions(pool_i, vis)
            score = dict(zip(cand.tolist(), s_c.tolist()))
            sel = gtopk[i][gtopk[i] >= 0]
            nsel = int((otopk >= 0).sum())
            assert len(sel) == nsel and np.all(gtopk[i][nsel:] == -1) and np.all(np.diff(sel) > 0)
            n_band += assert_sets_equal_modulo_band(sel, otopk[:nsel], lambda j: np.array([score[int(x)] for x in j]),
                                                    self.K, what=f"{mode} topk q{i}")
            # every layer on the GPU's list (Reuse layers share it)
            for layer, (qf_l, sc8, ss8) in enumerate(ref_layers):
                o_ref, l_ref = attention.sparse_swa_attention(
                    qf_l[i], rc[s0:s0 + vis], rs[s0:s0 + vis], indexer.reuse(gtopk[i]), vis,
                    sc8[i * self.W:(i + 1) * self.W], ss8[i * self.W:(i + 1) * self.W], self.D ** -0.5)
                _check_attn_one(o_ref, l_ref, outs[layer][0][i], outs[layer][1][i])
        return n_band


@pytest.mark.parametrize("shape", ["c0", "c1_20_layers", "c3_ragged_20_layers"])
def test_decoder_groups_match_oracle(shape):
    """Decode groups in the decoder's layout: C0 (Full + 3 Reuse, fp32
    queries), the 64K decoder through all 5 groups / 20 layers, and the ragged
    batch of 32 sequences (32K..256K entries each, caches drawn as raw FP4
    bytes) through all 20 layers."""
    if shape == "c0":
        dec = _Decoder(0, [4096], 128, 8, "f32", 64, 4, 64, 64, 128, raw=False)
        modes = ["full"]
    elif shape == "c1_20_layers":
        dec = _Decoder(1, [65536], 512, 64, "bf16", 128, 8, 2048, 512, 128, raw=False)
        modes = ["full"] + ["reindex"] * 4
    else:
        dec = _Decoder(3, synth.workload(3).seq_lens, 512, 64, "bf16", 128, 8, 2048, 512, 128, raw=True)
        modes = ["full"] + ["reindex"] * 4
    layer0 = 0
    for mode in modes:
        announce("group step", shape, mode, "layers", layer0, layer0 + 3)
        dec.run_group(mode, layer0, 4)
        layer0 += 4


def test_encoder_group_step_matches_oracle():
    """One encoder group (Full + 5 Reuse, flat Top-512, ratio 2) over a
    256-token prefill chunk: tokens 3840 .. 4095 of a 4,096-token prompt, so
    the chunk writes the last 128 of the 2,048 compressed entries and every
    query sees 1,920 .. 2,048 of them.  The write path is checked byte for
    byte, every query's list against the oracle's flat Top-K (modulo the
    near-tie band), and the six layers' outputs of 32 sampled queries on the
    GPU's own lists."""
    cfg, E, D, H, DI, HI, K, W, ratio, n_layers = 330, 2048, 512, 64, 128, 8, 512, 128, 2, 6
    T, M = ratio * E, 256
    R = M // ratio
    announce("encoder group step", E, M)
    x = synth.main_kv_rows(cfg, 0, 0, E, D)
    w_ik = synth.w_ik(cfg, D, DI)
    kv_c, kv_s = empty_u8(E, D // 2), empty_u8(E, D // 16)
    ik_c, ik_s = empty_u8(E, DI // 2), empty_u8(E, DI // 16)
    for z in (kv_c, kv_s, ik_c, ik_s):
        z.zero_()
    csa2.csa2_quantize_fp4(t(x[:E - R]), kv_c, kv_s, w_ik=t(w_ik), ik_codes=ik_c, ik_scales=ik_s)
    rc, rs = codec.fp4_encode(x)
    ikc, iks = codec.indexer_key(rc, rs, w_ik)
    seq_start, seq_len = t(np.zeros(1, np.int64)), t(np.array([E], np.int32))
    kv = csa2.fp4_cache(kv_c, kv_s, seq_start, seq_len, D, E, ratio)
    idx = csa2.fp4_cache(ik_c, ik_s, seq_start, seq_len, DI, E, ratio)
    q_pos = np.arange(T - M, T, dtype=np.int32)
    qs = csa2.queries(t(np.zeros(M, np.int32)), t(q_pos))
    qi, wi = synth.q_idx(cfg, 0, M, HI, DI), synth.w_idx(cfg, 0, M, HI)
    q_list, swa_list, out_list, lse_list, swx_list, qh_list = [], [], [], [], [], []
    nsw = M + W - 1
    for layer in range(n_layers):
        qh_list.append(synth.q_main(cfg, layer, M, H, D, "bf16"))
        q_list.append(t(qh_list[-1]).view(torch.bfloat16))
        swx = synth.swa_rows(cfg, layer, 0, nsw, D)
        sc, ss = empty_u8(nsw, D), torch.empty((nsw,), dtype=torch.float32, device=dev())
        csa2.csa2_quantize_fp8_rows(t(swx), sc, ss)
        swa_list.append(csa2.swa(sc, ss, t(np.arange(M, dtype=np.int32)), t(np.full(M, W, np.int32)), D, W))
        swx_list.append((swx, sc, ss))
        out_list.append(torch.empty((M, H, D), dtype=torch.float32, device=dev()))
        lse_list.append(torch.empty((M, H), dtype=torch.float32, device=dev()))
    topk = torch.full((M, K), -7, dtype=torch.int32, device=dev())
    g = csa2.Group(csa2.CSA2_MODE_FULL, kv, idx, qs, t(qi).view(torch.bfloat16), t(wi), 0, K, None, None, topk, None,
                   q_list, csa2.CSA2_BF16, H, swa_list, out_list, lse_list, D ** -0.5,
                   new_kv=t(x[E - R:]), new_dst_row=t(np.arange(E - R, E, dtype=np.int64)), w_ik=t(w_ik))
    ws = workspace(csa2.csa2_group_workspace_size(g))
    csa2.csa2_group_step(g, ws)
    assert np.array_equal(h(kv_c), rc) and np.array_equal(h(kv_s), rs)
    assert np.array_equal(h(ik_c), ikc) and np.array_equal(h(ik_s), iks)
    gtopk = h(topk)
    qf = synth.bf16_bits_to_f32(qi)
    keys = codec.fp4_decode(ikc, iks)
    exact = []
    for i in range(M):
        vis = indexer.visible_count(E, int(q_pos[i]), ratio)
        otopk, s = indexer.index_flat(qf[i], wi[i], keys[:vis], K)
        sel = gtopk[i][gtopk[i] >= 0]
        assert len(sel) == K and np.all(np.diff(sel) > 0)
        if assert_sets_equal_modulo_band(sel, otopk, lambda j: s[j], K, what="encoder topk") == 0:
            exact.append(i)
    # attention of all six layers, on the GPU's own lists (teacher-forced), for
    # 32 sampled queries including the chunk's first and last; where the list
    # equals the oracle's, the whole group composition is compared as well
    rng = np.random.default_rng(331)
    sample = sorted(set([0, M - 1] + rng.choice(M, 30, replace=False).tolist()))
    outs = [(h(o), h(l)) for o, l in zip(out_list, lse_list)]
    sc_h = [(h(sc), h(ss)) for _, sc, ss in swx_list]
    for i in sample:
        vis = indexer.visible_count(E, int(q_pos[i]), ratio)
        layers = []
        for layer, (swx, _, _) in enumerate(swx_list):
            c8, s8 = codec.fp8_rows_encode(swx[i:i + W])
            assert np.array_equal(sc_h[layer][0][i:i + W], c8) and np.array_equal(sc_h[layer][1][i:i + W], s8)
            qm = synth.bf16_bits_to_f32(qh_list[layer][i]).astype(np.float64)
            layers.append((qm, c8, s8))
        if i in exact:
            ref = ogroup.encoder_group_query(rc, rs, ikc, iks, int(q_pos[i]), ratio, qf[i], wi[i], K, layers,
                                             D ** -0.5)
            assert np.array_equal(gtopk[i], ref["idx"])
        for layer, (qm, c8, s8) in enumerate(layers):
            o_ref, l_ref = attention.sparse_swa_attention(qm, rc, rs, indexer.reuse(gtopk[i]), vis, c8, s8,
                                                          D ** -0.5)
            _check_attn_one(o_ref, l_ref, outs[layer][0][i], outs[layer][1][i])


def test_group_workspace_shared_by_groups_of_other_shapes():
    """One caller workspace, filled with garbage once, serves a large group,
    a smaller one and the large one again: no call depends on what an earlier
    call left there, so each result equals that of a fresh workspace (same
    kernels, same inputs: bit-identical)."""
    big, small = random_group(611, [70000, 33333], 3), random_group(612, [9000], 2)
    g_big, _ = big()
    shared = torch.full((csa2.csa2_group_workspace_size(g_big),), 0xA5, dtype=torch.uint8, device=dev())
    for label, outputs in (("large group", big), ("smaller group", small), ("large group again", big)):
        g_ref, ref = outputs()
        announce("group step, fresh workspace", label)
        csa2.csa2_group_step(g_ref, torch.zeros((csa2.csa2_group_workspace_size(g_ref),), dtype=torch.uint8,
                                                device=dev()))
        g_got, got = outputs()
        announce("group step, shared workspace", label)
        csa2.csa2_group_step(g_got, shared)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert np.array_equal(h(a), h(b), equal_nan=True), label
        assert not np.any(h(got[4]) == 7.0), label    # every output row written


def _stack(cfg, lens, modes, write_groups, P=2048, K=512, D=512, H=64, DI=128, HI=8, W=128, shared_cache=True):
    """A stack of decode groups over raw FP4 caches; returns a builder of fresh
    (groups, outputs) on fresh copies of the caches.  write_groups: indices of
    Full groups that also write one new entry per sequence."""
    M = len(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    n = int(sum(lens))
    n_caches = 1 if shared_cache else len(modes)
    raw = [(synth.fp4_bytes(cfg, 2 * c, n, D), synth.fp4_bytes(cfg, 2 * c + 1, n, DI)) for c in range(n_caches)]
    st, ln = t(starts), t(np.asarray(lens, np.int32))
    qs = csa2.queries(t(np.arange(M, dtype=np.int32)), t((np.asarray(lens) - 1).astype(np.int32)))
    w_ik = t(synth.w_ik(cfg, D, DI))
    layer_in = []
    for gi in range(len(modes)):
        qi, wi = synth.q_idx(cfg, gi, M, HI, DI), synth.w_idx(cfg, gi, M, HI)
        qs_l, sw_l = [], []
        for layer in range(4):
            qs_l.append(t(synth.q_main(cfg, 4 * gi + layer, M, H, D, "bf16")).view(torch.bfloat16))
            sc, ss = empty_u8(M * W, D), torch.empty((M * W,), dtype=torch.float32, device=dev())
            csa2.csa2_quantize_fp8_rows(t(synth.swa_rows(cfg, 4 * gi + layer, 0, M * W, D)), sc, ss)
            sw_l.append(csa2.swa(sc, ss, t(np.arange(M, dtype=np.int32) * W), t(np.full(M, W, np.int32)), D, W))
        new = t(synth.gaussian_rows(cfg, synth.TAG_MAIN_KV, 10 + gi, 0, 0, M, D))
        dst = t((starts + np.asarray(lens) - 1 - gi).astype(np.int64))
        layer_in.append((t(qi).view(torch.bfloat16), t(wi), qs_l, sw_l, new, dst))

    def build():
        caches = []
        for (rc, rs), (ic, is_) in raw:
            caches.append((t(rc), t(rs), t(ic), t(is_)))
        kvs = [(csa2.fp4_cache(c[0], c[1], st, ln, D, max(lens), 1), csa2.fp4_cache(c[2], c[3], st, ln, DI, max(lens), 1))
               for c in caches]
        pool = torch.full((M, P), -7, dtype=torch.int32, device=dev())
        cnt = torch.full((M,), -7, dtype=torch.int32, device=dev())
        groups, outs = [], [pool, cnt] + [x for c in caches for x in c]
        for gi, mode in enumerate(modes):
            kv, idx = kvs[0 if shared_cache else gi]
            qi, wi, q_l, sw_l, new, dst = layer_in[gi]
            topk = torch.full((M, K), -7, dtype=torch.int32, device=dev())
            score = torch.full((M, K), -7.0, dtype=torch.float32, device=dev())
            out = [torch.full((M, H, D), 7.0, dtype=torch.float32, device=dev()) for _ in range(4)]
            lse = [torch.full((M, H), 7.0, dtype=torch.float32, device=dev()) for _ in range(4)]
            wr = gi in write_groups
            g = csa2.Group(csa2.CSA2_MODE_FULL if mode == "full" else csa2.CSA2_MODE_REINDEX, kv, idx, qs, qi, wi, P,
                           K, pool, cnt, topk, score, q_l, csa2.CSA2_BF16, H, sw_l, out, lse, D ** -0.5,
                           new_kv=new if wr else None, new_dst_row=dst if wr else None, w_ik=w_ik if wr else None)
            g.keep = (kv, idx)
            groups.append(g)
            outs += [topk, score] + out + lse
        return groups, outs

    return build


@pytest.mark.parametrize("case", ["decoder_64k", "decoder_ragged_32", "writes_between", "own_caches",
                                  "ten_sets_one_pool", "flat_groups"])
def test_group_steps_equal_group_by_group(case):
    """csa2_group_steps (every group's index first, then the attention of all
    layers batched across groups) gives bit-identical results to
    csa2_group_step called group by group, which the tests above check
    against the oracle: the decoder's 5 groups at 64K and on the ragged
    32-sequence batch; a stack where a later Full group writes into the cache
    the earlier groups attend over; and Full groups with caches of their own."""
    if case == "decoder_64k":
        build = _stack(31, [65536], ["full"] + ["reindex"] * 4, {0})
    elif case == "decoder_ragged_32":
        build = _stack(32, synth.workload(3).seq_lens, ["full"] + ["reindex"] * 4, {0})
    elif case == "writes_between":
        build = _stack(33, [40000, 9000, 70001], ["full", "reindex", "full", "reindex"], {0, 2})
    elif case == "own_caches":
        build = _stack(34, [30000, 50000], ["full", "full", "full"], {0, 1, 2}, P=512, K=256, shared_cache=False)
    elif case == "ten_sets_one_pool":
        # more query sets on one pool than one re-score launch takes: a second
        # family headed by a Reindex group
        build = _stack(35, [20000, 44444], ["full"] + ["reindex"] * 9, {0}, P=256, K=128)
    else:
        # pool_blocks = 0: flat Top-K groups (the encoder's), one with a write
        build = _stack(36, [9000, 15001], ["full", "full"], {0}, P=0, K=128, shared_cache=False)
    announce("group steps", case)
    ref_groups, ref_out = build()
    for g in ref_groups:
        csa2.csa2_group_step(g, workspace(csa2.csa2_group_workspace_size(g)))
    ref = [h(x) for x in ref_out]
    groups, outs = build()
    csa2.csa2_group_steps(groups, workspace(csa2.csa2_group_steps_workspace_size(groups)))
    for i, (a, b) in enumerate(zip(ref, [h(x) for x in outs])):
        assert np.array_equal(a, b), i
