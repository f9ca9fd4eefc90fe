// CSA2 core attention, prefill schedule for the 512-channel shared latent
// with bf16 queries (the encoder chunk shape): selected FP4 main-KV entries
// concatenated with the query's own FP8 window rows, one joint softmax (P5
// figure caption of the attention diagram: Selection / Top-K /
// Concatenation; P1 CSA2 section).  Keys double as values (MQA over the
// latent), so every decoded key serves all 64 heads twice: once in
// S = Q K^T and once in O = P V.
//
// One workgroup per (query, 64 heads), one wave per SIMD.  The query's 64
// heads x 512 channels sit in the accumulation registers of every wave (they
// are only ever MFMA operands), which lets each wave take a different quarter
// of the keys and still see every head:
//
//   chunk of 64 key slots, wave w owns slots 16w .. 16w+15
//   S^T = K Q^T  : wave w decodes its 16 keys straight into MFMA A operands
//                  (FP4 x E4M3 -> exact f16, or E4M3 window codes) and meets
//                  the 64 heads held as B operands; the decoded keys are also
//                  written to an LDS tile [key][dim] for the second product;
//   softmax      : per-head chunk maxima meet in LDS; the running maximum is
//                  only raised when a chunk exceeds it by more than 2^8 (P
//                  then stays below 2^8 in f16, and the accumulator is
//                  rescaled rarely instead of on every chunk);
//   O^T = V^T P^T: wave w produces output channels 128w .. 128w+127 for all
//                  64 heads; V^T comes from the LDS tile through the
//                  transposing LDS load, P^T from the probability tile.
//
// The probability tile is double-buffered by chunk parity and the decoded-key
// tile is single, so three workgroup barriers per chunk suffice.  The next
// chunk's key bytes are loaded (buffer loads, invisible or empty slots at
// out-of-range offsets, which read zeros) while the current chunk is being
// computed.  The next query's heads are staged as f16 in LDS by the current
// query's chunks, two 16-byte parts per thread each, so a query switch reads
// its B operands from LDS instead of waiting for memory and converting them
// in every wave.
//
// Exactness as in the other schedules: FP4 and E4M3 entries are f16 numbers;
// bf16 queries convert to f16 exactly inside the f16 normal range; window
// rows carry an fp32 row scale r that multiplies the logits and the
// probabilities entering P V, with P lifted by a power of two 2^e (undone on
// the accumulator); P is rounded to f16; everything else accumulates in fp32.
#include "csa2_internal.hpp"
#include "csa2_indexer.hpp"

#include <algorithm>

namespace csa2 {

constexpr int kPD = 512;           // latent channels
constexpr int kPC = 64;            // key slots per chunk (16 per wave)
constexpr int kPH = 64;            // heads per workgroup (4 column tiles of 16)
constexpr int kPTs = kPD + 8;      // [key][dim] row stride of a decoded chunk (f16)
constexpr int kPPs = kPC + 8;      // [head][key] row stride of the probability tile (f16)
constexpr float kLazyMax = 8.0f;   // log2 headroom before the running maximum is raised

constexpr int kQParts = kPH * kPD / 8 / 256;  // 16-byte parts of a query's heads per thread (16)

struct alignas(16) PrefillLds {
  _Float16 t[kPC * kPTs];          // decoded keys of the current chunk
  _Float16 qn[kPH * kPTs];         // the next query's heads as f16 [head][channel]
  _Float16 p[2][kPH * kPPs];       // probabilities P[head][key], by item parity
  float cmax[2][kPH][4];           // per-wave chunk maxima of each head (log2 units)
  float rmax[2][4];                // per-wave maxima of the key scales
  float ks[2][kPC];                // per key slot: 1 (main entry), r (window row), 0 (empty)
  float lsum[kPH][4];              // per-wave softmax denominators of a query
};

// Loads of one lane's key for a chunk: the lane (key row, quad) holds
// channels quad*128 .. +127 of its key: 64 FP4 code bytes + 8 scale bytes of
// a main entry, or the first 64 of the 128 E4M3 bytes of a window row (the
// other 64 are read at the start of the chunk's item, from offset o2).
struct KeyBytes {
  uint32_t w[16];
  uint32_t s[2];
  uint32_t r;      // window row scale bits (0 for main entries)
  uint32_t o2;     // window rows: offset of the second 64 bytes
  float ks_main;   // main entries: 1 when the entry is visible, else 0; window rows: -1 (use r)
};
CSA2_DEV float key_scale(const KeyBytes &kb) { return kb.ks_main >= 0.0f ? kb.ks_main : __uint_as_float(kb.r); }

CSA2_DEV half8_t main_slice(const KeyBytes &kb, int kk) {
  const uint32_t sb = (kb.s[kk >> 3] >> (8 * ((kk >> 1) & 3))) & 0xFFu;
  return fp4x8_dequant_f16(kb.w[kk], e4m3x2_to_f16(sb)[0]);
}

// Position in a workgroup's stream of work items: chunk c of its k-th query.
struct Cursor {
  int k, c;
};

// Grid (G, ceil(H / 64)): workgroup x takes queries x, x + G, x + 2G, ... in
// batches of up to 64 (lane k of every wave holds the facts of the batch's
// k-th query) and walks their chunks as one stream, so the loads of the next
// query's first chunks overlap the current query's last ones.
__global__ __launch_bounds__(256) void k_attn_prefill(const uint16_t *__restrict__ q, int M, int H,
                                                      const uint8_t *__restrict__ kv_codes,
                                                      const uint8_t *__restrict__ kv_scales,
                                                      const int64_t *__restrict__ seq_start,
                                                      const int32_t *__restrict__ seq_len, int ratio,
                                                      const int32_t *__restrict__ q_seq,
                                                      const int32_t *__restrict__ q_pos,
                                                      const int32_t *__restrict__ topk, int K,
                                                      const uint8_t *__restrict__ swa_codes,
                                                      const float *__restrict__ swa_scale,
                                                      const int32_t *__restrict__ swa_start,
                                                      const int32_t *__restrict__ swa_count, int W, float tau2,
                                                      float *__restrict__ out, float *__restrict__ lse) {
  __shared__ PrefillLds L;
  const int G = gridDim.x, h0 = blockIdx.y * kPH;
  const int l = lane_id(), row = l & 15, quad = l >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NC = (K + W + kPC - 1) / kPC;  // chunks per query (slots past a query's window count are empty)
  const int hq = min(kPH, H - h0);          // heads of this block
  const float kNegInf = -INFINITY;

  for (int mb = blockIdx.x; mb < M; mb += 64 * G) {
    const int nq = min(64, (M - mb + G - 1) / G);
    // ---- facts of the batch's queries, lane k = query mb + k G ----
    int f_vis = 0, f_wstart = 0, f_wcount = 0;
    int64_t f_row0 = 0;
    if (l < nq) {
      const int m = mb + l * G;
      const int s = q_seq[m];
      const int64_t lim = ((int64_t)q_pos[m] + 1) / ratio;
      f_vis = (int)max<int64_t>(0, min<int64_t>(seq_len[s], lim));
      f_row0 = seq_start[s];
      f_wcount = (W > 0) ? min(swa_count[m], W) : 0;
      f_wstart = (W > 0) ? swa_start[m] : 0;
    }
    auto vis_of = [&](int k) { return __builtin_amdgcn_readlane(f_vis, k); };
    auto row0_of = [&](int k) {
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)f_row0, k);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)f_row0 >> 32), k);
      return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    auto wcount_of = [&](int k) { return __builtin_amdgcn_readlane(f_wcount, k); };
    auto wstart_of = [&](int k) { return __builtin_amdgcn_readlane(f_wstart, k); };
    auto next = [&](Cursor &u) {
      if (++u.c == NC) { u.c = 0; ++u.k; }
    };
    // index of this lane's slot (main groups only), 0 past the batch
    auto index_of = [&](const Cursor &u) -> int32_t {
      const int sl = kPC * u.c + 16 * wv + row;
      const bool ok = u.k < nq && kPC * u.c + 16 * wv < K;
      const rsrc_t r = make_rsrc(topk + (int64_t)(mb + (ok ? u.k : 0) * G) * K, (uint32_t)(K * 4));
      return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r, ok ? (uint32_t)sl * 4u : kOutOfRange, 0, 0);
    };
    // Loads that bring the lines of a chunk's keys into the caches (their
    // values are discarded): lanes of quads 0 and 2 touch the two code lines
    // of a main entry and quad 1 its scale line; for window rows each quad
    // touches one of the row's four lines.  Every lane issues both loads, at
    // offsets past the descriptors where it has nothing to touch.
    auto touch_keys = [&](const Cursor &u, int32_t j) -> uint32_t {
      const bool live = u.k < nq;
      const int kq = live ? u.k : 0;
      const int sl0 = kPC * u.c + 16 * wv;
      const bool main = sl0 < K;
      const int64_t vis = vis_of(kq), row0 = row0_of(kq);
      const int wc = wcount_of(kq), wi = sl0 + row - K;
      const rsrc_t r_codes = make_rsrc(kv_codes + row0 * (kPD / 2), (uint32_t)(vis * (kPD / 2)));
      const rsrc_t r_scales = make_rsrc(kv_scales + row0 * (kPD / 16), (uint32_t)(vis * (kPD / 16)));
      const rsrc_t r_win = make_rsrc(wc ? swa_codes + (int64_t)wstart_of(kq) * kPD : nullptr, (uint32_t)(wc * kPD));
      const bool okm = live && main && j >= 0 && j < vis;
      const bool okw = live && !main && wi < wc;
      const uint32_t co = (okm && (quad & 1) == 0) ? (uint32_t)j * (kPD / 2) + quad * 64u
                          : okw ? (uint32_t)wi * kPD + quad * 128u : kOutOfRange;
      const uint32_t so = (okm && quad == 1) ? (uint32_t)j * (kPD / 16) : kOutOfRange;
      const uint32_t a = __builtin_amdgcn_raw_buffer_load_b32(main ? r_codes : r_win, co, 0, 0);
      const uint32_t b = __builtin_amdgcn_raw_buffer_load_b32(r_scales, so, 0, 0);
      return a ^ b;
    };
    // Every lane issues the same loads whatever its slot holds (offsets past
    // a descriptor read zeros), so no branch joins wait on them.
    auto load_keys = [&](const Cursor &u, int32_t j, KeyBytes &kb) {
      const bool live = u.k < nq;
      const int kq = live ? u.k : 0;
      const int sl0 = kPC * u.c + 16 * wv;
      const bool main = sl0 < K;
      const int64_t vis = vis_of(kq), row0 = row0_of(kq);
      const int wc = wcount_of(kq), wi = sl0 + row - K;
      const int64_t ws = wstart_of(kq);
      const rsrc_t r_codes = make_rsrc(kv_codes + row0 * (kPD / 2), (uint32_t)(vis * (kPD / 2)));
      const rsrc_t r_scales = make_rsrc(kv_scales + row0 * (kPD / 16), (uint32_t)(vis * (kPD / 16)));
      const rsrc_t r_win = make_rsrc(wc ? swa_codes + ws * kPD : nullptr, (uint32_t)(wc * kPD));
      const rsrc_t r_wsc = make_rsrc(wc ? swa_scale + ws : nullptr, (uint32_t)(wc * 4));
      const rsrc_t rc = main ? r_codes : r_win;
      const bool okm = live && main && j >= 0 && j < vis;
      const bool okw = live && !main && wi < wc;
      const uint32_t co = okm ? (uint32_t)j * (kPD / 2) + quad * 64u : okw ? (uint32_t)wi * kPD + quad * 128u : kOutOfRange;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rc, co + 16u * i, 0, 0);
        kb.w[4 * i] = x[0]; kb.w[4 * i + 1] = x[1]; kb.w[4 * i + 2] = x[2]; kb.w[4 * i + 3] = x[3];
      }
      const u32x2_t y = __builtin_amdgcn_raw_buffer_load_b64(r_scales, okm ? (uint32_t)j * (kPD / 16) + quad * 8u : kOutOfRange, 0, 0);
      kb.s[0] = y[0];
      kb.s[1] = y[1];
      kb.r = __builtin_amdgcn_raw_buffer_load_b32(r_wsc, okw ? (uint32_t)wi * 4u : kOutOfRange, 0, 0);
      kb.o2 = okw ? co + 64u : kOutOfRange;
      kb.ks_main = main ? (okm ? 1.0f : 0.0f) : -1.0f;
    };
    // Query k's heads h0 .. h0+hq-1 (bf16, hq KB; empty past the batch) and
    // their staging into L.qn: part p of thread t is the 8 channels
    // 8 * (i % 64) .. +7 of head i / 64, i = 256 p + t.
    auto q_rsrc = [&](int k) {
      const bool ok = k < nq;
      return make_rsrc(q + ((int64_t)(mb + (ok ? k : 0) * G) * H + h0) * kPD, ok ? (uint32_t)(hq * kPD * 2) : 0u);
    };
    auto q_part_load = [&](rsrc_t r, int p, bool want) -> u32x4_t {
      return __builtin_amdgcn_raw_buffer_load_b128(r, want ? (uint32_t)(256 * p + threadIdx.x) * 16u : kOutOfRange, 0, 0);
    };
    // (head 4p + t/64, channels 8 (t % 64) ..: one base per thread plus 4p rows)
    const int qn_base = (int)(threadIdx.x >> 6) * kPTs + 8 * (int)(threadIdx.x & 63);
    auto q_part_store = [&](int p, const u32x4_t &x) {
      half8_t h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[2 * e] = (_Float16)__uint_as_float(x[e] << 16);
        h[2 * e + 1] = (_Float16)__uint_as_float(x[e] & 0xFFFF0000u);
      }
      *reinterpret_cast<half8_t *>(&L.qn[qn_base + p * (4 * kPTs)]) = h;
    };

    // ---- stream set-up: indices of items 0..3, lines of items 1, 2, bytes of item 0 ----
    const int items = nq * NC;
    Cursor cur{0, 0}, c1{0, 0}, c3{0, 0}, c4{0, 0};
    next(c1);
    next(c3); next(c3); next(c3);
    c4 = c3;
    next(c4);
    int32_t j1, j2, j3;
    KeyBytes kb;
    {
      Cursor u{0, 0};
      const int32_t j0 = index_of(u);
      next(u); j1 = index_of(u);
      next(u); j2 = index_of(u);
      next(u); j3 = index_of(u);
      load_keys(Cursor{0, 0}, j0, kb);
    }
    uint32_t t1, t2;
    int pf_done = 0;   // parts of the next query's heads already staged in L.qn
    {
      Cursor u{0, 0};
      next(u); t1 = touch_keys(u, j1);
      next(u); t2 = touch_keys(u, j2);
    }

    half8_t qb[4][16];
    float4_t o[8][4];  // O^T: dims 128w + 16rt + 4quad + j, head 16ct + row
    float m_run[4], l_part[4];
    int e_cur = 0;     // accumulator exponent: true O = o * 2^-e_cur

    for (int it = 0; it < items; ++it) {
      const int buf = it & 1;
      const int m = mb + cur.k * G;
      if (cur.c == 0) {
        // ---- a new query: parts of its heads that the previous query's items
        //      did not stage (all of them for the batch's first query) are
        //      staged now; then each wave takes its B operands from L.qn:
        //      lane (head 16ct + row, quad) holds channels quad*128 + 8kk .. +7
        //      in qb[ct][kk] ----
        if (pf_done < kQParts) {
          const rsrc_t r_q = q_rsrc(cur.k);
          u32x4_t raw[kQParts];
#pragma unroll
          for (int p = 0; p < kQParts; ++p) raw[p] = q_part_load(r_q, p, p >= pf_done);
#pragma unroll
          for (int p = 0; p < kQParts; ++p)
            if (p >= pf_done) q_part_store(p, raw[p]);
          __syncthreads();
        }
        pf_done = 0;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int kk = 0; kk < 16; ++kk) {
            qb[ct][kk] = *reinterpret_cast<const half8_t *>(&L.qn[(16 * ct + row) * kPTs + quad * 128 + 8 * kk]);
            asm("" : "+a"(qb[ct][kk]));
          }
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) o[rt][ct] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) { m_run[ct] = kNegInf; l_part[ct] = 0.0f; }
        e_cur = 0;
      }
      // ---- window items: the second 64 bytes of each row, issued before the
      //      look-ahead loads so that waiting for them does not also wait for
      //      those (loads complete in issue order); main items read out of range ----
      uint32_t w2[16];
      {
        const int wc = wcount_of(cur.k);
        const rsrc_t r_win = make_rsrc(wc ? swa_codes + (int64_t)wstart_of(cur.k) * kPD : nullptr, (uint32_t)(wc * kPD));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r_win, kb.o2 + 16u * i, 0, 0);
          w2[4 * i] = x[0]; w2[4 * i + 1] = x[1]; w2[4 * i + 2] = x[2]; w2[4 * i + 3] = x[3];
        }
      }
      // ---- look-ahead: index of item it+4, lines of item it+3 ----
      const int32_t j4 = index_of(c4);
      const uint32_t t3 = touch_keys(c3, j3);
      asm volatile("" ::"v"(t1));
      // ---- two parts of the next query's heads, staged after the chunk maxima meet (the
      //      query's last item stages none) ----
      const bool pf = cur.c < NC - 1 && pf_done < kQParts;
      u32x4_t pfr[2];
      {
        const rsrc_t r_q = q_rsrc(cur.k + 1);
#pragma unroll
        for (int i = 0; i < 2; ++i) pfr[i] = q_part_load(r_q, pf_done + i, pf && pf_done + i < kQParts);
      }

      // ---- this wave's 16 keys: scales to LDS, S^T = K Q^T, decoded keys to the tile ----
      _Float16 *tile = L.t;
      const float kbs = key_scale(kb);
      if (quad == 0) L.ks[buf][16 * wv + row] = kbs;
      const float kbm = max16_lanes(kbs);
      if (l == 0) L.rmax[buf][wv] = kbm;
      __builtin_amdgcn_wave_barrier();
      const float4 kq = *reinterpret_cast<const float4 *>(&L.ks[buf][16 * wv + 4 * quad]);
      float4_t sacc[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) sacc[ct] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
      _Float16 *trow = tile + (16 * wv + row) * kPTs + quad * 128;
      if (kPC * cur.c + 16 * wv < K) {
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const half8_t a = main_slice(kb, kk);
          *reinterpret_cast<half8_t *>(trow + 8 * kk) = a;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) sacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[ct][kk], sacc[ct], 0, 0, 0);
        }
      } else {
        // window rows: E4M3 codes, the first 64 bytes from kb, the rest from w2
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const half8_t a = kk < 8 ? e4m3x8_to_f16(kb.w[2 * kk], kb.w[2 * kk + 1])
                                   : e4m3x8_to_f16(w2[2 * kk - 16], w2[2 * kk - 15]);
          *reinterpret_cast<half8_t *>(trow + 8 * kk) = a;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) sacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[ct][kk], sacc[ct], 0, 0, 0);
        }
      }
      // ---- next item's key bytes; rotate the look-ahead ----
      load_keys(c1, j1, kb);
      j1 = j2; j2 = j3; j3 = j4;
      t1 = t2; t2 = t3;
      // ---- logits (log2 units; empty slots -inf) and this wave's chunk maxima ----
      const float ksj[4] = {kq.x, kq.y, kq.z, kq.w};
      float z[4][4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          z[ct][j] = fmaf(sacc[ct][j], tau2 * ksj[j], ksj[j] != 0.0f ? 0.0f : kNegInf);
          mx = fmaxf(mx, z[ct][j]);
        }
        mx = max_rows4(mx);
        if (quad == 0) L.cmax[buf][16 * ct + row][wv] = mx;
      }
      __syncthreads();
      // ---- the staged parts of the next query's heads (every wave has read
      //      the current query's from L.qn before the barrier above) ----
      if (pf) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (pf_done + i < kQParts) q_part_store(pf_done + i, pfr[i]);
        pf_done = min(kQParts, pf_done + 2);
      }
      // ---- softmax statistics, lazily raised running maximum ----
      const float4 rv = *reinterpret_cast<const float4 *>(&L.rmax[buf][0]);
      float4 cvs[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) cvs[ct] = *reinterpret_cast<const float4 *>(&L.cmax[buf][16 * ct + row][0]);
      const float rmax = fmaxf(fmaxf(rv.x, rv.y), fmaxf(rv.z, rv.w));
      int e_c = e_cur;
      if (rmax > 0.0f) {
        (void)frexpf(rmax, &e_c);
        e_c = 1 - e_c;  // rmax * 2^e_c in [1, 2)
      }
      float oscale[4], msub[4];
      bool rescale = false;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const float4 cv = cvs[ct];
        const float cm = fmaxf(fmaxf(cv.x, cv.y), fmaxf(cv.z, cv.w));
        float mn = m_run[ct];
        if (m_run[ct] == kNegInf || cm > m_run[ct] + kLazyMax) mn = cm;
        const float alpha = (m_run[ct] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(m_run[ct] - mn);
        l_part[ct] *= alpha;
        m_run[ct] = mn;
        msub[ct] = (mn == kNegInf) ? 0.0f : mn;  // with no key seen yet every z is -inf: p = 0
        oscale[ct] = ldexpf(alpha, e_c - e_cur);
        rescale |= oscale[ct] != 1.0f;
      }
      if (cur.c > 0 && __any(rescale)) {
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) o[rt][ct][j] *= oscale[ct];
      }
      e_cur = e_c;
      // P enters P V as p * r * 2^e; main entries have r in {0, 1}, and with
      // e = 0 that is p itself
      const bool plain = e_c == 0 && kPC * (cur.c + 1) <= K;
      float ksc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ksc[j] = ldexpf(ksj[j], e_c);
      _Float16 *pt = L.p[buf];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(z[ct][j] - msub[ct]);
        l_part[ct] += (p[0] + p[1]) + (p[2] + p[3]);
        if (!plain) {
#pragma unroll
          for (int j = 0; j < 4; ++j) p[j] *= ksc[j];
        }
        const half4_t pv = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
        *reinterpret_cast<half4_t *>(pt + (16 * ct + row) * kPPs + 16 * wv + 4 * quad) = pv;
      }
      __syncthreads();
      // ---- O^T += V^T P^T: this wave's 128 output channels, all 64 heads;
      //      the LDS operands of the next row tile are read ahead ----
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        half8_t pb[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          pb[ct] = *reinterpret_cast<const half8_t *>(pt + (16 * ct + row) * kPPs + 32 * k2 + 8 * quad);
        half8_t va[2];
        va[0] = v_operand_tr(tile, kPTs, 32 * k2, 128 * wv, row, quad);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
          if (rt + 1 < 8) va[(rt + 1) & 1] = v_operand_tr(tile, kPTs, 32 * k2, 128 * wv + 16 * (rt + 1), row, quad);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            o[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[rt & 1], pb[ct], o[rt][ct], 0, 0, 0);
        }
      }

      // the tile is free for the next chunk and the staged heads are complete
      __syncthreads();
      if (cur.c == NC - 1) {
        // ---- the query's last chunk: denominators across key quarters and waves, outputs ----
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const float lw = sum_rows4(l_part[ct]);
          if (quad == 0) L.lsum[16 * ct + row][wv] = lw;
        }
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int h = h0 + 16 * ct + row;
          if (h >= H) continue;
          const float4 lv = *reinterpret_cast<const float4 *>(&L.lsum[16 * ct + row][0]);
          const float lt = (lv.x + lv.y) + (lv.z + lv.w);
          const float inv = (lt > 0.0f) ? ldexpf(1.0f / lt, -e_cur) : 0.0f;
          float *dst = out + ((int64_t)m * H + h) * kPD + 128 * wv + 4 * quad;
#pragma unroll
          for (int rt = 0; rt < 8; ++rt)
            *reinterpret_cast<float4 *>(dst + 16 * rt) =
                make_float4(o[rt][ct][0] * inv, o[rt][ct][1] * inv, o[rt][ct][2] * inv, o[rt][ct][3] * inv);
          if (wv == 0 && quad == 0 && lse)
            lse[(int64_t)m * H + h] = (lt > 0.0f) ? (m_run[ct] + log2f(lt)) * 0.6931471805599453f : kNegInf;
        }
      }
      next(cur); next(c1); next(c3); next(c4);
    }
    asm volatile("" ::"v"(t1), "v"(t2));
    __syncthreads();  // LDS of this batch is free
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool attn_prefill_supported(const csa2_fp4_cache &kv, int q_dtype, int top_k) {
  return kv.dim == kPD && q_dtype == CSA2_BF16 && top_k % 16 == 0 &&
         (int64_t)kv.max_len * (kPD / 2) < kMaxRsrcBytes;
}

int launch_attn_prefill(const csa2_fp4_cache &kv, const csa2_queries &qs, const void *q, int heads,
                        const int32_t *topk, int top_k, const csa2_swa &swa, float scale, float *out, float *lse,
                        hipStream_t stream) {
  if (qs.m == 0) return CSA2_OK;
  const float tau2 = scale * 1.4426950408889634f;  // log2-domain softmax: p = 2^(z - max)
  // one workgroup per CU (each uses most of a CU's LDS and registers), looping over queries
  const int hb = (heads + kPH - 1) / kPH;
  const int g = std::max(1, std::min(qs.m, 256 / hb));
  const dim3 grid(g, hb);
  CSA2_TIMED_LAUNCH(kTimedAttn, k_attn_prefill, grid, dim3(256), stream, static_cast<const uint16_t *>(q), qs.m,
                    heads, kv.codes, kv.scales, kv.seq_start, kv.seq_len, kv.ratio, qs.seq, qs.pos, topk, top_k,
                    swa.codes, swa.scale, swa.start, swa.count, swa.window, tau2, out, lse);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

}  // namespace csa2
