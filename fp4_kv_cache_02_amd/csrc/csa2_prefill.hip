// CSA2 flat Top-K indexer for encoder prefill chunks (P4 section 二: encoder
// groups select without a candidate pool; P1 section "Compressed Sparse
// Attention 2 (CSA2)" for the score and for which compressed entries a token
// may see).
//
// Scoring.  The queries of a prefill chunk share their sequence's indexer
// cache, so scoring is a dense contraction [queries x heads] x [channels] x
// [entries] and runs on MFMA.  A workgroup takes 16 queries of up to 8 heads
// (128 rows = 8 row tiles; 8 queries for up to 16 heads) and keeps them as A
// operands in the registers of each of its 4 waves (one per SIMD, so the
// queries can sit in the accumulation registers); wave w streams the
// 16-entry column tiles w, w + 4, ... of the cache.  Each column tile is
// decoded once (FP4 -> exact f16) and meets every row tile: 32 MFMAs per
// tile for 128 channels.  The epilogue takes the weighted ReLU over each
// query's heads, masks entries the query may not see, reduces 8-entry blocks
// to their maximum and writes it to bmax.  The entries that all workgroups
// stream stay in L2, so the loads are plain (not streamed past the caches).
//
// Selection.  The flat Top-K lies inside the top K blocks by (block max desc,
// block id asc): every block ranked above a block that holds a Top-K
// position holds its own maximum position, ranked above that Top-K position,
// and there are fewer than K of those.  So the block select keeps P = K
// blocks per query, their 8K positions are re-scored and the Top-K is taken
// from them, with the same stages as the decoder's Full layer.
#include "csa2_internal.hpp"
#include "csa2_indexer.hpp"

#include <type_traits>

namespace csa2 {

constexpr int kMqWaves = 4;  // waves per scoring workgroup: one per SIMD, so each has the full register file
constexpr int kMqValuPerMfma = 4;  // vector instructions scheduled between consecutive MFMAs
constexpr int kMqRing = 8;   // LDS slots per wave for column tiles loaded ahead

// One column tile as it lands in LDS, in lane order: lane (entry n, quarter
// g) = 16g + n owns its DI/8 code bytes and the word holding its scale bytes,
// so every lane reads its own words back without bank conflicts.
template <int DI>
struct MqTile {
  static constexpr int NW = DI / 32;                 // code words per lane
  static constexpr int V = (NW % 4 == 0) ? 4 : 1;    // words per load into LDS
  static constexpr int NL = NW / V + 1;              // loads into LDS per tile
  uint32_t w[NW / V][kWave][V];
  uint32_t s[kWave];
};

// Buffer descriptor words (as scalar operands of the loads below): base,
// no stride, `bytes` valid bytes (offsets past them read zeros).
CSA2_DEV u32x4_t rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return (u32x4_t){(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}
// Loads into LDS: lane i of the wave puts its 16 (4) bytes at LDS byte
// address lds + 16i (4i).  Written out so that the compiler, which cannot
// tell the ring's slots apart, does not drain every load into LDS before
// each LDS read; the ring's own waits (wait_vm) order them instead.  They
// return nothing to registers.
CSA2_DEV void lds_load16(const u32x4_t &rs, uint32_t lds, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}
CSA2_DEV void lds_load4(const u32x4_t &rs, uint32_t lds, uint32_t voff) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}
CSA2_DEV uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p; }

// s_waitcnt with only the vector memory count bounded (n < 64)
template <int N>
CSA2_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// RT_: row tiles held by every wave (0: the default, 8, or 4 for 256 channels);
// fewer when the queries come in short runs of one sequence, so that a
// workgroup's queries belong to one run (no pass scores rows of other
// sequences' queries)
template <int DI, int RPQ, int RT_ = 0>
struct MqShape {
  static constexpr int RT = RT_ ? RT_ : (DI == 256) ? 4 : 8;
  static constexpr int QB = RT * 16 / RPQ;        // queries per workgroup
  static constexpr int NG = QB / 4;               // groups of four queries
  static constexpr int TPG = RPQ / 4;             // row tiles per group
  static constexpr int KT = DI / 32;              // MFMAs per (row tile, column tile)
  static_assert(NG >= 1 && (TPG == 2 || TPG == 4), "multi-query tiling");
};

// Block maxima of one column tile for NG groups of four queries at once.
// v[p] holds, in lane (row g, column n), the score of entry n for query
// 4p + row_tile(g); each half-row (8 lanes) is one block.  The groups are
// spread over the lanes while they are reduced: the first exchange (lane i
// with 7 - i) halves the groups each lane keeps, the second (i with i ^ 1)
// halves them again, the third (i with i ^ 2) only takes the maximum.  Lane i
// (= n % 8) ends with the block maximum of group lane_group<NG>(i); two lanes
// hold each group and lane_stores<NG>(i) picks one.
template <int NG>
CSA2_DEV float block_max_groups(const float (&v)[NG], int i) {
  if constexpr (NG == 4) {
    const bool q1 = i >= 4, odd = (i & 1) != 0;
    const float sa = q1 ? v[0] : v[2], sb = q1 ? v[1] : v[3];
    const float ka = q1 ? v[2] : v[0], kb = q1 ? v[3] : v[1];
    const float wa = max_f(ka, dpp_f<kDppHalfMirror>(sa));
    const float wb = max_f(kb, dpp_f<kDppHalfMirror>(sb));
    const float x = max_f(odd ? wb : wa, dpp_f<kDppXor1>(odd ? wa : wb));
    return max_f(x, dpp_f<kDppXor2>(x));
  } else if constexpr (NG == 2) {
    const bool q1 = i >= 4;
    float x = max_f(q1 ? v[1] : v[0], dpp_f<kDppHalfMirror>(q1 ? v[0] : v[1]));
    x = max_f(x, dpp_f<kDppXor1>(x));
    return max_f(x, dpp_f<kDppXor2>(x));
  } else {
    return max8_scores(v[0]);
  }
}
template <int NG>
CSA2_DEV int lane_group(int i) { return NG == 4 ? 2 * (i >> 2) + (i & 1) : NG == 2 ? (i >> 2) : 0; }
template <int NG>
CSA2_DEV bool lane_stores(int i) { return NG == 4 ? (i & 2) == 0 : NG == 2 ? (i & 3) == 0 : i == 0; }

// Grid: (ceil(M / QB), column chunks) workgroups of 64 * kMqWaves threads.
// Rows of the workgroup's A block: row = RPQ * qi + h (query m0 + qi, head
// h).  The queries of one workgroup may belong to several sequences: each
// sequence is one pass over its entries with the other queries left out.
// Workgroup y of a query block takes the column tiles [y*ct, (y+1)*ct) of
// every pass (ct = 0: all of them), so a few query blocks - the tokens of a
// multi-token decode - still spread over the chip.
template <int DI, int RPQ, int RT>
__global__ __launch_bounds__(64 * kMqWaves) void k_score_mq(const uint8_t *__restrict__ codes,
                                                           const uint8_t *__restrict__ scales,
                                                           const int64_t *__restrict__ seq_start,
                                                           const int32_t *__restrict__ seq_len, int ratio,
                                                           const int32_t *__restrict__ q_seq,
                                                           const int32_t *__restrict__ q_pos, int M,
                                                           const uint16_t *__restrict__ q_idx,
                                                           const float *__restrict__ w_idx, int H,
                                                           float *__restrict__ bmax, int64_t nb_stride, int ct) {
  using S = MqShape<DI, RPQ, RT>;
  constexpr int kNone = 0x7FFFFFFF;
  __shared__ int s_seq[S::QB], s_vis[S::QB];
  __shared__ MqTile<DI> ring[kMqWaves][kMqRing];
  const int m0 = blockIdx.x * S::QB;
  if (threadIdx.x < S::QB) {
    const int m = m0 + threadIdx.x;
    int s = kNone, v = 0;
    if (m < M) {
      int ss;
      v = (int)visible_entries(seq_len, q_seq, q_pos, ratio, m, &ss);
      s = ss;
    }
    s_seq[threadIdx.x] = s;
    s_vis[threadIdx.x] = v;
  }
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  half8_t A[S::RT][S::KT];
  float W[S::RT][4];
#pragma unroll
  for (int r = 0; r < S::RT; ++r) {
    const int row = r * 16 + n;
    const int qi = row / RPQ, h = row % RPQ;
    const bool valid = (m0 + qi < M) && (h < H);
    const int64_t mh = valid ? (int64_t)(m0 + qi) * H + h : 0;
    load_query_rows<DI>(q_idx + mh * DI, valid, valid ? w_idx[mh] : 0.0f, A[r], W[r]);
  }
  // the query operands are only read by MFMA: keep them in the accumulation
  // registers, which leaves the vector registers to the accumulators and the
  // epilogue (the vector ALUs cannot read accumulation registers)
#pragma unroll
  for (int r = 0; r < S::RT; ++r)
#pragma unroll
    for (int t = 0; t < S::KT; ++t) asm volatile("" : "+a"(A[r][t]));
  __syncthreads();

  // finished queries of the workgroup (bit q), uniform across the workgroup
  uint32_t done = 0;
#pragma unroll
  for (int q = 0; q < S::QB; ++q)
    if (s_seq[q] == kNone || s_vis[q] == 0) done |= 1u << q;
  done = __builtin_amdgcn_readfirstlane(done);
  constexpr uint32_t kAll = (S::QB == 32) ? 0xFFFFFFFFu : ((1u << S::QB) - 1u);

  const int i8 = n & 7;
  const int q_store = 4 * lane_group<S::NG>(i8) + row_tile(g);  // query whose block maximum this lane stores
  // the workgroup's rows of bmax; stores of lanes with nothing to store go past its end
  const rsrc_t rb = make_rsrc(bmax + (int64_t)m0 * nb_stride, (uint32_t)(min(S::QB, M - m0) * nb_stride * 4));

  while (done != kAll) {
    // next sequence: the smallest one among the unfinished queries
    int sc = kNone;
#pragma unroll
    for (int q = 0; q < S::QB; ++q)
      if (!((done >> q) & 1u)) sc = min(sc, s_seq[q]);
    sc = __builtin_amdgcn_readfirstlane(sc);
    uint32_t act = 0;
    int maxvis = 0, minvis = kNone;
#pragma unroll
    for (int q = 0; q < S::QB; ++q) {
      if (!((done >> q) & 1u) && s_seq[q] == sc) {
        act |= 1u << q;
        maxvis = max(maxvis, s_vis[q]);
        minvis = min(minvis, s_vis[q]);
      }
    }
    act = __builtin_amdgcn_readfirstlane(act);
    maxvis = __builtin_amdgcn_readfirstlane(maxvis);
    minvis = __builtin_amdgcn_readfirstlane(minvis);
    done |= act;
    // visible entries of this lane's query in each group (tail tiles only)
    int vis_l[S::NG];
#pragma unroll
    for (int p = 0; p < S::NG; ++p) vis_l[p] = s_vis[4 * p + row_tile(g)];
    const uint32_t soff = (lane_stores<S::NG>(i8) && ((act >> q_store) & 1u))
                              ? (uint32_t)((q_store * nb_stride + (n >> 3)) * 4) : kOutOfRange;
    // this workgroup's column tiles of the pass: [cb, ce)
    const int cb = ct ? (int)blockIdx.y * ct : 0;
    const int ntile = ct ? min((maxvis + 15) / 16, cb + ct) : (maxvis + 15) / 16;
    const int full = min(ntile, minvis / 16);  // tiles every query of the pass sees whole
    const int64_t row0 = seq_start[sc];
    const uint8_t *cbase = codes + row0 * (DI / 2);
    const uint8_t *sbase = scales + row0 * (DI / 16);

    // rows past the pass's visible range are clamped to its last entry (in bounds, never stored)
    auto load = [&](int c, LaneCodes<DI> &buf) {
      const int e = min(c * 16 + n, maxvis - 1);
      load_lane_codes_rel<DI, false>(cbase, sbase, (uint32_t)e, (uint32_t)g, buf);
    };
    // all row tiles against one column tile: RT independent accumulation chains
    auto mfmas = [&](const half8_t (&B)[S::KT], float4_t (&acc)[S::RT]) {
#pragma unroll
      for (int t = 0; t < S::KT; ++t)
#pragma unroll
        for (int r = 0; r < S::RT; ++r) {
          const float4_t c0 = {0.0f, 0.0f, 0.0f, 0.0f};
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[r][t], B[t], t == 0 ? c0 : acc[r], 0, 0, 0);
        }
    };
    // weighted ReLU and head sums per query, block maxima, one store per lane
    auto epilogue = [&](const float4_t (&acc)[S::RT], int c, auto mask_tag) {
      float v[S::NG];
#pragma unroll
      for (int p = 0; p < S::NG; ++p) {
        float part[S::TPG];
#pragma unroll
        for (int u = 0; u < S::TPG; ++u) part[u] = weighted_relu4(W[p * S::TPG + u], acc[p * S::TPG + u]);
        if constexpr (S::TPG == 2) v[p] = tile_scores_x2(part[0], part[1]);
        else v[p] = tile_scores_x4(part[0], part[1], part[2], part[3]);
        if constexpr (decltype(mask_tag)::value)
          if (c * 16 + n >= vis_l[p]) v[p] = -INFINITY;
      }
      const float x = block_max_groups<S::NG>(v, i8);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rb, soff + 8u * (uint32_t)c, 0, 0);
    };

    // Tiles every query of the pass sees whole, software-pipelined: step i
    // loads tile i + kMqRing - 1 straight into this wave's LDS ring (entries
    // past the pass's visible range lie past the descriptors and arrive as
    // zeros), issues the MFMAs of tile i, the epilogue of tile i - 1 and the
    // decode of tile i + 1, read from the ring, so the matrix cores and the
    // vector ALUs work on independent data and no registers hold tiles in
    // flight.
    const int T = (full > cb + wv) ? (full - cb - wv + kMqWaves - 1) / kMqWaves : 0;  // this wave's whole tiles
    if (T > 0) {
      using Tl = MqTile<DI>;
      const u32x4_t rc = rsrc_words(cbase, (uint32_t)maxvis * (DI / 2));
      const u32x4_t rs = rsrc_words(sbase, (uint32_t)maxvis * (DI / 16));
      const uint32_t sshift = 8u * ((uint32_t)(g * (DI / 64)) & 3u);
      auto tile_of = [&](int i) { return cb + wv + kMqWaves * i; };
      auto issue = [&](int i) {
        Tl &t = ring[wv][i % kMqRing];
        const uint32_t e = (uint32_t)(tile_of(i) * 16 + n);
#pragma unroll
        for (int r = 0; r < Tl::NW / Tl::V; ++r) {
          const uint32_t off = e * (DI / 2) + (uint32_t)g * (DI / 8) + 4u * Tl::V * r;
          if constexpr (Tl::V == 4) lds_load16(rc, lds_addr(&t.w[r][0][0]), off);
          else lds_load4(rc, lds_addr(&t.w[r][0][0]), off);
        }
        lds_load4(rs, lds_addr(&t.s[0]), e * (DI / 16) + (((uint32_t)g * (DI / 64)) & ~3u));
      };
      auto read = [&](int i, LaneCodes<DI> &c) {
        const Tl &t = ring[wv][i % kMqRing];
#pragma unroll
        for (int r = 0; r < Tl::NW / Tl::V; ++r) {
          if constexpr (Tl::V == 4) {
            const u32x4_t x = *reinterpret_cast<const u32x4_t *>(&t.w[r][l][0]);
            c.w[4 * r] = x[0]; c.w[4 * r + 1] = x[1]; c.w[4 * r + 2] = x[2]; c.w[4 * r + 3] = x[3];
          } else {
            c.w[r] = t.w[r][l][0];
          }
        }
        c.s = t.s[l] >> sshift;
      };
      half8_t B[2][S::KT];
      float4_t acc[2][S::RT];
      LaneCodes<DI> cn[2];  // codes of tiles i + 1 and i + 2, read from the ring two steps ahead
#pragma unroll
      for (int i = 0; i < kMqRing - 1; ++i) issue(i);
      wait_vm<0>();
      {
        LaneCodes<DI> c0;
        read(0, c0);
        decode_keys<DI>(c0, B[0]);
      }
      read(1, cn[1]);
      read(2, cn[0]);
      // the ring slot of tile i + 3 has landed once at most (kMqRing - 5)
      // tiles' loads and as many epilogue stores are younger than its loads
      constexpr int kVm = (kMqRing - 5) * (MqTile<DI>::NL + 1);
      // step i: the MFMAs of tile i, the epilogue of tile i - 1 and the
      // decode of tile i + 1 as one interleaved stretch; then tile i + 3 from
      // the ring and the load of tile i + kMqRing - 1 into the slot tile i - 1
      // left
      auto step = [&](auto kc, auto epi, int i) {
        constexpr int K = decltype(kc)::value;  // i % 2
        mfmas(B[K], acc[K]);
        if constexpr (decltype(epi)::value) epilogue(acc[K ^ 1], tile_of(i - 1), std::false_type{});
        decode_keys<DI>(cn[K ^ 1], B[K ^ 1]);
        // interleave: each MFMA followed by a few independent vector instructions
#pragma unroll
        for (int k = 0; k < S::RT * S::KT; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, K);
          __builtin_amdgcn_sched_group_barrier(0x002, kMqValuPerMfma, K);
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<kVm>();
        read(i + 3, cn[K ^ 1]);
        issue(i + kMqRing - 1);
        __builtin_amdgcn_sched_barrier(0);
      };
      using K0 = std::integral_constant<int, 0>;
      using K1 = std::integral_constant<int, 1>;
      step(K0{}, std::false_type{}, 0);
      // pairs of steps with one exit test, so that both steps of a pair are
      // one block (the compiler moves no work from one step into the next)
      int i = 1;
      for (; i + 1 < T; i += 2) {
        step(K1{}, std::true_type{}, i);
        step(K0{}, std::true_type{}, i + 1);
      }
      if (i < T) {
        step(K1{}, std::true_type{}, i);
        epilogue(acc[1], tile_of(i), std::false_type{});
      } else {
        epilogue(acc[0], tile_of(i - 1), std::false_type{});
      }
      wait_vm<0>();  // the ring is idle before the next pass or the end
    }
    // the last tiles, which some query sees only in part: masked, one at a time
    for (int c = cb + wv + kMqWaves * T; c < ntile; c += kMqWaves) {
      LaneCodes<DI> cur;
      half8_t B[S::KT];
      float4_t acc[S::RT];
      load(c, cur);
      decode_keys<DI>(cur, B);
      mfmas(B, acc);
      epilogue(acc, c, std::true_type{});
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Workspace of the flat indexer, all offsets 256-byte aligned.
struct FlatWs {
  size_t bmax, pool, pool_count, pscore, total;
  int64_t nb_stride;  // block slots per query (covers every column tile's pair of blocks)
};

static FlatWs flat_ws_layout(int64_t max_len, int m, int top_k) {
  FlatWs w{};
  const int64_t pairs = (max_len + 15) / 16;
  w.nb_stride = ((2 * pairs + 63) / 64) * 64;
  if (w.nb_stride == 0) w.nb_stride = 64;
  size_t off = 0;
  w.bmax = off;       off = align256(off + sizeof(float) * (size_t)m * (size_t)w.nb_stride);
  w.pool = off;       off = align256(off + sizeof(int32_t) * (size_t)m * (size_t)top_k);
  w.pool_count = off; off = align256(off + sizeof(int32_t) * (size_t)m);
  w.pscore = off;     off = align256(off + sizeof(float) * (size_t)m * 8 * (size_t)top_k);
  w.total = off;
  return w;
}

size_t flat_ws_bytes(int64_t max_len, int m, int top_k) { return flat_ws_layout(max_len, m, top_k).total; }

// Column chunks: enough workgroups to fill the chip when the query blocks
// alone do not (a multi-token decode), chunks of at least 64 tiles; with
// fewer row tiles a workgroup needs fewer registers and more of them fit a
// CU (up to 4 per CU at 2 row tiles).
template <int DI, int RPQ, int RT>
static void launch_score_mq(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                            const float *w_idx, int heads, float *bmax, int64_t nb_stride, hipStream_t stream) {
  using S = MqShape<DI, RPQ, RT>;
  const int qb = (qs.m + S::QB - 1) / S::QB;
  const int64_t tiles = (idx.max_len + 15) / 16;
  const int64_t target = 256 * (8 / S::RT);   // 256 workgroups, 512 at 4 row tiles, 1,024 at 2
  int chunks = 1;
  while ((int64_t)qb * chunks < target && tiles / (2 * chunks) >= 64) chunks *= 2;
  const int ct = chunks > 1 ? (int)((tiles + chunks - 1) / chunks) : 0;
  const dim3 grid((unsigned)qb, (unsigned)chunks);
  CSA2_TIMED_LAUNCH(kTimedScan, (k_score_mq<DI, RPQ, RT>), grid, dim3(64 * kMqWaves), stream, idx.codes,
                    idx.scales, idx.seq_start, idx.seq_len, idx.ratio, qs.seq, qs.pos, qs.m, q_idx, w_idx, heads,
                    bmax, nb_stride, ct);
}

// Row tiles per wave from the run hint: a workgroup holds QB = 16 RT / RPQ
// queries, so runs of up to 4 (8) tokens of 8 heads take 2 (4) row tiles and
// one run per workgroup; 16 heads take 4 row tiles for runs of up to 4.
template <int DI, int RPQ>
static void launch_score_run(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                             const float *w_idx, int heads, float *bmax, int64_t nb_stride, hipStream_t stream) {
  constexpr int RTD = MqShape<DI, RPQ>::RT;
  const int run = qs.run;
  if constexpr (RPQ == 8) {
    if (run >= 2 && run <= 4) {
      launch_score_mq<DI, RPQ, 2>(idx, qs, q_idx, w_idx, heads, bmax, nb_stride, stream);
      return;
    }
  }
  if constexpr (RTD > 4) {
    if (run >= 2 && run <= 4 * 16 / RPQ) {
      launch_score_mq<DI, RPQ, 4>(idx, qs, q_idx, w_idx, heads, bmax, nb_stride, stream);
      return;
    }
  }
  launch_score_mq<DI, RPQ, RTD>(idx, qs, q_idx, w_idx, heads, bmax, nb_stride, stream);
}

int launch_score_blocks(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                        const float *w_idx, int heads, float *bmax, int64_t nb_stride, hipStream_t stream) {
  if (idx.max_len == 0 || qs.m == 0) return CSA2_OK;
  const bool wide = heads > 8;
  switch (idx.dim) {
    case 64:
      if (wide) launch_score_run<64, 16>(idx, qs, q_idx, w_idx, heads, bmax, nb_stride, stream);
      else launch_score_run<64, 8>(idx, qs, q_idx, w_idx, heads, bmax, nb_stride, stream);
      break;
    case 128:
      if (wide) launch_score_run<128, 16>(idx, qs, q_idx, w_idx, heads, bmax, nb_stride, stream);
      else launch_score_run<128, 8>(idx, qs, q_idx, w_idx, heads, bmax, nb_stride, stream);
      break;
    case 256:
      if (wide) launch_score_run<256, 16>(idx, qs, q_idx, w_idx, heads, bmax, nb_stride, stream);
      else launch_score_run<256, 8>(idx, qs, q_idx, w_idx, heads, bmax, nb_stride, stream);
      break;
    default:
      return CSA2_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

int launch_index_flat(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                      const float *w_idx, int heads, int top_k, int32_t *topk_out, float *topk_score, void *ws,
                      hipStream_t stream) {
  if (qs.m == 0) return CSA2_OK;
  if (heads < 1 || heads > 16) return CSA2_ERR_UNSUPPORTED;
  const int64_t nb_max = (idx.max_len + kBlock - 1) / kBlock;
  if (nb_max > kBlockSelectMax) return CSA2_ERR_UNSUPPORTED;
  if (idx.dim != 64 && idx.dim != 128 && idx.dim != 256) return CSA2_ERR_UNSUPPORTED;
  const FlatWs L = flat_ws_layout(idx.max_len, qs.m, top_k);
  char *base = static_cast<char *>(ws);
  float *bmax = reinterpret_cast<float *>(base + L.bmax);
  int32_t *pool = reinterpret_cast<int32_t *>(base + L.pool);
  int32_t *pool_count = reinterpret_cast<int32_t *>(base + L.pool_count);
  float *pscore = reinterpret_cast<float *>(base + L.pscore);
  int st = launch_score_blocks(idx, qs, q_idx, w_idx, heads, bmax, L.nb_stride, stream);
  if (st != CSA2_OK) return st;
  st = launch_block_select(bmax, L.nb_stride, nb_max > 0 ? nb_max : 1, idx, qs, top_k, pool, pool_count,
                               stream);
  if (st != CSA2_OK) return st;
  const SelSet set{q_idx, w_idx, topk_out, topk_score};
  return launch_rescore_select(idx, qs, heads, pool, pool_count, top_k, top_k, &set, 1, pscore, stream);
}

}  // namespace csa2
