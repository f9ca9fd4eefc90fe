// CSA2 Hierarchical Sparse Indexer for decode (P1 section "Compressed Sparse
// Attention 2 (CSA2)"; P2 section 03; P4 section 二 and its mode table; P5
// figure caption "Hierarchical Sparse Indexer").
//
// Full layer:  scan every visible indexer entry -> block maxima over 8
//              positions (+ a 4096-bin histogram of their keys)
//              -> pool of the top P blocks (threshold bin, exact resolution
//              of the boundary bin) -> re-score the pool positions -> Top-K.
// Reindex:     re-score the given pool with the layer's own query -> Top-K.
//
// Score s_j = sum_h w_h * max(0, q_h . k_j).  The dot products run on MFMA
// (v_mfma_f32_16x16x32_f16): rows = indexer heads, columns = 16 positions,
// k = channels.  FP4 keys decode exactly to f16 (e2m1 * e4m3 has <= 6
// significant bits); each head's bf16 query is scaled by a power of two so
// its largest element lies in [2^14, 2^15) and converts exactly to f16, and
// the inverse power of two is folded into w_h.  Products are therefore exact
// and only the fp32 accumulation rounds.
#include "csa2_internal.hpp"
#include "csa2_indexer.hpp"

namespace csa2 {

constexpr int kScanWaves = 8;                    // waves per scan workgroup
constexpr int kScanTiles = 1024;                 // 16-position tiles per scan workgroup (largest chunk)
constexpr int kScanChunk = kScanTiles * 16;      // 16384 positions
constexpr int kScanBlocks = kScanChunk / kBlock; // 2048 block maxima
constexpr int kFilterBlocks = 2048;              // blocks per pool-filter workgroup (one list reservation each)
constexpr int kRescoreEntries = 64;              // pool blocks per re-score workgroup (at most)


// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

// Zero n words from p, 16 bytes per thread (p 16-byte aligned, n % 4 == 0).
__global__ void k_zero_u32(uint32_t *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * i < n) reinterpret_cast<uint4 *>(p)[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Radix digit search shared by the selection kernels: s_hist[256] holds the
// counts of one 8-bit digit; find the digit v (scanning from 255 down) whose
// bin holds the rem-th largest element.  Run by wave 0; writes the digit, the
// rank left inside its bin, and the bin count.
CSA2_DEV void find_digit(const uint32_t *s_hist, int rem, int *s_digit, int *s_rem, int *s_cnt) {
  if (threadIdx.x >= 64) return;
  const int l = threadIdx.x;
  int h[4];
  int local = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = (int)s_hist[255 - 4 * l - e];
    local += h[e];
  }
  const int incl = wave_incl_scan(local);
  int excl = incl - local;
  if (excl < rem && incl >= rem) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (excl + h[e] >= rem) {
        *s_digit = 255 - 4 * l - e;
        *s_rem = rem - excl;
        *s_cnt = h[e];
        break;
      }
      excl += h[e];
    }
  }
}

// First scan: grid (chunks, queries), WAVES waves, TILES * 16 positions per
// workgroup, scored in batches of U consecutive tiles: all loads of a batch
// are issued before any of it is scored, and the other waves of the CU cover
// the latency.  Wave w starts with batch w and then claims the next unclaimed
// batch from an LDS counter, so the waves of a workgroup finish together
// even when the memory system serves them unevenly (a fixed round-robin left
// them several microseconds apart).  Large chunks amortise the per-workgroup
// set-up (query load, histogram clear and flush); the host picks the chunk so
// that the grid still fills the chip.  Four tiles at a time share the
// cross-lane reduction (tile_scores_x4).  Block maxima are staged in LDS,
// written out once, and counted into an LDS histogram whose non-zero bins are
// added to one of the query's hist_rep global histogram replicas (chunk %
// hist_rep): every workgroup of a query hits the same few bins, and device
// atomics on one address serialise.
constexpr int kScanU = 8;
constexpr int kScanMinGrid = 240;  // workgroups that count as filling the 256 CUs
constexpr int kHistMaxReplicas = 8;

template <int DI, int WAVES = kScanWaves, int TILES = kScanTiles, int U = kScanU>
__global__ __launch_bounds__(64 * WAVES) void k_scan(const uint8_t *__restrict__ codes,
                                                     const uint8_t *__restrict__ scales,
                                                     const int64_t *__restrict__ seq_start,
                                                     const int32_t *__restrict__ seq_len, int ratio,
                                                     const int32_t *__restrict__ q_seq,
                                                     const int32_t *__restrict__ q_pos,
                                                     const uint16_t *__restrict__ q_idx,
                                                     const float *__restrict__ w_idx, int H,
                                                     float *__restrict__ bmax, int64_t nb_stride,
                                                     uint32_t *__restrict__ hist, int hist_rep) {
  constexpr int CHUNK = TILES * 16;
  constexpr int BLOCKS = CHUNK / kBlock;
  static_assert(TILES % (WAVES * U) == 0 && U % 4 == 0, "scan tiling");
  __shared__ float s_bmax[BLOCKS];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHistBins];
  __shared__ int s_next;  // next unclaimed batch
  const int m = blockIdx.y;
  int s;
  const int64_t vis = visible_entries(seq_len, q_seq, q_pos, ratio, m, &s);
  const int64_t p_begin = (int64_t)blockIdx.x * CHUNK;
  if (p_begin >= vis) return;
  for (int i = threadIdx.x; i < kHistBins / 4; i += blockDim.x)
    reinterpret_cast<uint4 *>(s_hist)[i] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) s_next = WAVES;

  IdxQuery<DI> Q;
  load_idx_query<DI>(q_idx + (int64_t)m * H * DI, w_idx + (int64_t)m * H, H, Q);

  const int l = lane_id(), n = l & 15, qq = l >> 4, wv = threadIdx.x >> 6;
  // positions of this chunk, relative to p_begin; the tail is clamped to the last visible entry
  const int n_here = (int)min<int64_t>(CHUNK, vis - p_begin);
  const uint8_t *cbase = codes + (seq_start[s] + p_begin) * (DI / 2);
  const uint8_t *sbase = scales + (seq_start[s] + p_begin) * (DI / 16);
  const int rt = row_tile(l >> 4);
  // batch b: tiles b*U .. b*U + U-1 (positions past the chunk's end are
  // clamped to its last entry and score -inf into slots nobody reads)
  const int n_batches = (n_here + U * 16 - 1) / (U * 16);
  auto load_batch = [&](int b, LaneCodes<DI> *c) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = min((b * U + u) * 16 + n, n_here - 1);
      load_lane_codes_rel<DI>(cbase, sbase, (uint32_t)p, (uint32_t)qq, c[u]);
    }
  };
  auto score_batch = [&](int b, const LaneCodes<DI> *c) {
#pragma unroll
    for (int g = 0; g < U / 4; ++g) {
      float v = tile_scores_x4(tile_partial<DI>(Q, c[4 * g]), tile_partial<DI>(Q, c[4 * g + 1]),
                               tile_partial<DI>(Q, c[4 * g + 2]), tile_partial<DI>(Q, c[4 * g + 3]));
      const int tile = b * U + 4 * g + rt;
      if (tile * 16 + n >= n_here) v = -INFINITY;
      v = max8_scores(v);
      if ((n & 7) == 0) s_bmax[tile * 2 + (n >> 3)] = v;
    }
  };
  auto claim = [&]() {
    int v = 0;
    if (l == 0) v = atomicAdd(&s_next, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  __syncthreads();  // s_next is set
  // the scheduling barriers keep each batch's loads issued together, ahead of
  // the scoring; the next claim is in flight while the batch is scored
  int b = __builtin_amdgcn_readfirstlane(wv);
  while (b < n_batches) {
    LaneCodes<DI> c[U];
    load_batch(b, c);
    const int next = claim();
    __builtin_amdgcn_sched_barrier(0);
    score_batch(b, c);
    b = next;
  }
  __syncthreads();
  const int nb_here = (n_here + kBlock - 1) / kBlock;
  float *dst = bmax + (int64_t)m * nb_stride + (int64_t)blockIdx.x * BLOCKS;
  for (int i = threadIdx.x; i < nb_here; i += blockDim.x) {
    const float v = s_bmax[i];
    dst[i] = v;
    atomicAdd(&s_hist[f2key(v) >> (32 - kHistBits)], 1u);
  }
  __syncthreads();
  // flush: the first block of each bin to arrive moves the bin's count out
  uint32_t *gh = hist + ((int64_t)m * hist_rep + blockIdx.x % hist_rep) * kHistBins;
  for (int i = threadIdx.x; i < nb_here; i += blockDim.x) {
    const uint32_t bin = f2key(s_bmax[i]) >> (32 - kHistBits);
    const uint32_t cnt = atomicExch(&s_hist[bin], 0u);
    if (cnt) atomicAdd(&gh[bin], cnt);
  }
}

// First scan for runs of R tokens of one sequence (R = 2 or 4 queries of at
// most 8 indexer heads; the run hint): one pass over the sequence's entries
// scores every streamed entry against the whole run.  Row tile g of the MFMA
// holds query 2g in rows 0-7 and query 2g+1 in rows 8-15 (missing heads are
// zero rows), so each decoded key tile feeds R/2 row tiles, and the bytes
// streamed are those of one query.  tile_scores_x2 adds each query's two
// quarters; the one-query scan adds the same two plus two quarters of zero
// rows, so the scores, block maxima and pools are the same bit for bit.
// Block maxima and histograms are kept per query exactly as k_scan keeps
// them.  A run whose queries belong to more than one sequence (a hint not
// kept) takes one pass per sequence, each leaving the run's other queries
// out.  grid (chunks, runs).
template <int DI, int R, int WAVES = kScanWaves, int TILES = kScanTiles, int U = kScanU>
__global__ __launch_bounds__(64 * WAVES) void k_scan_run(const uint8_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales,
                                                         const int64_t *__restrict__ seq_start,
                                                         const int32_t *__restrict__ seq_len, int ratio,
                                                         const int32_t *__restrict__ q_seq,
                                                         const int32_t *__restrict__ q_pos,
                                                         const uint16_t *__restrict__ q_idx,
                                                         const float *__restrict__ w_idx, int H,
                                                         float *__restrict__ bmax, int64_t nb_stride,
                                                         uint32_t *__restrict__ hist, int hist_rep) {
  constexpr int CHUNK = TILES * 16;
  constexpr int BLOCKS = CHUNK / kBlock;
  constexpr int RT = R / 2;
  static_assert(R == 2 || R == 4, "run length");
  static_assert(TILES % (WAVES * U) == 0 && U % 2 == 0, "scan tiling");
  __shared__ float s_bmax[R][BLOCKS];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[R][kHistBins];
  __shared__ int s_next;  // next unclaimed batch
  const int m0 = blockIdx.y * R;
  const int64_t p_begin = (int64_t)blockIdx.x * CHUNK;
  // the run's queries: sequence and entries visible in this chunk (uniform)
  int sq[R], vrel[R];
  bool any = false;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int s;
    const int64_t v = visible_entries(seq_len, q_seq, q_pos, ratio, m0 + r, &s);
    sq[r] = __builtin_amdgcn_readfirstlane(s);
    vrel[r] = __builtin_amdgcn_readfirstlane((int)max<int64_t>(0, min<int64_t>(CHUNK, v - p_begin)));
    any |= vrel[r] > 0;
  }
  if (!any) return;
  for (int i = threadIdx.x; i < R * kHistBins / 4; i += blockDim.x)
    reinterpret_cast<uint4 *>(&s_hist[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);

  const int l = lane_id(), n = l & 15, qq = l >> 4, row = l >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t done = 0;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if ((done >> k) & 1u) continue;
    // this pass: the sequence of query k and every query of the run in it
    const int S = sq[k];
    uint32_t inc = 0;
    int n_here = 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (!((done >> r) & 1u) && sq[r] == S) {
        inc |= 1u << r;
        n_here = max(n_here, vrel[r]);
      }
    done |= inc;
    if (n_here == 0) continue;
    IdxQuery<DI> Q[RT];
#pragma unroll
    for (int g = 0; g < RT; ++g) {
      const int qr = 2 * g + (n >> 3), h = n & 7;
      const bool valid = ((inc >> qr) & 1u) && h < H;
      const int64_t qm = m0 + qr;
      load_query_rows<DI>(q_idx + (qm * H + (valid ? h : 0)) * DI, valid, valid ? w_idx[qm * H + h] : 0.0f, Q[g].a,
                          Q[g].w);
    }
    const int64_t row0 = seq_start[S] + p_begin;
    const uint8_t *cbase = codes + row0 * (DI / 2);
    const uint8_t *sbase = scales + row0 * (DI / 16);
    if (threadIdx.x == 0) s_next = WAVES;
    __syncthreads();  // s_next is set; the previous pass's flush is done
    // batch b: tiles b*U .. b*U + U-1 (positions past n_here are clamped to
    // its last entry and score -inf)
    const int n_batches = (n_here + U * 16 - 1) / (U * 16);
    auto load_batch = [&](int b, LaneCodes<DI> *c) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = min((b * U + u) * 16 + n, n_here - 1);
        load_lane_codes_rel<DI>(cbase, sbase, (uint32_t)p, (uint32_t)qq, c[u]);
      }
    };
    // a lane's share of row tile g's scores for decoded keys kb (each key
    // tile is decoded once for all the row tiles)
    auto partial = [&](int g, const half8_t *kb) {
      float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < DI / 32; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Q[g].a[t], kb[t], acc, 0, 0, 0);
      return weighted_relu4(Q[g].w, acc);
    };
    auto score_batch = [&](int b, const LaneCodes<DI> *c) {
#pragma unroll
      for (int pr = 0; pr < U / 2; ++pr) {
        half8_t ka[DI / 32], kb[DI / 32];
        decode_keys<DI>(c[2 * pr], ka);
        decode_keys<DI>(c[2 * pr + 1], kb);
#pragma unroll
        for (int g = 0; g < RT; ++g) {
          // lane row r: tile 2 pr + (r & 1) of the batch, query 2 g + (r >> 1)
          float v = tile_scores_x2(partial(g, ka), partial(g, kb));
          const int tile = b * U + 2 * pr + (row & 1);
          const int qr = 2 * g + (row >> 1);
          const int vq = (row >> 1) ? vrel[2 * g + 1] : vrel[2 * g];
          if (tile * 16 + n >= vq) v = -INFINITY;
          v = max8_scores(v);
          if ((n & 7) == 0 && ((inc >> qr) & 1u)) s_bmax[qr][tile * 2 + (n >> 3)] = v;
        }
      }
    };
    auto claim = [&]() {
      int v = 0;
      if (l == 0) v = atomicAdd(&s_next, 1);
      return __builtin_amdgcn_readfirstlane(v);
    };
    int b = wv;
    while (b < n_batches) {
      LaneCodes<DI> c[U];
      load_batch(b, c);
      const int next = claim();
      __builtin_amdgcn_sched_barrier(0);
      score_batch(b, c);
      b = next;
    }
    __syncthreads();
    // this pass's queries: block maxima out, counted into their histograms
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!((inc >> r) & 1u)) continue;
      const int nb_r = (vrel[r] + kBlock - 1) / kBlock;
      float *dst = bmax + (int64_t)(m0 + r) * nb_stride + (int64_t)blockIdx.x * BLOCKS;
      for (int i = threadIdx.x; i < nb_r; i += blockDim.x) {
        const float v = s_bmax[r][i];
        dst[i] = v;
        atomicAdd(&s_hist[r][f2key(v) >> (32 - kHistBits)], 1u);
      }
    }
    __syncthreads();
    // flush: the first block of each bin to arrive moves the bin's count out
    // (which leaves the LDS histograms cleared for the next pass)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!((inc >> r) & 1u)) continue;
      const int nb_r = (vrel[r] + kBlock - 1) / kBlock;
      uint32_t *gh = hist + ((int64_t)(m0 + r) * hist_rep + blockIdx.x % hist_rep) * kHistBins;
      for (int i = threadIdx.x; i < nb_r; i += blockDim.x) {
        const uint32_t bin = f2key(s_bmax[r][i]) >> (32 - kHistBits);
        const uint32_t cnt = atomicExch(&s_hist[r][bin], 0u);
        if (cnt) atomicAdd(&gh[bin], cnt);
      }
    }
    __syncthreads();
  }
}

// Wave-aggregated append of the `pred` lanes to list[*counter ...].
CSA2_DEV void wave_append(bool pred, int32_t value, int *counter, int32_t *list) {
  const uint64_t mask = __ballot(pred);
  if (!mask) return;
  const int l = lane_id();
  const int leader = __ffsll((unsigned long long)mask) - 1;
  int base = 0;
  if (l == leader) base = atomicAdd(counter, (int)__popcll(mask));
  base = __shfl(base, leader, 64);
  if (pred) list[base + __popcll(mask & ((1ull << l) - 1ull))] = value;
}


// Histogram of block-maximum keys (top kHistBits bits) when the block
// maxima come from the multi-query scoring kernel: grid (chunks of
// kFilterBlocks blocks, queries), one LDS histogram per workgroup whose
// non-zero bins are added to replica (chunk % hist_rep) of the query's
// histogram - the same histogram the decode scan builds as it goes.
__global__ __launch_bounds__(256) void k_bmax_hist(const float *__restrict__ bmax, int64_t nb_stride,
                                                   const int32_t *__restrict__ seq_len,
                                                   const int32_t *__restrict__ q_seq,
                                                   const int32_t *__restrict__ q_pos, int ratio,
                                                   uint32_t *__restrict__ hist, int hist_rep) {
  __shared__ uint32_t s_hist[kHistBins];
  const int m = blockIdx.y;
  int s;
  const int64_t vis = visible_entries(seq_len, q_seq, q_pos, ratio, m, &s);
  const int64_t nb = (vis + kBlock - 1) / kBlock;
  const int64_t b0 = (int64_t)blockIdx.x * kFilterBlocks;
  if (b0 >= nb) return;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) s_hist[i] = 0u;
  __syncthreads();
  const float *bm = bmax + (int64_t)m * nb_stride;
  for (int j = 0; j < kFilterBlocks / 256; ++j) {
    const int64_t b = b0 + j * 256 + threadIdx.x;
    if (b < nb) atomicAdd(&s_hist[f2key(bm[b]) >> (32 - kHistBits)], 1u);
  }
  __syncthreads();
  uint32_t *hq = hist + ((int64_t)m * hist_rep + (int)(blockIdx.x % hist_rep)) * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
    if (s_hist[i]) atomicAdd(&hq[i], s_hist[i]);
}

// Pool filter.  Every workgroup first finds the query's threshold bin T -
// the bin of the need-th largest block maximum, need = min(P, visible
// blocks), -1 when every block is taken - from the scan's histogram
// replicas (workgroup 0 records it in counters[4m + 2] for the
// finalisation).  Blocks above T are in the pool for sure, blocks in it go
// to the tie list and are counted by their next 12 key bits into the
// query's fine histogram (fine[m][4096], zeroed with the coarse one).
// Appends are gathered in LDS and reserved in the global lists with one
// atomic per list per workgroup; a workgroup's block maxima are all loaded
// before any is looked at.
__global__ __launch_bounds__(256) void k_pool_filter(const float *__restrict__ bmax, int64_t nb_stride,
                                                     const uint32_t *__restrict__ hist, int hist_rep,
                                                     const int32_t *__restrict__ seq_len, const int32_t *__restrict__ q_seq,
                                                     const int32_t *__restrict__ q_pos, int ratio, int P,
                                                     uint32_t *__restrict__ counters, uint32_t *__restrict__ fine,
                                                     int32_t *__restrict__ sure, int32_t *__restrict__ tie) {
  constexpr int PT = kFilterBlocks / 256;
  __shared__ int s_ns, s_nt, s_bs, s_bt, s_T;
  __shared__ int s_scan[5];
  __shared__ int32_t s_sure[kFilterBlocks], s_tie[kFilterBlocks];
  __shared__ uint32_t s_fine[kHistBins];
  const int m = blockIdx.y;
  const int64_t b0 = (int64_t)blockIdx.x * kFilterBlocks;
  // the workgroup's block maxima and every replica's histogram bins are
  // loaded before the query's visible count is known (both are in range of
  // the workspace whatever it is; entries past the visible blocks are
  // ignored below), so their latency overlaps the sequence lookup.  Thread t
  // owns bins [4096-16(t+1), 4096-16t) (thread 0 = highest bins); replicas
  // past hist_rep read replica 0 and count nothing
  const rsrc_t r_bm = make_rsrc(bmax + (int64_t)m * nb_stride + b0,
                                (uint32_t)(max<int64_t>(0, min<int64_t>(nb_stride - b0, kFilterBlocks)) * 4));
  float v[PT];
#pragma unroll
  for (int j = 0; j < PT; ++j)
    v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_bm, (uint32_t)(j * 256 + threadIdx.x) * 4u, 0, 0));
  const int hi = kHistBins - 16 * threadIdx.x;
  uint4 x[kHistMaxReplicas][4];
#pragma unroll
  for (int r = 0; r < kHistMaxReplicas; ++r) {
    const int rr = r < hist_rep ? r : 0;
    const uint4 *h4 = reinterpret_cast<const uint4 *>(hist + ((int64_t)m * hist_rep + rr) * kHistBins + hi - 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) x[r][k] = h4[k];
  }
  int s;
  const int64_t vis = visible_entries(seq_len, q_seq, q_pos, ratio, m, &s);
  const int64_t nb = (vis + kBlock - 1) / kBlock;
  if (b0 >= nb) return;
  for (int i = threadIdx.x; i < kHistBins; i += 256) s_fine[i] = 0u;
  if (threadIdx.x == 0) { s_ns = 0; s_nt = 0; s_T = -1; }
  if (nb > P) {
    int hv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) hv[k] = 0;
#pragma unroll
    for (int r = 0; r < kHistMaxReplicas; ++r) {
      if (r >= hist_rep) continue;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hv[4 * k] += (int)x[r][k].x; hv[4 * k + 1] += (int)x[r][k].y;
        hv[4 * k + 2] += (int)x[r][k].z; hv[4 * k + 3] += (int)x[r][k].w;
      }
    }
    int c = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) c += hv[k];
    int tot;
    const int before = block_exclusive_scan<256>(c, s_scan, &tot);
    if (before < P && before + c >= P) {
      int cum = before;
      for (int k = 15; k >= 0; --k) {
        cum += hv[k];
        if (cum >= P) { s_T = hi - 16 + k; break; }
      }
    }
  }
  __syncthreads();
  const int T = s_T;
  if (blockIdx.x == 0 && threadIdx.x == 0) counters[m * 4 + 2] = (uint32_t)T;
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const int64_t b = b0 + j * 256 + threadIdx.x;
    const bool ok = b < nb;
    const uint32_t key = f2key(v[j]);
    const int bin = ok ? (int)(key >> (32 - kHistBits)) : -2;
    wave_append(ok && bin > T, (int32_t)b, &s_ns, s_sure);
    wave_append(ok && bin == T, (int32_t)b, &s_nt, s_tie);
    if (ok && bin == T) atomicAdd(&s_fine[(key >> 8) & (kHistBins - 1)], 1u);
  }
  __syncthreads();
  if (s_nt > 0) {
    uint32_t *fq = fine + (int64_t)m * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256)
      if (s_fine[i]) atomicAdd(&fq[i], s_fine[i]);
  }
  if (threadIdx.x == 0) {
    s_bs = s_ns ? (int)atomicAdd(&counters[m * 4 + 0], (uint32_t)s_ns) : 0;
    s_bt = s_nt ? (int)atomicAdd(&counters[m * 4 + 1], (uint32_t)s_nt) : 0;
  }
  __syncthreads();
  // the lists hold P sure blocks and nb_stride tie blocks per query; a
  // histogram that disagreed with the block maxima could ask for more, and
  // those appends are dropped rather than written past the lists
  int32_t *su = sure + (int64_t)m * P + s_bs;
  int32_t *ti = tie + (int64_t)m * nb_stride + s_bt;
  const int ns = max(0, min(s_ns, P - s_bs));
  const int nt = (int)max<int64_t>(0, min<int64_t>(s_nt, nb_stride - s_bt));
  for (int i = threadIdx.x; i < ns; i += blockDim.x) su[i] = s_sure[i];
  for (int i = threadIdx.x; i < nt; i += blockDim.x) ti[i] = s_tie[i];
}

// Pool finalisation, one workgroup per query: resolve the boundary bin
// exactly on (key desc, block asc), then emit the pool in ascending block
// order by compacting a bitmap of the chosen blocks.
constexpr int kMaxPool = 4096;
constexpr int kBitmapWords = 16384;  // blocks up to 2^19 go through the bitmap
constexpr int kFineCand = 2048;      // fine-threshold-bin ties resolved in LDS

CSA2_DEV void wave_refine(const uint64_t *cand, int n, int rem, uint32_t *h, int *s_digit, int *s_rem,
                          int *s_cnt, uint64_t &prefix, uint64_t &mask);
CSA2_DEV uint32_t wave_incl_max(uint32_t v);

struct FinLds {
  uint32_t bits[kBitmapWords];
  int32_t pool[kMaxPool];
  uint64_t cand[kFineCand];
  uint32_t h[256];
  int scan[17];
  int digit, rem, cnt, n, nc, Tf, af, nf;
  uint64_t cut;
};

// The finalisation of query m by a workgroup of 1024 threads; s_T is the
// threshold bin (-1 when every visible block is taken).
// cnt4: the query's counters (sure count, tie count, threshold bin); fine4:
// this thread's four fine-histogram bins; su_pre: sure-list entries
// threadIdx.x + 1024 u (all loaded before the visible count was known).
CSA2_DEV void pool_finalize_body(FinLds &F, const float *__restrict__ bmax, int64_t nb_stride, const uint4 &cnt4,
                                 const uint4 &fine4, const int32_t (&su_pre)[4],
                                 const int32_t *__restrict__ tie, int m, int64_t nb, uint32_t s_T, int P,
                                 int32_t *__restrict__ pool_out, int32_t *__restrict__ pool_count) {
  // counts as far as the lists reach (they never exceed them when the
  // histogram agrees with the block maxima)
  const int n_sure = (int)min<uint32_t>(cnt4.x, (uint32_t)P);
  const int n_tie = (int)min<int64_t>((int64_t)cnt4.y, nb_stride);
  const int need = (int)min<int64_t>(min<int64_t>(P, nb), (int64_t)n_sure + n_tie);
  const int need_t = need - n_sure;
  const int32_t *ti = tie + (int64_t)m * nb_stride;
  const float *bm = bmax + (int64_t)m * nb_stride;
  const bool use_bits = nb <= 32 * (int64_t)kBitmapWords;
  const int words = (int)((nb + 31) / 32);
  if (use_bits)
    for (int i = threadIdx.x; i < words; i += blockDim.x) F.bits[i] = 0u;
  if (threadIdx.x == 0) F.n = 0;
  __syncthreads();
  auto take = [&](int32_t b) {
    if (use_bits) atomicOr(&F.bits[b >> 5], 1u << (b & 31));
    else {
      const int slot = atomicAdd(&F.n, 1);
      if (slot < kMaxPool) F.pool[slot] = b;
    }
  };
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if ((int)threadIdx.x + 1024 * u < n_sure && (uint64_t)su_pre[u] < (uint64_t)nb) take(su_pre[u]);
  // the fine threshold bin of the ties (thread 0 = highest fine bins)
  if (threadIdx.x == 0) { F.Tf = 0; F.af = 0; F.nf = 0; F.nc = 0; }
  bool fine_ok = false;
  if (need_t > 0 && need_t < n_tie) {
    const int hi = kHistBins - 4 * (int)threadIdx.x;
    const int hv[4] = {(int)fine4.x, (int)fine4.y, (int)fine4.z, (int)fine4.w};
    const int c = hv[0] + hv[1] + hv[2] + hv[3];
    int tot;
    const int before = block_exclusive_scan<1024>(c, F.scan, &tot);
    if (before < need_t && before + c >= need_t) {
      int cum = before;
      for (int k = 3; k >= 0; --k) {
        if (cum + hv[k] >= need_t) { F.Tf = hi - 4 + k; F.af = cum; F.nf = hv[k]; break; }
        cum += hv[k];
      }
    }
    __syncthreads();
    // the fine histogram counts every tie (it agrees with the tie list unless
    // the lists overflowed); its threshold bin must fit the LDS candidates
    fine_ok = tot == n_tie && F.nf <= kFineCand;
  }
  if (need_t > 0 && need_t < n_tie && fine_ok) {
    const uint32_t Tf = (uint32_t)F.Tf;
    const int rem_f = need_t - F.af, nf = F.nf;
    const bool whole = rem_f == nf;
    // ties above Tf (and all of Tf when it is taken whole) in one gather
    // pass; Tf's composites to LDS.  Batches of 8 ties per thread: the ids,
    // then their block maxima, all in flight before any is used (loads past
    // the list or the visible blocks read 0 and are skipped)
    const rsrc_t r_ti = make_rsrc(ti, (uint32_t)(n_tie * 4));
    const rsrc_t r_bm = make_rsrc(bm, (uint32_t)(nb * 4));
    for (int i0 = 0; i0 < n_tie; i0 += 8 * (int)blockDim.x) {
      int32_t ids[8];
      float bv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        ids[u] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_ti, (uint32_t)(i0 + u * blockDim.x + threadIdx.x) * 4u,
                                                                 0, 0);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        bv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            r_bm, ((uint64_t)ids[u] < (uint64_t)nb) ? (uint32_t)ids[u] * 4u : kOutOfRange, 0, 0));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * blockDim.x + threadIdx.x;
        const int32_t b = ids[u];
        if (i >= n_tie || (uint64_t)b >= (uint64_t)nb) continue;
        const uint32_t key = f2key(bv[u]);
        const uint32_t f = (key >> 8) & (kHistBins - 1);
        if (f > Tf || (f == Tf && whole)) take(b);
        else if (f == Tf) {
          const int slot = atomicAdd(&F.nc, 1);
          if (slot < kFineCand) F.cand[slot] = ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)b);
        }
      }
    }
    __syncthreads();
    if (!whole) {
      const int n2 = min(F.nc, kFineCand);
      const int lane = threadIdx.x & 63;
      if (n2 <= 64) {
        if (threadIdx.x < 64) {
          const uint64_t c = (lane < n2) ? F.cand[lane] : 0ull;
          const uint32_t clo = (uint32_t)c, chi = (uint32_t)(c >> 32);
          int r = 0;
          for (int j = 0; j < n2; ++j) {
            const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)chi, j) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane((int)clo, j);
            r += o > c;
          }
          if (lane < n2 && r < rem_f) take((int32_t)(~(uint32_t)c));
        }
      } else {
        if (threadIdx.x < 64) {
          uint64_t pf = 0ull, mk = 0ull;
          wave_refine(F.cand, n2, rem_f, F.h, &F.digit, &F.rem, &F.cnt, pf, mk);
          if (threadIdx.x == 0) F.cut = pf;
        }
        __syncthreads();
        const uint64_t cut = F.cut;
        for (int i = threadIdx.x; i < n2; i += blockDim.x)
          if (F.cand[i] >= cut) take((int32_t)(~(uint32_t)F.cand[i]));
      }
    }
  } else if (need_t > 0) {
    if (need_t >= n_tie) {
      for (int i = threadIdx.x; i < n_tie; i += blockDim.x)
        if ((uint64_t)ti[i] < (uint64_t)nb) take(ti[i]);
    } else {
      // composite key: larger score first, then smaller block id.  Every tie
      // entry shares the threshold bin (the top kHistBits of the score key),
      // so the digits start below it; the passes stop as soon as the cut's bin
      // holds exactly the entries still needed.
      constexpr int kKnown = kHistBits;
      uint64_t prefix = (uint64_t)s_T << (64 - kKnown);
      uint64_t mask = ((1ull << kKnown) - 1ull) << (64 - kKnown);
      int rem = need_t;
      for (int hi = 64 - kKnown; hi > 0; hi -= 8) {
        const int width = hi < 8 ? hi : 8;
        const int shift = hi - width;
        const uint64_t dmask = (1ull << width) - 1ull;
        for (int i = threadIdx.x; i < 256; i += blockDim.x) F.h[i] = 0u;
        __syncthreads();
        for (int i = threadIdx.x; i < n_tie; i += blockDim.x) {
          const int32_t b = ti[i];
          if ((uint64_t)b >= (uint64_t)nb) continue;
          const uint64_t c = ((uint64_t)f2key(bm[b]) << 32) | (uint64_t)(~(uint32_t)b);
          if ((c & mask) == prefix) atomicAdd(&F.h[(c >> shift) & dmask], 1u);
        }
        __syncthreads();
        find_digit(F.h, rem, &F.digit, &F.rem, &F.cnt);
        __syncthreads();
        prefix |= (uint64_t)F.digit << shift;
        mask |= dmask << shift;
        rem = F.rem;
        if (F.cnt == rem) break;
      }
      for (int i = threadIdx.x; i < n_tie; i += blockDim.x) {
        const int32_t b = ti[i];
        if ((uint64_t)b >= (uint64_t)nb) continue;
        const uint64_t c = ((uint64_t)f2key(bm[b]) << 32) | (uint64_t)(~(uint32_t)b);
        if ((c & mask) >= prefix) take(b);
      }
    }
  }
  __syncthreads();
  int32_t *out = pool_out + (int64_t)m * P;
  if (use_bits) {
    // thread t compacts words [t*wpt, (t+1)*wpt)
    const int wpt = (words + 1023) / 1024;
    int cnt = 0;
    for (int k = 0; k < wpt; ++k) {
      const int w = threadIdx.x * wpt + k;
      if (w < words) cnt += __popc(F.bits[w]);
    }
    int tot;
    int pos = block_exclusive_scan<1024>(cnt, F.scan, &tot);
    for (int k = 0; k < wpt; ++k) {
      const int w = threadIdx.x * wpt + k;
      if (w >= words) break;
      uint32_t bits = F.bits[w];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        if (pos < P) out[pos] = w * 32 + bit;
        ++pos;
      }
    }
    for (int i = min(tot, need) + threadIdx.x; i < need; i += blockDim.x) out[i] = -1;
  } else {
    int n2 = 64;
    while (n2 < need) n2 <<= 1;
    // slots past what was taken sort last (rescoring treats them as not visible)
    for (int i = min(F.n, need) + threadIdx.x; i < n2; i += blockDim.x) F.pool[i] = 0x7FFFFFFF;
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = threadIdx.x; i < n2; i += blockDim.x) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const int32_t a = F.pool[i], b = F.pool[ixj];
            const bool up = (i & k) == 0;
            if ((a > b) == up) { F.pool[i] = b; F.pool[ixj] = a; }
          }
        }
        __syncthreads();
      }
    }
    for (int i = threadIdx.x; i < need; i += blockDim.x) out[i] = F.pool[i];
  }
  for (int i = need + threadIdx.x; i < P; i += blockDim.x) out[i] = -1;
  if (threadIdx.x == 0) pool_count[m] = need;
}

__global__ __launch_bounds__(1024) void k_pool_finalize(const float *__restrict__ bmax, int64_t nb_stride,
                                                        const uint32_t *__restrict__ counters,
                                                        const uint32_t *__restrict__ fine,
                                                        const int32_t *__restrict__ sure,
                                                        const int32_t *__restrict__ tie,
                                                        const int32_t *__restrict__ seq_len,
                                                        const int32_t *__restrict__ q_seq,
                                                        const int32_t *__restrict__ q_pos, int ratio, int P,
                                                        int32_t *__restrict__ pool_out,
                                                        int32_t *__restrict__ pool_count) {
  __shared__ FinLds F;
  static_assert(kMaxPool <= 4 * 1024, "sure-list loads per thread");
  const int m = blockIdx.x;
  // everything that does not depend on the visible count first
  const uint4 cnt4 = *reinterpret_cast<const uint4 *>(counters + m * 4);
  const uint4 fine4 = *reinterpret_cast<const uint4 *>(fine + (int64_t)m * kHistBins + kHistBins - 4 * (threadIdx.x + 1));
  const rsrc_t r_su = make_rsrc(sure + (int64_t)m * P, (uint32_t)(P * 4));
  int32_t su_pre[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    su_pre[u] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_su, (uint32_t)(threadIdx.x + 1024 * u) * 4u, 0, 0);
  int s;
  const int64_t vis = visible_entries(seq_len, q_seq, q_pos, ratio, m, &s);
  const int64_t nb = (vis + kBlock - 1) / kBlock;
  pool_finalize_body(F, bmax, nb_stride, cnt4, fine4, su_pre, tie, m, nb, cnt4.z, P, pool_out, pool_count);
}


// Re-score the positions of E pool blocks per workgroup (E = 64, or fewer
// when that leaves most of the chip idle).  Slot 8*e + r of a query holds
// the score of position 8*pool[e] + r (-inf when not visible).  Each wave
// first loads its pool entries, then all its rows, then scores.
struct SelBatch {
  SelSet s[kSelSets];
};

// grid (pool chunks, queries, query sets).
template <int DI, int E>
__global__ __launch_bounds__(256) void k_rescore(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                 const int64_t *__restrict__ seq_start,
                                                 const int32_t *__restrict__ seq_len, int ratio,
                                                 const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos,
                                                 int H, const int32_t *__restrict__ pool,
                                                 const int32_t *__restrict__ pool_count, int P,
                                                 float *__restrict__ pscore, SelBatch sb) {
  const int m = blockIdx.y, set = blockIdx.z;
  const uint16_t *q_idx = sb.s[set].q_idx;
  const float *w_idx = sb.s[set].w_idx;
  const int e0 = blockIdx.x * E;
  const int l = lane_id(), n = l & 15, qq = l >> 4, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int TPW = E / 2 / 4;  // tiles per wave
  // the pool entries and the query first: neither depends on the visible
  // count or the pool's length, so their latency overlaps those lookups
  const rsrc_t r_pl = make_rsrc(pool + (int64_t)m * P, (uint32_t)(P * 4));
  int32_t blk_raw[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int e = e0 + 2 * (wv + 4 * k) + (n >> 3);
    blk_raw[k] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_pl, (uint32_t)e * 4u, 0, 0);
  }
  IdxQuery<DI> Q;
  load_idx_query<DI>(q_idx + (int64_t)m * H * DI, w_idx + (int64_t)m * H, H, Q);
  int s;
  const int64_t vis = visible_entries(seq_len, q_seq, q_pos, ratio, m, &s);
  const int cnt = min(pool_count[m], P);
  if (e0 >= cnt) return;
  float *ps = pscore + ((int64_t)set * gridDim.y + m) * 8 * P;
  if (vis == 0) {
    for (int i = threadIdx.x; i < 8 * E; i += blockDim.x)
      if (e0 * 8 + i < 8 * cnt) ps[e0 * 8 + i] = -INFINITY;
    return;
  }
  const int64_t row0 = seq_start[s];
  int64_t pos[TPW];
  bool valid[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int e = e0 + 2 * (wv + 4 * k) + (n >> 3);
    const int32_t blk = (e < cnt) ? blk_raw[k] : -1;
    pos[k] = (int64_t)blk * kBlock + (n & 7);
    valid[k] = blk >= 0 && pos[k] < vis;
  }
  LaneCodes<DI> c[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) load_lane_codes<DI>(codes, scales, row0 + (valid[k] ? pos[k] : 0), qq, c[k]);
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int e = e0 + 2 * (wv + 4 * k) + (n >> 3);
    float sc = tile_score<DI>(Q, c[k]);
    if (!valid[k]) sc = -INFINITY;
    if (qq == 0 && e < cnt) ps[8 * e + (n & 7)] = sc;
  }
}

// Top-K of the scores of one query's slots, run by a workgroup of NT
// threads: thread t owns slots [t*PER, (t+1)*PER), sv[] their scores (-inf:
// no candidate).  The ranking is (score desc, slot asc): on the composite
// G = key << 32 | ~slot (key the order-preserving image of the score), the
// selection is every G >= cut with cut the composite of the K-th entry.  The
// selected slots are handed to emit(rank, i, score) in ascending slot order
// (i the thread-local slot index, rank the output position).  Returns the
// number selected, min(K, #candidates).
//
// Finding the cut: a 4096-bin histogram of d = kmax - key over a window
// anchored at the largest key (bins of 2^13 key units, 1/1024 of an octave;
// the whole key range when the window holds fewer than K keys) gives the bin
// T holding the K-th entry.  Fine bins keep both the LDS atomics (the keys of
// a query cluster within a few octaves) and bin T small: its entries are
// ranked against each other by one wave when at most 64, else narrowed by
// radix passes over their composites.
constexpr int kSelectCand = 2048;   // threshold-bin entries refined by one wave
constexpr int kSelectShift = 13;    // log2 key units per bin of the first window
constexpr int kSelectShiftAll = 32 - kHistBits;

template <int NT>
struct SelectLds {
  uint32_t hist[kHistBins];
  uint32_t h[256];
  uint32_t wmax[NT / 64];
  int wcnt[NT / 64];
  int wsum[NT / 64];
  int T, above, nT, digit, rem, cnt;
  // the selection by output rank, written out in one coalesced pass (a
  // wave's scattered masked stores would queue one instruction per slot)
  int32_t stage[4096];
  float stage_score[2048];
  // the composites of the threshold bin
  uint64_t cand[kSelectCand];
  int ncand;
  uint64_t cut;
};

CSA2_DEV uint32_t wave_incl_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

// Order LDS accesses among the lanes of one wave (no other wave takes part).
CSA2_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Run by wave 0 alone: radix passes of 8 bits from the top over the n
// composites cand[], narrowing (prefix, mask) to the cut of the rem largest;
// stops as soon as the cut's digit bin holds exactly the entries still
// needed.  Afterwards the rem largest are exactly those >= prefix.
CSA2_DEV void wave_refine(const uint64_t *cand, int n, int rem, uint32_t *h, int *s_digit, int *s_rem,
                          int *s_cnt, uint64_t &prefix, uint64_t &mask) {
  const int l = lane_id();
  for (int hi = 64; hi > 0; hi -= 8) {
    const int shift = hi - 8;
    for (int i = l; i < 256; i += 64) h[i] = 0u;
    wave_lds_sync();
    for (int i = l; i < n; i += 64) {
      const uint64_t c = cand[i];
      if ((c & mask) == prefix) atomicAdd(&h[(uint32_t)((c >> shift) & 0xFFull)], 1u);
    }
    wave_lds_sync();
    find_digit(h, rem, s_digit, s_rem, s_cnt);
    wave_lds_sync();
    prefix |= (uint64_t)*s_digit << shift;
    mask |= 0xFFull << shift;
    rem = *s_rem;
    if (*s_cnt == rem) break;
  }
}

template <int NT, int PER, typename Emit>
CSA2_DEV int select_topk(const float (&sv)[PER], int K, SelectLds<NT> &sm, Emit emit) {
  constexpr int NW = NT / 64;
  constexpr int BPT = kHistBins / NT;   // histogram bins per thread in the threshold scan
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t key[PER];
  uint32_t kmx = 0u;
  int nv = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    key[i] = (sv[i] > -INFINITY) ? f2key(sv[i]) : 0u;
    kmx = max(kmx, key[i]);
    nv += key[i] != 0u;
  }
  auto G = [&](int i) { return ((uint64_t)key[i] << 32) | (uint64_t)(~(uint32_t)(tid * PER + i)); };
  for (int i = tid; i < kHistBins / 4; i += NT) reinterpret_cast<uint4 *>(sm.hist)[i] = make_uint4(0u, 0u, 0u, 0u);
  kmx = wave_incl_max(kmx);
  nv = wave_incl_scan(nv);
  if (lane == 63) { sm.wmax[wv] = kmx; sm.wcnt[wv] = nv; }
  if (tid == 0) sm.ncand = 0;
  __syncthreads();
  kmx = 0u;
  int tot_valid = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) { kmx = max(kmx, sm.wmax[w]); tot_valid += sm.wcnt[w]; }
  const int Kp = min(K, tot_valid);
  uint64_t cut = ~0ull;
  if (Kp > 0) {
    // ---- threshold bin T over the window, widened once if it holds < Kp keys ----
    int SH = kSelectShift;
    int T = 0, above = 0, nT = 0;
    for (;;) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint32_t bin = (kmx - key[i]) >> SH;
        if (key[i] != 0u && bin < (uint32_t)kHistBins) atomicAdd(&sm.hist[bin], 1u);
      }
      __syncthreads();
      uint32_t hv[BPT];
      int c = 0;
#pragma unroll
      for (int k = 0; k < BPT; k += 4) {
        const uint4 q = reinterpret_cast<const uint4 *>(sm.hist)[(tid * BPT + k) / 4];
        hv[k] = q.x; hv[k + 1] = q.y; hv[k + 2] = q.z; hv[k + 3] = q.w;
        c += (int)(q.x + q.y + q.z + q.w);
      }
      const int incl = wave_incl_scan(c);
      if (lane == 63) sm.wsum[wv] = incl;
      __syncthreads();
      int before = incl - c, tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int x = sm.wsum[w];
        before += (w < wv) ? x : 0;
        tot += x;
      }
      if (tot >= Kp) {
        if (before < Kp && before + c >= Kp) {
          int cum = before;
#pragma unroll
          for (int k = 0; k < BPT; ++k) {
            if (cum + (int)hv[k] >= Kp) { sm.T = tid * BPT + k; sm.above = cum; sm.nT = (int)hv[k]; break; }
            cum += (int)hv[k];
          }
        }
        __syncthreads();
        T = sm.T; above = sm.above; nT = sm.nT;
        break;
      }
      // fewer than Kp keys in the window: one pass over the whole key range
      for (int i = tid; i < kHistBins / 4; i += NT) reinterpret_cast<uint4 *>(sm.hist)[i] = make_uint4(0u, 0u, 0u, 0u);
      SH = kSelectShiftAll;
      __syncthreads();
    }
    const int rem = Kp - above;
    // keys of bin T: d in [T << SH, (T + 1) << SH), i.e. key in [lo_key, hi_key]
    const uint64_t span_lo = (uint64_t)(T + 1) << SH;
    const uint32_t lo_key = (span_lo > (uint64_t)kmx) ? 1u : kmx - (uint32_t)span_lo + 1u;
    if (rem == nT) {
      cut = (uint64_t)lo_key << 32;             // the whole bin is taken
    } else {
      // ---- bin T's composites into LDS (one atomic per wave) ----
      const uint32_t hi_key = kmx - (uint32_t)((uint64_t)T << SH);
      int nc = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) nc += (key[i] >= lo_key && key[i] <= hi_key);
      const int incl = wave_incl_scan(nc);
      int base = 0;
      if (lane == 63) base = atomicAdd(&sm.ncand, incl);
      base = __builtin_amdgcn_readlane(base, 63) + incl - nc;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (key[i] >= lo_key && key[i] <= hi_key) {
          if (base < kSelectCand) sm.cand[base] = G(i);
          ++base;
        }
      __syncthreads();
      const int n = sm.ncand;
      if (n <= 64) {
        // rank every candidate against the others; the rem-th largest is the cut
        if (wv == 0) {
          const uint64_t c = (lane < n) ? sm.cand[lane] : 0ull;
          const uint32_t clo = (uint32_t)c, chi = (uint32_t)(c >> 32);
          int r = 0;
          for (int j = 0; j < n; ++j) {
            const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)chi, j) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane((int)clo, j);
            r += o > c;
          }
          if (lane < n && r == rem - 1) sm.cut = c;
        }
      } else if (n <= kSelectCand) {
        if (wv == 0) {
          uint64_t pf = 0ull, mk = 0ull;
          wave_refine(sm.cand, n, rem, sm.h, &sm.digit, &sm.rem, &sm.cnt, pf, mk);
          if (tid == 0) sm.cut = pf;
        }
      } else {
        // block-wide radix passes over bin T's composites held in registers
        uint64_t prefix = 0ull, mask = 0ull;
        int r2 = rem;
        for (int hi = 64; hi > 0; hi -= 8) {
          const int shift = hi - 8;
          for (int i = tid; i < 256; i += NT) sm.h[i] = 0u;
          __syncthreads();
#pragma unroll
          for (int i = 0; i < PER; ++i)
            if (key[i] >= lo_key && key[i] <= hi_key && (G(i) & mask) == prefix)
              atomicAdd(&sm.h[(uint32_t)((G(i) >> shift) & 0xFFull)], 1u);
          __syncthreads();
          find_digit(sm.h, r2, &sm.digit, &sm.rem, &sm.cnt);
          __syncthreads();
          prefix |= (uint64_t)sm.digit << shift;
          mask |= 0xFFull << shift;
          r2 = sm.rem;
          if (sm.cnt == r2) break;
        }
        if (tid == 0) sm.cut = prefix;
      }
      __syncthreads();
      cut = sm.cut;
    }
  }
  // ---- selection (G >= cut) in ascending slot order ----
  int nsel = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) nsel += G(i) >= cut;
  const int incl = wave_incl_scan(nsel);
  if (lane == 63) sm.wsum[wv] = incl;
  __syncthreads();
  int rank = incl - nsel;
#pragma unroll
  for (int w = 0; w < NW; ++w) rank += (w < wv) ? sm.wsum[w] : 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (G(i) >= cut) {
      emit(rank, i, sv[i]);
      ++rank;
    }
  }
  return Kp;
}

// The PER scores of thread t's slots [t*PER, (t+1)*PER) of ps[0 .. n).
// ps must be 16-byte aligned.
template <int PER>
CSA2_DEV void load_slot_scores(const float *__restrict__ ps, int n, float (&sv)[PER]) {
  if ((int)(threadIdx.x + 1) * PER <= n) {
    const float4 *src = reinterpret_cast<const float4 *>(ps + threadIdx.x * PER);
#pragma unroll
    for (int k = 0; k < PER / 4; ++k) {
      const float4 v = src[k];
      sv[4 * k] = v.x; sv[4 * k + 1] = v.y; sv[4 * k + 2] = v.z; sv[4 * k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int slot = threadIdx.x * PER + i;
      sv[i] = (slot < n) ? ps[slot] : -INFINITY;
    }
  }
}

// Top-K over the re-scored pool, one workgroup per query.  Slot 8e + r is
// position 8*pool[e] + r; slot order equals position order because the pool
// is ascending, so ties on the score resolve to the lower position and the
// output comes out in ascending position order.
// grid (queries, query sets).
template <int NT, int PER>
__global__ __launch_bounds__(NT) void k_topk_select(const float *__restrict__ pscore,
                                                    const int32_t *__restrict__ pool,
                                                    const int32_t *__restrict__ pool_count, int P, int K,
                                                    SelBatch sb) {
  __shared__ __attribute__((aligned(16))) SelectLds<NT> sm;
  const int m = blockIdx.x, set = blockIdx.y;
  int32_t *__restrict__ topk_out = sb.s[set].topk;
  float *__restrict__ topk_score = sb.s[set].score;
  pscore += (int64_t)set * gridDim.x * 8 * P;
  // the pool blocks and scores of this thread's slots are loaded before the
  // pool's length is known (slots past it are masked once it is)
  const rsrc_t r_pl = make_rsrc(pool + (int64_t)m * P, (uint32_t)(P * 4));
  int32_t blk[PER / kBlock];
#pragma unroll
  for (int b = 0; b < PER / kBlock; ++b)
    blk[b] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
        r_pl, (uint32_t)((int)threadIdx.x * (PER / kBlock) + b) * 4u, 0, 0);
  const rsrc_t r_ps = make_rsrc(pscore + (int64_t)m * 8 * P, (uint32_t)(8 * P * 4));
  float sv[PER];
#pragma unroll
  for (int k = 0; k < PER / 4; ++k) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r_ps, (uint32_t)(threadIdx.x * PER + 4 * k) * 4u, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[4 * k + e] = __uint_as_float(x[e]);
  }
  const int cnt = min(pool_count[m], P);
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if ((int)threadIdx.x * PER + i >= 8 * cnt) sv[i] = -INFINITY;
  int32_t *out = topk_out + (int64_t)m * K;
  float *osc = topk_score ? topk_score + (int64_t)m * K : nullptr;
  const int Kp = select_topk<NT, PER>(sv, K, sm, [&](int rank, int i, float v) {
    sm.stage[rank] = blk[i / kBlock] * kBlock + (i % kBlock);
    sm.stage_score[rank] = v;
  });
  __syncthreads();
  for (int i = threadIdx.x; i < K; i += NT) {
    out[i] = (i < Kp) ? sm.stage[i] : -1;
    if (osc) osc[i] = (i < Kp) ? sm.stage_score[i] : __builtin_nanf("");
  }
}

// Pool of the top P blocks by (block max desc, block id asc) straight from
// the block maxima, one workgroup per query: the blocks that hold a visible
// position are the slots.  Used when every block of a query fits the
// workgroup's registers.
template <int NT, int PER>
__global__ __launch_bounds__(NT) void k_block_select(const float *__restrict__ bmax, int64_t nb_stride,
                                                     const int32_t *__restrict__ seq_len,
                                                     const int32_t *__restrict__ q_seq,
                                                     const int32_t *__restrict__ q_pos, int ratio, int P,
                                                     int32_t *__restrict__ pool_out, int32_t *__restrict__ pool_count) {
  __shared__ __attribute__((aligned(16))) SelectLds<NT> sm;
  const int m = blockIdx.x;
  int s;
  const int64_t vis = visible_entries(seq_len, q_seq, q_pos, ratio, m, &s);
  const int nb = (int)((vis + kBlock - 1) / kBlock);
  float sv[PER];
  load_slot_scores<PER>(bmax + (int64_t)m * nb_stride, nb, sv);
  int32_t *out = pool_out + (int64_t)m * P;
  const int Kp = select_topk<NT, PER>(sv, P, sm, [&](int rank, int i, float) {
    sm.stage[rank] = (int32_t)(threadIdx.x * PER + i);
  });
  __syncthreads();
  for (int i = threadIdx.x; i < P; i += NT) out[i] = (i < Kp) ? sm.stage[i] : -1;
  if (threadIdx.x == 0) pool_count[m] = Kp;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Tiles per scan workgroup: the largest chunk whose grid still gives about
// one workgroup per CU.
static int scan_tiles(int64_t max_len, int m) {
  auto chunks_of = [&](int chunk) { return (max_len + chunk - 1) / chunk; };
  if (chunks_of(kScanChunk) * m >= kScanMinGrid) return kScanTiles;
  if (chunks_of(kScanChunk / 4) * m >= kScanMinGrid) return kScanTiles / 4;
  return kScanTiles / 16;
}

// Histogram replicas per query: about 8 scan workgroups share each one.
static int hist_replicas(int64_t max_len, int m) {
  const int64_t chunk = 16 * (int64_t)scan_tiles(max_len, m);
  const int64_t wgs = (max_len + chunk - 1) / chunk;  // workgroups per query
  return (int)std::max<int64_t>(1, std::min<int64_t>(kHistMaxReplicas, wgs / 8));
}

IndexWs index_ws_layout(int64_t max_len, int m, int pool_blocks, int top_k, int n_sets) {
  (void)top_k;
  IndexWs w{};
  w.hist_rep = hist_replicas(max_len, m);
  // room for the largest scan chunk's rounding (smaller chunks need less)
  const int64_t chunks = (max_len + kScanChunk - 1) / kScanChunk;
  w.nb_max = (chunks > 0 ? chunks : 1) * kScanBlocks;
  w.slots = 8 * pool_blocks;
  size_t off = 0;
  w.bmax = off;     off = align256(off + sizeof(float) * (size_t)m * w.nb_max);
  w.hist = off;     off = align256(off + sizeof(uint32_t) * (size_t)m * w.hist_rep * kHistBins);
  w.counters = off; off = align256(off + sizeof(uint32_t) * (size_t)m * 4);
  w.fine = off;     off = align256(off + sizeof(uint32_t) * (size_t)m * kHistBins);
  w.sure = off;     off = align256(off + sizeof(int32_t) * (size_t)m * pool_blocks);
  w.tie = off;      off = align256(off + sizeof(int32_t) * (size_t)m * w.nb_max);
  w.pscore = off;   off = align256(off + sizeof(float) * (size_t)std::max(1, n_sets) * m * w.slots);
  w.total = off;
  return w;
}

template <int DI>
static int rescore_and_select(const csa2_fp4_cache &idx, const csa2_queries &qs, int heads, const int32_t *pool,
                              const int32_t *pool_count, int P, int K, const SelSet *sets, int n_sets,
                              float *pscore, hipStream_t stream) {
  for (int b0 = 0; b0 < n_sets; b0 += kSelSets) {
    const int ns = std::min(kSelSets, n_sets - b0);
    SelBatch sb{};
    for (int i = 0; i < ns; ++i) sb.s[i] = sets[b0 + i];
    float *ps = pscore + (size_t)b0 * qs.m * 8 * P;
    // 64 blocks per workgroup, or 16 when that would leave most CUs idle (few queries)
    if ((int64_t)((P + kRescoreEntries - 1) / kRescoreEntries) * qs.m * ns >= 512) {
      const dim3 g5((P + kRescoreEntries - 1) / kRescoreEntries, qs.m, ns);
      hipLaunchKernelGGL((k_rescore<DI, kRescoreEntries>), g5, dim3(256), 0, stream, idx.codes, idx.scales,
                         idx.seq_start, idx.seq_len, idx.ratio, qs.seq, qs.pos, heads, pool, pool_count, P, ps, sb);
    } else {
      const dim3 g5((P + 15) / 16, qs.m, ns);
      hipLaunchKernelGGL((k_rescore<DI, 16>), g5, dim3(256), 0, stream, idx.codes, idx.scales, idx.seq_start,
                         idx.seq_len, idx.ratio, qs.seq, qs.pos, heads, pool, pool_count, P, ps, sb);
    }
    // 8P <= 32768 slots (P <= 4096)
    const dim3 g6(qs.m, ns);
    if (8 * P <= 256 * 16)
      hipLaunchKernelGGL((k_topk_select<256, 16>), g6, dim3(256), 0, stream, ps, pool, pool_count, P, K, sb);
    else if (8 * P <= 1024 * 16)
      hipLaunchKernelGGL((k_topk_select<1024, 16>), g6, dim3(1024), 0, stream, ps, pool, pool_count, P, K, sb);
    else
      hipLaunchKernelGGL((k_topk_select<1024, 32>), g6, dim3(1024), 0, stream, ps, pool, pool_count, P, K, sb);
  }
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

// The pool from the block maxima and their histogram: the filter (which
// finds the threshold bin itself), then the finalisation.
static void pool_from_hist(const csa2_fp4_cache &idx, const csa2_queries &qs, int P, int64_t nbq, const IndexWs &L,
                           const float *bmax, const uint32_t *hist, uint32_t *counters, int32_t *sure, int32_t *tie,
                           int32_t *pool_out, int32_t *pool_count, hipStream_t stream) {
  (void)nbq;
  const dim3 g3((unsigned)((L.nb_max + kFilterBlocks - 1) / kFilterBlocks), qs.m);
  uint32_t *fine = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(counters) + (L.fine - L.counters));
  hipLaunchKernelGGL(k_pool_filter, g3, dim3(256), 0, stream, bmax, L.nb_max, hist, L.hist_rep, idx.seq_len, qs.seq,
                     qs.pos, idx.ratio, P, counters, fine, sure, tie);
  hipLaunchKernelGGL(k_pool_finalize, dim3(qs.m), dim3(1024), 0, stream, bmax, L.nb_max, counters, fine, sure, tie,
                     idx.seq_len, qs.seq, qs.pos, idx.ratio, P, pool_out, pool_count);
}

template <int DI>
static int index_pool_impl(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                           const float *w_idx, int heads, int P, int K, int32_t *pool_out, int32_t *pool_count,
                           void *ws, hipStream_t stream, bool cleared) {
  const IndexWs L = index_ws_layout(idx.max_len, qs.m, P, K);
  char *base = static_cast<char *>(ws);
  float *bmax = reinterpret_cast<float *>(base + L.bmax);
  uint32_t *hist = reinterpret_cast<uint32_t *>(base + L.hist);
  uint32_t *counters = reinterpret_cast<uint32_t *>(base + L.counters);
  int32_t *sure = reinterpret_cast<int32_t *>(base + L.sure);
  int32_t *tie = reinterpret_cast<int32_t *>(base + L.tie);

  // hist, counters and fine are adjacent: clear them with one fill kernel
  const int64_t nz = (int64_t)((L.sure - L.hist) / sizeof(uint32_t));   // a multiple of 64 (256-byte offsets)
  const int64_t nbq = (idx.max_len + kBlock - 1) / kBlock;   // blocks of the longest sequence
  if ((qs.run == 2 || qs.run == 4) && heads <= 8 && qs.m % qs.run == 0 && nbq > kBlockSelectMax) {
    // long contexts, runs of 2 or 4 tokens: the first scan with the run's
    // queries sharing each MFMA tile, then the pool from the histograms
    if (!cleared)
      hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((nz / 4 + 255) / 256)), dim3(256), 0, stream, hist, nz);
    const int runs = qs.m / qs.run;
    auto chunks_of = [&](int chunk) { return (idx.max_len + chunk - 1) / chunk; };
#define CSA2_SCAN_RUN(RR, T)                                                                                  \
  CSA2_TIMED_LAUNCH(kTimedScan, (k_scan_run<DI, RR, kScanWaves, T>), dim3((unsigned)chunks_of(T * 16), runs),   \
                    dim3(64 * kScanWaves), stream, idx.codes, idx.scales, idx.seq_start, idx.seq_len, idx.ratio, \
                    qs.seq, qs.pos, q_idx, w_idx, heads, bmax, L.nb_max, hist, L.hist_rep)
#define CSA2_SCAN_RUN_T(RR)                                                        \
    switch (scan_tiles(idx.max_len, runs)) {                                       \
      case kScanTiles: CSA2_SCAN_RUN(RR, kScanTiles); break;                       \
      case kScanTiles / 4: CSA2_SCAN_RUN(RR, kScanTiles / 4); break;               \
      default: CSA2_SCAN_RUN(RR, kScanTiles / 16); break;                          \
    }
    if (qs.run == 2) { CSA2_SCAN_RUN_T(2); } else { CSA2_SCAN_RUN_T(4); }
#undef CSA2_SCAN_RUN_T
#undef CSA2_SCAN_RUN
    pool_from_hist(idx, qs, P, nbq, L, bmax, hist, counters, sure, tie, pool_out, pool_count, stream);
    return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
  }
  if (qs.run >= 2) {
    // queries in runs of one sequence: every streamed indexer entry is scored
    // against all the queries of its sequence at once (multi-query MFMA
    // kernel), then each query's pool comes from its block maxima
    int st = launch_score_blocks(idx, qs, q_idx, w_idx, heads, bmax, L.nb_max, stream);
    if (st != CSA2_OK) return st;
    if (nbq <= kBlockSelectMax) {
      st = launch_block_select(bmax, L.nb_max, nbq > 0 ? nbq : 1, idx, qs, P, pool_out, pool_count, stream);
      if (st != CSA2_OK) return st;
    } else {
      if (!cleared)
        hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((nz / 4 + 255) / 256)), dim3(256), 0, stream, hist, nz);
      hipLaunchKernelGGL(k_bmax_hist, dim3((unsigned)((nbq + kFilterBlocks - 1) / kFilterBlocks), qs.m), dim3(256),
                         0, stream, bmax, L.nb_max, idx.seq_len, qs.seq, qs.pos, idx.ratio, hist, L.hist_rep);
      pool_from_hist(idx, qs, P, nbq, L, bmax, hist, counters, sure, tie, pool_out, pool_count, stream);
    }
    return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
  }
  if (!cleared)
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((nz / 4 + 255) / 256)), dim3(256), 0, stream, hist, nz);
  if (idx.max_len > 0) {
    auto chunks_of = [&](int chunk) { return (idx.max_len + chunk - 1) / chunk; };
#define CSA2_SCAN(T)                                                                                        \
  CSA2_TIMED_LAUNCH(kTimedScan, (k_scan<DI, kScanWaves, T>), dim3((unsigned)chunks_of(T * 16), qs.m),    \
                    dim3(64 * kScanWaves), stream, idx.codes, idx.scales, idx.seq_start, idx.seq_len, idx.ratio, \
                    qs.seq, qs.pos, q_idx, w_idx, heads, bmax, L.nb_max, hist, L.hist_rep)
    switch (scan_tiles(idx.max_len, qs.m)) {
      case kScanTiles: CSA2_SCAN(kScanTiles); break;
      case kScanTiles / 4: CSA2_SCAN(kScanTiles / 4); break;
      default: CSA2_SCAN(kScanTiles / 16); break;
    }
#undef CSA2_SCAN
  }
  pool_from_hist(idx, qs, P, nbq, L, bmax, hist, counters, sure, tie, pool_out, pool_count, stream);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

int launch_index_pool(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx, const float *w_idx,
                      int heads, int P, int K, int32_t *pool_out, int32_t *pool_count, void *ws,
                      hipStream_t stream, bool ws_cleared) {
  switch (idx.dim) {
    case 64:
      return index_pool_impl<64>(idx, qs, q_idx, w_idx, heads, P, K, pool_out, pool_count, ws, stream, ws_cleared);
    case 128:
      return index_pool_impl<128>(idx, qs, q_idx, w_idx, heads, P, K, pool_out, pool_count, ws, stream, ws_cleared);
    case 256:
      return index_pool_impl<256>(idx, qs, q_idx, w_idx, heads, P, K, pool_out, pool_count, ws, stream, ws_cleared);
    default: return CSA2_ERR_UNSUPPORTED;
  }
}

int launch_rescore_select(const csa2_fp4_cache &idx, const csa2_queries &qs, int heads, const int32_t *pool,
                          const int32_t *pool_count, int P, int K, const SelSet *sets, int n_sets, float *pscore,
                          hipStream_t stream) {
  switch (idx.dim) {
    case 64: return rescore_and_select<64>(idx, qs, heads, pool, pool_count, P, K, sets, n_sets, pscore, stream);
    case 128: return rescore_and_select<128>(idx, qs, heads, pool, pool_count, P, K, sets, n_sets, pscore, stream);
    case 256: return rescore_and_select<256>(idx, qs, heads, pool, pool_count, P, K, sets, n_sets, pscore, stream);
    default: return CSA2_ERR_UNSUPPORTED;
  }
}

int launch_index_full(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                      const float *w_idx, int heads, int P, int K, int32_t *pool_out, int32_t *pool_count,
                      int32_t *topk_out, float *topk_score, void *ws, hipStream_t stream) {
  int st = launch_index_pool(idx, qs, q_idx, w_idx, heads, P, K, pool_out, pool_count, ws, stream);
  if (st) return st;
  const IndexWs L = index_ws_layout(idx.max_len, qs.m, P, K);
  const SelSet set{q_idx, w_idx, topk_out, topk_score};
  return launch_rescore_select(idx, qs, heads, pool_out, pool_count, P, K, &set, 1,
                               reinterpret_cast<float *>(static_cast<char *>(ws) + L.pscore), stream);
}

int launch_block_select(const float *bmax, int64_t nb_stride, int64_t nb_max, const csa2_fp4_cache &idx,
                        const csa2_queries &qs, int P, int32_t *pool_out, int32_t *pool_count, hipStream_t stream) {
  if (qs.m == 0) return CSA2_OK;
#define CSA2_BSEL(NT, PER)                                                                                      \
  hipLaunchKernelGGL((k_block_select<NT, PER>), dim3(qs.m), dim3(NT), 0, stream, bmax, nb_stride, idx.seq_len, \
                     qs.seq, qs.pos, idx.ratio, P, pool_out, pool_count)
  if (nb_max <= 256 * 16) CSA2_BSEL(256, 16);
  else if (nb_max <= 256 * 32) CSA2_BSEL(256, 32);
  else if (nb_max <= 256 * 64) CSA2_BSEL(256, 64);
  else if (nb_max <= 1024 * 32) CSA2_BSEL(1024, 32);
  else if (nb_max <= kBlockSelectMax) CSA2_BSEL(1024, 64);
  else return CSA2_ERR_UNSUPPORTED;
#undef CSA2_BSEL
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

int launch_reindex(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx, const float *w_idx,
                   int heads, const int32_t *pool_in, const int32_t *pool_count, int P, int K, int32_t *topk_out,
                   float *topk_score, void *ws, hipStream_t stream) {
  const IndexWs L = index_ws_layout(idx.max_len, qs.m, P, K);
  float *pscore = reinterpret_cast<float *>(static_cast<char *>(ws) + L.pscore);
  const SelSet set{q_idx, w_idx, topk_out, topk_score};
  return launch_rescore_select(idx, qs, heads, pool_in, pool_count, P, K, &set, 1, pscore, stream);
}

}  // namespace csa2
