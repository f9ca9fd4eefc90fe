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
constexpr int kFilterBlocks = 4096;              // blocks per pool-filter workgroup (fewer workgroups share each list counter)
constexpr int kRescoreEntries = 64;              // pool blocks per re-score workgroup (at most)


// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

__global__ void k_zero_u32(uint32_t *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
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

// Threshold bin of each query (one workgroup per query): merge the scan's
// histogram replicas and find the bin that holds the need-th largest block
// maximum, need = min(P, visible blocks); -1 when every block is taken.
// Written to counters[4m + 2] for the filter and the finalisation.
__global__ __launch_bounds__(256) void k_hist_threshold(const uint32_t *__restrict__ hist, int hist_rep,
                                                        const int32_t *__restrict__ seq_len,
                                                        const int32_t *__restrict__ q_seq,
                                                        const int32_t *__restrict__ q_pos, int ratio, int P,
                                                        uint32_t *__restrict__ counters) {
  __shared__ int s_scan[8];
  __shared__ int s_T;
  const int m = blockIdx.x;
  int s;
  const int64_t vis = visible_entries(seq_len, q_seq, q_pos, ratio, m, &s);
  const int64_t nb = (vis + kBlock - 1) / kBlock;
  if (threadIdx.x == 0) s_T = -1;
  __syncthreads();
  if (nb > P) {
    const int64_t need = P;
    // thread t owns bins [4096-16(t+1), 4096-16t) (thread 0 = highest bins)
    const int hi = kHistBins - 16 * threadIdx.x;
    int hv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) hv[k] = 0;
    // every replica's loads in flight at once (a fixed trip count, replicas
    // past hist_rep read replica 0 and count nothing)
    uint4 x[kHistMaxReplicas][4];
#pragma unroll
    for (int r = 0; r < kHistMaxReplicas; ++r) {
      const int rr = r < hist_rep ? r : 0;
      const uint4 *h4 = reinterpret_cast<const uint4 *>(hist + ((int64_t)m * hist_rep + rr) * kHistBins + hi - 16);
#pragma unroll
      for (int k = 0; k < 4; ++k) x[r][k] = h4[k];
    }
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
    if (before < need && before + c >= need) {
      int cum = before;
      for (int k = 15; k >= 0; --k) {
        cum += hv[k];
        if (cum >= need) { s_T = hi - 16 + k; break; }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) counters[m * 4 + 2] = (uint32_t)s_T;
}

// Pool filter: blocks above the threshold bin are in the pool for sure,
// blocks in it go to the tie list.  Appends are gathered in
// LDS and reserved in the global lists with one atomic per list per workgroup.
__global__ __launch_bounds__(256) void k_pool_filter(const float *__restrict__ bmax, int64_t nb_stride,
                                                     const int32_t *__restrict__ seq_len, const int32_t *__restrict__ q_seq,
                                                     const int32_t *__restrict__ q_pos, int ratio, int P,
                                                     uint32_t *__restrict__ counters, int32_t *__restrict__ sure,
                                                     int32_t *__restrict__ tie) {
  __shared__ int s_ns, s_nt, s_bs, s_bt;
  __shared__ int32_t s_sure[kFilterBlocks], s_tie[kFilterBlocks];
  const int m = blockIdx.y;
  int s;
  const int64_t vis = visible_entries(seq_len, q_seq, q_pos, ratio, m, &s);
  const int64_t nb = (vis + kBlock - 1) / kBlock;
  const int64_t b0 = (int64_t)blockIdx.x * kFilterBlocks;
  if (b0 >= nb) return;
  if (threadIdx.x == 0) { s_ns = 0; s_nt = 0; }
  __syncthreads();
  const int T = (int)counters[m * 4 + 2];
  const float *bm = bmax + (int64_t)m * nb_stride;
  for (int j = 0; j < kFilterBlocks / 256; ++j) {
    const int64_t b = b0 + j * 256 + threadIdx.x;
    const bool ok = b < nb;
    const int bin = ok ? (int)(f2key(bm[b]) >> (32 - kHistBits)) : -2;
    wave_append(ok && bin > T, (int32_t)b, &s_ns, s_sure);
    wave_append(ok && bin == T, (int32_t)b, &s_nt, s_tie);
  }
  __syncthreads();
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

__global__ __launch_bounds__(1024) void k_pool_finalize(const float *__restrict__ bmax, int64_t nb_stride,
                                                        const uint32_t *__restrict__ counters,
                                                        const int32_t *__restrict__ sure,
                                                        const int32_t *__restrict__ tie,
                                                        const int32_t *__restrict__ seq_len,
                                                        const int32_t *__restrict__ q_seq,
                                                        const int32_t *__restrict__ q_pos, int ratio, int P,
                                                        int32_t *__restrict__ pool_out,
                                                        int32_t *__restrict__ pool_count) {
  __shared__ uint32_t s_bits[kBitmapWords];
  __shared__ int32_t s_pool[kMaxPool];
  __shared__ uint32_t s_h[256];
  __shared__ int s_scan[17];
  __shared__ int s_digit, s_rem, s_cnt, s_n;
  const int m = blockIdx.x;
  int s;
  const int64_t vis = visible_entries(seq_len, q_seq, q_pos, ratio, m, &s);
  const int64_t nb = (vis + kBlock - 1) / kBlock;
  // counts as far as the lists reach (they never exceed them when the
  // histogram agrees with the block maxima)
  const int n_sure = (int)min<uint32_t>(counters[m * 4 + 0], (uint32_t)P);
  const int n_tie = (int)min<int64_t>((int64_t)counters[m * 4 + 1], nb_stride);
  const uint32_t s_T = counters[m * 4 + 2];  // threshold bin (meaningful when there are ties)
  const int need = (int)min<int64_t>(min<int64_t>(P, nb), (int64_t)n_sure + n_tie);
  const int need_t = need - n_sure;
  const int32_t *su = sure + (int64_t)m * P;
  const int32_t *ti = tie + (int64_t)m * nb_stride;
  const float *bm = bmax + (int64_t)m * nb_stride;
  const bool use_bits = nb <= 32 * (int64_t)kBitmapWords;
  const int words = (int)((nb + 31) / 32);
  if (use_bits)
    for (int i = threadIdx.x; i < words; i += blockDim.x) s_bits[i] = 0u;
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  auto take = [&](int32_t b) {
    if (use_bits) atomicOr(&s_bits[b >> 5], 1u << (b & 31));
    else {
      const int slot = atomicAdd(&s_n, 1);
      if (slot < kMaxPool) s_pool[slot] = b;
    }
  };
  for (int i = threadIdx.x; i < n_sure; i += blockDim.x)
    if ((uint64_t)su[i] < (uint64_t)nb) take(su[i]);
  if (need_t > 0) {
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
        for (int i = threadIdx.x; i < 256; i += blockDim.x) s_h[i] = 0u;
        __syncthreads();
        for (int i = threadIdx.x; i < n_tie; i += blockDim.x) {
          const int32_t b = ti[i];
          if ((uint64_t)b >= (uint64_t)nb) continue;
          const uint64_t c = ((uint64_t)f2key(bm[b]) << 32) | (uint64_t)(~(uint32_t)b);
          if ((c & mask) == prefix) atomicAdd(&s_h[(c >> shift) & dmask], 1u);
        }
        __syncthreads();
        find_digit(s_h, rem, &s_digit, &s_rem, &s_cnt);
        __syncthreads();
        prefix |= (uint64_t)s_digit << shift;
        mask |= dmask << shift;
        rem = s_rem;
        if (s_cnt == rem) break;
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
      if (w < words) cnt += __popc(s_bits[w]);
    }
    int tot;
    int pos = block_exclusive_scan<1024>(cnt, s_scan, &tot);
    for (int k = 0; k < wpt; ++k) {
      const int w = threadIdx.x * wpt + k;
      if (w >= words) break;
      uint32_t bits = s_bits[w];
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
    for (int i = min(s_n, need) + threadIdx.x; i < n2; i += blockDim.x) s_pool[i] = 0x7FFFFFFF;
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = threadIdx.x; i < n2; i += blockDim.x) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const int32_t a = s_pool[i], b = s_pool[ixj];
            const bool up = (i & k) == 0;
            if ((a > b) == up) { s_pool[i] = b; s_pool[ixj] = a; }
          }
        }
        __syncthreads();
      }
    }
    for (int i = threadIdx.x; i < need; i += blockDim.x) out[i] = s_pool[i];
  }
  for (int i = need + threadIdx.x; i < P; i += blockDim.x) out[i] = -1;
  if (threadIdx.x == 0) pool_count[m] = need;
}

// Re-score the positions of E pool blocks per workgroup (E = 64, or fewer
// when that leaves most of the chip idle).  Slot 8*e + r of a query holds
// the score of position 8*pool[e] + r (-inf when not visible).  Each wave
// first loads its pool entries, then all its rows, then scores.
template <int DI, int E>
__global__ __launch_bounds__(256) void k_rescore(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                 const int64_t *__restrict__ seq_start,
                                                 const int32_t *__restrict__ seq_len, int ratio,
                                                 const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos,
                                                 const uint16_t *__restrict__ q_idx, const float *__restrict__ w_idx,
                                                 int H, const int32_t *__restrict__ pool,
                                                 const int32_t *__restrict__ pool_count, int P,
                                                 float *__restrict__ pscore) {
  const int m = blockIdx.y;
  int s;
  const int64_t vis = visible_entries(seq_len, q_seq, q_pos, ratio, m, &s);
  const int cnt = min(pool_count[m], P);
  const int e0 = blockIdx.x * E;
  if (e0 >= cnt) return;
  float *ps = pscore + (int64_t)m * 8 * P;
  const int l = lane_id(), n = l & 15, qq = l >> 4, wv = threadIdx.x >> 6;
  if (vis == 0) {
    for (int i = threadIdx.x; i < 8 * E; i += blockDim.x)
      if (e0 * 8 + i < 8 * cnt) ps[e0 * 8 + i] = -INFINITY;
    return;
  }
  const int64_t row0 = seq_start[s];
  const int32_t *pl = pool + (int64_t)m * P;
  constexpr int TPW = E / 2 / 4;  // tiles per wave
  int64_t pos[TPW];
  bool valid[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int e = e0 + 2 * (wv + 4 * k) + (n >> 3);
    const int32_t blk = (e < cnt) ? pl[e] : -1;
    pos[k] = (int64_t)blk * kBlock + (n & 7);
    valid[k] = blk >= 0 && pos[k] < vis;
  }
  LaneCodes<DI> c[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) load_lane_codes<DI>(codes, scales, row0 + (valid[k] ? pos[k] : 0), qq, c[k]);
  IdxQuery<DI> Q;
  load_idx_query<DI>(q_idx + (int64_t)m * H * DI, w_idx + (int64_t)m * H, H, Q);
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int e = e0 + 2 * (wv + 4 * k) + (n >> 3);
    float sc = tile_score<DI>(Q, c[k]);
    if (!valid[k]) sc = -INFINITY;
    if (qq == 0 && e < cnt) ps[8 * e + (n & 7)] = sc;
  }
}

// Top-K by radix select over the scores of one query's slots, run by a
// workgroup of NT threads: thread t owns slots [t*PER, (t+1)*PER), sv[] their
// scores (-inf: no candidate).  The ranking is (score desc, slot asc); the
// selected slots are handed to emit(rank, i, score) in ascending slot order
// (i the thread-local slot index, rank the output position).  Radix passes
// count into one 256-bin histogram per wave, then merge.  Returns the number
// selected, min(K, #candidates).
template <int NT>
struct SelectLds {
  uint32_t wh[NT / 64 * 256];
  uint32_t h[256];
  int scan[NT / 64 + 1];
  int digit, rem, cnt;
};

template <int NT, int PER, typename Emit>
CSA2_DEV int select_topk(const float (&sv)[PER], int K, SelectLds<NT> &sm, Emit emit) {
  constexpr int NW = NT / 64;
  const int wv = threadIdx.x >> 6;
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = (sv[i] > -INFINITY) ? f2key(sv[i]) : 0u;
  int nvalid = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) nvalid += key[i] != 0u;
  int total;
  (void)block_exclusive_scan<NT>(nvalid, sm.scan, &total);
  const int Kp = min(K, total);
  uint32_t kstar = 0xFFFFFFFFu, kmask = 0xFFFFFFFFu;
  int rem = 0;
  if (Kp > 0) {
    uint32_t prefix = 0, mask = 0;
    rem = Kp;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = threadIdx.x; i < NW * 256 / 4; i += NT)
        reinterpret_cast<uint4 *>(sm.wh)[i] = make_uint4(0u, 0u, 0u, 0u);
      __syncthreads();
      uint32_t *wh = sm.wh + wv * 256;
      // Scores cluster in a few digit values (the high digits especially), so
      // the lanes of a wave would hit one LDS counter together: each thread
      // first folds its keys into at most two (digit, count) pairs.
      uint32_t d0 = 0u, c0 = 0u, d1 = 0u, c1 = 0u;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (key[i] == 0u || (key[i] & mask) != prefix) continue;
        const uint32_t d = (key[i] >> shift) & 255u;
        if (c0 == 0u || d == d0) { d0 = d; ++c0; }
        else if (c1 == 0u || d == d1) { d1 = d; ++c1; }
        else atomicAdd(&wh[d], 1u);
      }
      if (c0) atomicAdd(&wh[d0], c0);
      if (c1) atomicAdd(&wh[d1], c1);
      __syncthreads();
      for (int i = threadIdx.x; i < 256; i += NT) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) t += sm.wh[w * 256 + i];
        sm.h[i] = t;
      }
      __syncthreads();
      find_digit(sm.h, rem, &sm.digit, &sm.rem, &sm.cnt);
      __syncthreads();
      prefix |= (uint32_t)sm.digit << shift;
      mask |= 255u << shift;
      rem = sm.rem;
      // every key left in the cut's bin is taken: the lower digits cannot matter
      if (sm.cnt == rem) break;
    }
    kstar = prefix;
    kmask = mask;
  }
  // keys above the cut (on the decided digits) are taken; keys equal to it
  // are ranked by slot (lowest first), then compaction
  int neq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) neq += (Kp > 0 && (key[i] & kmask) == kstar);
  int tmp;
  int eq_before = block_exclusive_scan<NT>(neq, sm.scan, &tmp);
  bool sel[PER];
  int nsel = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    bool takeit = false;
    if (Kp > 0 && key[i] != 0u) {
      const uint32_t km = key[i] & kmask;
      if (km > kstar) takeit = true;
      else if (km == kstar) { takeit = eq_before < rem; ++eq_before; }
    }
    sel[i] = takeit;
    nsel += takeit;
  }
  int rank = block_exclusive_scan<NT>(nsel, sm.scan, &tmp);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (sel[i]) {
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
template <int NT, int PER>
__global__ __launch_bounds__(NT) void k_topk_select(const float *__restrict__ pscore,
                                                    const int32_t *__restrict__ pool,
                                                    const int32_t *__restrict__ pool_count, int P, int K,
                                                    int32_t *__restrict__ topk_out, float *__restrict__ topk_score) {
  __shared__ __attribute__((aligned(16))) SelectLds<NT> sm;
  const int m = blockIdx.x;
  const int cnt = min(pool_count[m], P);
  int32_t blk[PER / kBlock];     // pool blocks of this thread's slots, loaded up front
  const int32_t *pl = pool + (int64_t)m * P;
#pragma unroll
  for (int b = 0; b < PER / kBlock; ++b) blk[b] = pl[min((int)threadIdx.x * (PER / kBlock) + b, max(cnt, 1) - 1)];
  float sv[PER];
  load_slot_scores<PER>(pscore + (int64_t)m * 8 * P, 8 * cnt, sv);
  int32_t *out = topk_out + (int64_t)m * K;
  float *osc = topk_score ? topk_score + (int64_t)m * K : nullptr;
  const int Kp = select_topk<NT, PER>(sv, K, sm, [&](int rank, int i, float v) {
    out[rank] = blk[i / kBlock] * kBlock + (i % kBlock);
    if (osc) osc[rank] = v;
  });
  for (int i = Kp + threadIdx.x; i < K; i += NT) {
    out[i] = -1;
    if (osc) osc[i] = __builtin_nanf("");
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
    out[rank] = (int32_t)(threadIdx.x * PER + i);
  });
  for (int i = Kp + threadIdx.x; i < P; i += NT) out[i] = -1;
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

IndexWs index_ws_layout(int64_t max_len, int m, int pool_blocks, int top_k) {
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
  w.sure = off;     off = align256(off + sizeof(int32_t) * (size_t)m * pool_blocks);
  w.tie = off;      off = align256(off + sizeof(int32_t) * (size_t)m * w.nb_max);
  w.pscore = off;   off = align256(off + sizeof(float) * (size_t)m * w.slots);
  w.total = off;
  return w;
}

template <int DI>
static int rescore_and_select(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                              const float *w_idx, int heads, const int32_t *pool, const int32_t *pool_count,
                              int P, int K, int32_t *topk_out, float *topk_score, float *pscore,
                              hipStream_t stream) {
  // 64 blocks per workgroup, or 16 when that would leave most CUs idle (few queries)
  if ((int64_t)((P + kRescoreEntries - 1) / kRescoreEntries) * qs.m >= 512) {
    const dim3 g5((P + kRescoreEntries - 1) / kRescoreEntries, qs.m);
    hipLaunchKernelGGL((k_rescore<DI, kRescoreEntries>), g5, dim3(256), 0, stream, idx.codes, idx.scales,
                       idx.seq_start, idx.seq_len, idx.ratio, qs.seq, qs.pos, q_idx, w_idx, heads, pool, pool_count,
                       P, pscore);
  } else {
    const dim3 g5((P + 15) / 16, qs.m);
    hipLaunchKernelGGL((k_rescore<DI, 16>), g5, dim3(256), 0, stream, idx.codes, idx.scales, idx.seq_start,
                       idx.seq_len, idx.ratio, qs.seq, qs.pos, q_idx, w_idx, heads, pool, pool_count, P, pscore);
  }
  // 8P <= 32768 slots (P <= 4096)
  if (8 * P <= 256 * 16)
    hipLaunchKernelGGL((k_topk_select<256, 16>), dim3(qs.m), dim3(256), 0, stream, pscore, pool, pool_count, P, K,
                       topk_out, topk_score);
  else if (8 * P <= 1024 * 16)
    hipLaunchKernelGGL((k_topk_select<1024, 16>), dim3(qs.m), dim3(1024), 0, stream, pscore, pool, pool_count, P,
                       K, topk_out, topk_score);
  else
    hipLaunchKernelGGL((k_topk_select<1024, 32>), dim3(qs.m), dim3(1024), 0, stream, pscore, pool, pool_count, P,
                       K, topk_out, topk_score);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

template <int DI>
static int index_full_impl(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                           const float *w_idx, int heads, int P, int K, int32_t *pool_out, int32_t *pool_count,
                           int32_t *topk_out, float *topk_score, void *ws, hipStream_t stream) {
  const IndexWs L = index_ws_layout(idx.max_len, qs.m, P, K);
  char *base = static_cast<char *>(ws);
  float *bmax = reinterpret_cast<float *>(base + L.bmax);
  uint32_t *hist = reinterpret_cast<uint32_t *>(base + L.hist);
  uint32_t *counters = reinterpret_cast<uint32_t *>(base + L.counters);
  int32_t *sure = reinterpret_cast<int32_t *>(base + L.sure);
  int32_t *tie = reinterpret_cast<int32_t *>(base + L.tie);
  float *pscore = reinterpret_cast<float *>(base + L.pscore);

  // hist and counters are adjacent: clear both with one fill kernel
  const int64_t nz = (int64_t)((L.sure - L.hist) / sizeof(uint32_t));
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, stream, hist, nz);
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
  hipLaunchKernelGGL(k_hist_threshold, dim3(qs.m), dim3(256), 0, stream, hist, L.hist_rep, idx.seq_len, qs.seq,
                     qs.pos, idx.ratio, P, counters);
  const dim3 g3((unsigned)((L.nb_max + kFilterBlocks - 1) / kFilterBlocks), qs.m);
  hipLaunchKernelGGL(k_pool_filter, g3, dim3(256), 0, stream, bmax, L.nb_max, idx.seq_len, qs.seq, qs.pos,
                     idx.ratio, P, counters, sure, tie);
  hipLaunchKernelGGL(k_pool_finalize, dim3(qs.m), dim3(1024), 0, stream, bmax, L.nb_max, counters, sure, tie,
                     idx.seq_len, qs.seq, qs.pos, idx.ratio, P, pool_out, pool_count);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_HIP;
  return rescore_and_select<DI>(idx, qs, q_idx, w_idx, heads, pool_out, pool_count, P, K, topk_out, topk_score,
                                pscore, stream);
}

int launch_index_full(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                      const float *w_idx, int heads, int P, int K, int32_t *pool_out, int32_t *pool_count,
                      int32_t *topk_out, float *topk_score, void *ws, hipStream_t stream) {
  switch (idx.dim) {
    case 64: return index_full_impl<64>(idx, qs, q_idx, w_idx, heads, P, K, pool_out, pool_count, topk_out,
                                        topk_score, ws, stream);
    case 128: return index_full_impl<128>(idx, qs, q_idx, w_idx, heads, P, K, pool_out, pool_count, topk_out,
                                          topk_score, ws, stream);
    case 256: return index_full_impl<256>(idx, qs, q_idx, w_idx, heads, P, K, pool_out, pool_count, topk_out,
                                          topk_score, ws, stream);
    default: return CSA2_ERR_UNSUPPORTED;
  }
}

int launch_rescore_select(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                          const float *w_idx, int heads, const int32_t *pool, const int32_t *pool_count, int P, int K,
                          int32_t *topk_out, float *topk_score, float *pscore, hipStream_t stream) {
  switch (idx.dim) {
    case 64: return rescore_and_select<64>(idx, qs, q_idx, w_idx, heads, pool, pool_count, P, K, topk_out,
                                           topk_score, pscore, stream);
    case 128: return rescore_and_select<128>(idx, qs, q_idx, w_idx, heads, pool, pool_count, P, K, topk_out,
                                             topk_score, pscore, stream);
    case 256: return rescore_and_select<256>(idx, qs, q_idx, w_idx, heads, pool, pool_count, P, K, topk_out,
                                             topk_score, pscore, stream);
    default: return CSA2_ERR_UNSUPPORTED;
  }
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
  return launch_rescore_select(idx, qs, q_idx, w_idx, heads, pool_in, pool_count, P, K, topk_out, topk_score,
                               pscore, stream);
}

}  // namespace csa2
