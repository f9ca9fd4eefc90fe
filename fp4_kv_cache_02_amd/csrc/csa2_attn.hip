// CSA2 per-layer core attention: the selected FP4 main-KV entries
// concatenated with the layer's own FP8 window rows, one joint softmax (P5
// figure caption of the attention diagram: Selection / Top-K /
// Concatenation; P1 CSA2 section: each layer keeps its own query and window
// KV).  Keys double as values (MQA over the shared latent).  Key slots
// 0..K-1 are the Top-K list, K..K+W-1 the window rows.
//
// Two schedules compute the same thing:
//
// * Few queries (decode): two kernels per batch of layers that share the
//   Top-K list and the main cache (a layer group).  k_attn_logits decodes
//   each 32-slot key chunk once and computes its logits for every layer and
//   head, storing p relative to the chunk maximum plus the chunk statistics;
//   k_attn_pv weights the chunks by those statistics and multiplies P by
//   its 32-dim slice of V.  No partial outputs are merged.
// * Many queries (prefill): k_attn, one workgroup per (query, 64 heads),
//   streams 64-key sub-chunks with an online softmax (flash style); the
//   512-channel bf16 case runs the prefill kernel of csa2_attn_prefill.hip.
//
// A decoded key tile sits in LDS as row-major f16 [key][dim]: S = Q K^T
// reads it as the MFMA B operand, and O = P V reads it through the gfx950
// transposing LDS load (ds_read_b64_tr_b16), which hands each lane four
// consecutive keys of one dimension - the B operand of the P V product -
// without a transposed copy.  Both products run on v_mfma_f32_16x16x32_f16.
//
// Exactness: FP4 entries and E4M3 window codes are f16 numbers; bf16 queries
// convert to f16 exactly inside the f16 normal range (|q| in [2^-14, 65504];
// smaller values round to f16 subnormals, larger ones are outside the
// supported input range) and fp32 queries are split into hi + lo f16 parts.
// Window rows carry an fp32 row scale r: it multiplies the logits
// (z = tau * r * q.c) and the probabilities entering P V, where P is lifted
// by a power of two 2^e (undone on the accumulator) to keep small p * r
// values out of the f16 subnormal range.  P is rounded to f16 (relative
// error <= 2^-11); everything else accumulates in fp32.
#include "csa2_internal.hpp"

#include <type_traits>

namespace csa2 {

constexpr int kKC = 64;    // keys per decoded tile (flash kernel)
constexpr int kHB = 64;    // heads per flash workgroup (4 waves x 16)

// Where key slot `slot` of query m comes from: the Top-K entry (main) or the
// window row, its scale (1 for main rows, the window row scale r, 0 when
// the slot is empty or the entry is not visible) and its row index.
struct KeySrc {
  float ks;
  int64_t row;
};
CSA2_DEV KeySrc key_source(int slot, int m, int K, int nk, const int32_t *topk, int64_t vis, int64_t row0,
                           int wcount, int64_t wstart, const float *swa_scale) {
  KeySrc r{0.0f, 0};
  if (slot < K) {
    const int32_t j = topk[(int64_t)m * K + slot];
    if (j >= 0 && j < vis) { r.ks = 1.0f; r.row = row0 + j; }
  } else if (slot < nk && slot - K < wcount) {
    r.row = wstart + (slot - K);
    r.ks = swa_scale[r.row];
  }
  return r;
}

// This wave's queries (16 heads from h0) as MFMA A operands: lane (head row,
// quad) holds dims 32*kk + 8*quad .. +7 for kk = 0 .. D/32-1.  bf16 converts
// to f16 directly; fp32 splits into hi + lo f16 parts.
template <int D, bool QF32>
CSA2_DEV void load_q_operands(const void *__restrict__ q_any, int m, int H, int h0, int row, int quad,
                              half8_t *qa, half8_t *qb) {
  constexpr int NK = D / 32;
  const int h = h0 + row;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const int64_t off = ((int64_t)m * H + h) * D + 32 * kk + 8 * quad;
    if constexpr (QF32) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (h < H) {
        a = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(q_any) + off)[0];
        b = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(q_any) + off)[1];
      }
      const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const _Float16 hi = (_Float16)v[i];
        qa[kk][i] = hi;
        qb[kk][i] = (_Float16)(v[i] - (float)hi);
      }
    } else {
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (h < H) x = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(q_any) + off);
      const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qa[kk][2 * i] = (_Float16)__uint_as_float(wd[i] << 16);
        qa[kk][2 * i + 1] = (_Float16)__uint_as_float(wd[i] & 0xFFFF0000u);
      }
    }
  }
}

// Decode kKC keys (slots sub .. sub+63; kscale / koff already in LDS) into
// the row-major f16 tile kt[key][dim] (row stride KT).  Item = 32 channels of
// one key; all loads of a thread are issued before any is decoded.  Empty
// slots decode to zeros.
template <int D>
CSA2_DEV void decode_tile_to_lds(_Float16 *kt, int KT, const float *kscale, const int64_t *koff, int sub, int K,
                                 const uint8_t *__restrict__ kv_codes, const uint8_t *__restrict__ kv_scales,
                                 const uint8_t *__restrict__ swa_codes) {
  constexpr int G32 = D / 32;
  constexpr int TOTAL = kKC * G32;
  constexpr int NIT = (TOTAL + 255) / 256;
  uint4 ca[NIT], cb[NIT];
  uint32_t sc[NIT];
#pragma unroll
  for (int u = 0; u < NIT; ++u) {
    const int item = threadIdx.x + 256 * u;
    ca[u] = make_uint4(0u, 0u, 0u, 0u);
    cb[u] = ca[u];
    sc[u] = 0u;
    if (item < TOTAL) {
      const int key = item / G32, g = item % G32;
      const int64_t r = koff[key];
      if (kscale[key] != 0.0f) {
        if (sub + key < K) {
          ca[u] = *reinterpret_cast<const uint4 *>(kv_codes + r * (D / 2) + g * 16);
          sc[u] = *reinterpret_cast<const uint16_t *>(kv_scales + r * (D / 16) + g * 2);
        } else {
          ca[u] = reinterpret_cast<const uint4 *>(swa_codes + r * D + g * 32)[0];
          cb[u] = reinterpret_cast<const uint4 *>(swa_codes + r * D + g * 32)[1];
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NIT; ++u) {
    const int item = threadIdx.x + 256 * u;
    if (item < TOTAL) {
      const int key = item / G32, g = item % G32;
      half8_t v[4];
      if (sub + key < K) {
        const half2_t s2 = e4m3x2_to_f16(sc[u]);
        v[0] = fp4x8_dequant_f16(ca[u].x, s2[0]);
        v[1] = fp4x8_dequant_f16(ca[u].y, s2[0]);
        v[2] = fp4x8_dequant_f16(ca[u].z, s2[1]);
        v[3] = fp4x8_dequant_f16(ca[u].w, s2[1]);
      } else {
        v[0] = e4m3x8_to_f16(ca[u].x, ca[u].y);
        v[1] = e4m3x8_to_f16(ca[u].z, ca[u].w);
        v[2] = e4m3x8_to_f16(cb[u].x, cb[u].y);
        v[3] = e4m3x8_to_f16(cb[u].z, cb[u].w);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<half8_t *>(&kt[key * KT + g * 32 + 8 * i]) = v[i];
    }
  }
}

// S = Q K^T for this wave's 16 heads x 64 keys (4 key tiles).  Lane result
// sacc[t][j]: key 16*t + (lane % 16), head 4*quad + j.
template <int D, bool QF32>
CSA2_DEV void qk_tile(const _Float16 *kt, int KT, const half8_t *qa, const half8_t *qb, int row, int quad,
                      float4_t sacc[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) sacc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const half8_t b = *reinterpret_cast<const half8_t *>(&kt[(16 * t + row) * KT + 32 * kk + 8 * quad]);
      sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kk], b, sacc[t], 0, 0, 0);
      if constexpr (QF32) sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qb[kk], b, sacc[t], 0, 0, 0);
    }
  }
}

// ===========================================================================
// decode schedule: logits by key chunk, then P V by output dims
// ===========================================================================
//
// Phase 1, k_attn_logits: one workgroup per (key chunk of 32 slots, query,
// layer).  It decodes the chunk's 32 keys into LDS - FP4 Top-K rows of the
// shared main cache or FP8 rows of the layer's window - and computes their
// logits for every head: p = 2^(z - m_c) stored as f16 (z the log2-domain
// logit, m_c the chunk's maximum) with the chunk statistics (m_c, sum p).
// A window row's p carries its row scale r and a power-of-two lift 2^e_c
// (r_max * 2^e_c in [1, 2)) that keeps p * r clear of the f16 subnormals.
// The layer-0 workgroups of the Top-K chunks also copy the chunk's raw FP4
// rows into a gathered array, and the window workgroups their FP8 rows, so
// phase 2 reads every key at a fixed place: no load of it waits for another.
//
// Phase 2, k_attn_pv: one workgroup per (32 output dims, query, layer).
// The chunk statistics give each head its maximum M and sum L and each chunk
// the weight w_c = 2^(m_c - M - e_c) / L; the workgroup decodes its 32-dim
// slice of every key slot (256 per block) into LDS and accumulates
// O += w_c * (P_c V_c) per 32-slot chunk: the chunk product on MFMA, the
// weighting in fp32.  No partial outputs, no merge, no atomics.

constexpr int kChunk = 32;                        // key slots per logit chunk = one P V k-step
constexpr int kLogitChunks = 2;   // key chunks per logits workgroup (its queries loaded once)
constexpr int kPvKeys = 256;                      // key slots per P V block (one per thread)
constexpr int kPvHeads = 64;                      // heads per P V workgroup
constexpr int kMaxChunks = (2048 + 1024) / kChunk;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

struct AttnBatch {
  AttnLayer l[kAttnBatch];
};

// Workgroups go to the 8 XCDs round-robin by linear id, and each XCD has its
// own L2.  The decode kernels run a grid of (M * per, layers) workgroups and
// map x to (query m, member k) = (x % M, x / M): the `per` members of a query
// - the workgroups that read the same queries or the same p values - then
// sit on the XCDs m + M k (mod 8), a single XCD when M is a multiple of 8 and
// M | 8 XCDs otherwise when M divides 8.  The layer comes from blockIdx.y.
CSA2_DEV void xcd_group(int x, int M, int &m, int &k) {
  m = x % M;
  k = x / M;
}
static unsigned xcd_grid(int per, int groups) { return (unsigned)(per * groups); }

// Buffer loads (make_rsrc, kOutOfRange) make every load unconditional: empty,
// padded or invisible keys and heads beyond H are read at out-of-range
// offsets, which return zeros.  Loads that stay unconditional also keep the
// number of loads in flight fixed, so the compiler waits only for the ones
// it needs.
template <int BYTES>
CSA2_DEV void buffer_load_words(uint32_t *dst, rsrc_t r, uint32_t off) {
  if constexpr (BYTES >= 16) {
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i) {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0);
      dst[4 * i] = x[0]; dst[4 * i + 1] = x[1]; dst[4 * i + 2] = x[2]; dst[4 * i + 3] = x[3];
    }
  } else if constexpr (BYTES == 8) {
    const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    dst[0] = x[0]; dst[1] = x[1];
  } else if constexpr (BYTES == 4) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (BYTES == 2) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
  }
}
template <int BYTES>
CSA2_DEV void buffer_store_words(const uint32_t *src, rsrc_t r, uint32_t off) {
  if constexpr (BYTES >= 16) {
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i)
      __builtin_amdgcn_raw_buffer_store_b128((u32x4_t){src[4 * i], src[4 * i + 1], src[4 * i + 2], src[4 * i + 3]}, r,
                                             off + 16 * i, 0, 0);
  } else if constexpr (BYTES == 8) {
    __builtin_amdgcn_raw_buffer_store_b64((u32x2_t){src[0], src[1]}, r, off, 0, 0);
  } else if constexpr (BYTES == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(src[0], r, off, 0, 0);
  } else if constexpr (BYTES == 2) {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)src[0], r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)src[0], r, off, 0, 0);
  }
}

// Two fp32 values with at most 8 significant bits -> their bf16 pair (low
// half first), exact: the upper halves of the fp32 bit patterns.
CSA2_DEV uint32_t bf16_pair(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Raw bytes of N consecutive dims (from dim d0, N % 8 == 0) of one FP4 row:
// N/2 code bytes and their E4M3 scale bytes.  Decoding gives exact values:
// e2m1 * e4m3 products have at most 6 significant bits, so they are f16 and
// bf16 numbers alike.
template <int D, int N>
struct Fp4Piece {
  static constexpr int SB = (N >= 16) ? N / 16 : 1;   // scale bytes loaded
  uint32_t w[N / 8];
  uint32_t s[(SB + 3) / 4];
  CSA2_DEV void load(rsrc_t codes, rsrc_t scales, bool ok, uint32_t j, int d0) {
    buffer_load_words<N / 2>(w, codes, ok ? j * (D / 2) + d0 / 2 : kOutOfRange);
    buffer_load_words<SB>(s, scales, ok ? j * (D / 16) + d0 / 16 : kOutOfRange);
  }
  CSA2_DEV void store(rsrc_t codes, rsrc_t scales, uint32_t j, int d0) const {
    buffer_store_words<N / 2>(w, codes, j * (D / 2) + d0 / 2);
    buffer_store_words<SB>(s, scales, j * (D / 16) + d0 / 16);
  }
  // scale byte of dims d0 + 8u .. +7 (d0 % 16 == 0 when N >= 16)
  CSA2_DEV uint32_t scale_byte(int u) const {
    const int g = (N >= 16) ? (8 * u) / 16 : 0;
    return s[g / 4] >> (8 * (g % 4));
  }
  // dims d0 + 8u .. +7 as f16
  CSA2_DEV half8_t get(int u) const { return fp4x8_dequant_f16(w[u], e4m3x2_to_f16(scale_byte(u))[0]); }
  // dims d0 + 8u .. +7 as bf16 (four pairs)
  CSA2_DEV u32x4_t get_bf16(int u) const {
    const float sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(scale_byte(u), 1.0f, false)[0];
    const float2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 0);
    const float2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 1);
    const float2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 2);
    const float2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 3);
    return (u32x4_t){bf16_pair(f0[0] * sc, f0[1] * sc), bf16_pair(f1[0] * sc, f1[1] * sc),
                     bf16_pair(f2[0] * sc, f2[1] * sc), bf16_pair(f3[0] * sc, f3[1] * sc)};
  }
};
// Raw bytes of N consecutive dims of one FP8 window row (E4M3 codes; the row
// scale is applied elsewhere).
template <int N>
struct Fp8Piece {
  uint32_t w[N / 4];
  CSA2_DEV void load(rsrc_t codes, bool ok, uint32_t row, int d0, int D) {
    buffer_load_words<N>(w, codes, ok ? row * (uint32_t)D + d0 : kOutOfRange);
  }
  CSA2_DEV void store(rsrc_t codes, uint32_t row, int d0, int D) const {
    buffer_store_words<N>(w, codes, row * (uint32_t)D + d0);
  }
  CSA2_DEV half8_t get(int u) const { return e4m3x8_to_f16(w[2 * u], w[2 * u + 1]); }
  CSA2_DEV u32x4_t get_bf16(int u) const {
    const float2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[2 * u], 1.0f, false);
    const float2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[2 * u], 1.0f, true);
    const float2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[2 * u + 1], 1.0f, false);
    const float2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[2 * u + 1], 1.0f, true);
    return (u32x4_t){bf16_pair(a[0], a[1]), bf16_pair(b[0], b[1]), bf16_pair(c[0], c[1]), bf16_pair(d[0], d[1])};
  }
};

// Visible main entries of query m: rows row0 .. row0 + vis - 1.
struct QueryRows {
  int64_t row0, vis;
};
CSA2_DEV QueryRows query_rows(const int64_t *seq_start, const int32_t *seq_len, int ratio, const int32_t *q_seq,
                              const int32_t *q_pos, int m) {
  const int s = q_seq[m];
  const int64_t lim = ((int64_t)q_pos[m] + 1) / ratio;
  return {seq_start[s], max<int64_t>(0, min<int64_t>(seq_len[s], lim))};
}

template <int D>
struct LogitLds {
  static constexpr int KT = D + 8;   // [key][dim] row stride of the decoded chunk (16-bit elements)
  uint16_t kt[kChunk * KT];          // bf16 keys (bf16 queries) or f16 keys (fp32 queries)
  float ks[kChunk];                  // per key: 1 (Top-K row), r (window row) or 0 (empty)
  float rmax[4];                     // per wave: largest row scale of the query's window
};

// One wave's queries of 16 heads (from h0) as raw words: lane (head row,
// quad) holds dims 32 kk + 8 quad .. +7 for every k-step kk, loaded through a
// descriptor over the query's [H][D] block (heads >= H read zeros).  bf16
// queries are the MFMA A operands as loaded (bf16 products over bf16 keys);
// fp32 queries split into hi + lo f16 parts (over f16 keys).
template <int D, bool QF32>
struct QRaw {
  static constexpr int NK = D / 32, WPK = QF32 ? 8 : 4;
  uint32_t w[NK][WPK];
  CSA2_DEV void load(rsrc_t rq, int h, int H, int quad, bool valid) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      buffer_load_words<WPK * 4>(w[kk], rq,
                                 (valid && h < H) ? (uint32_t)((h * D + 32 * kk + 8 * quad) * (QF32 ? 4 : 2))
                                                  : kOutOfRange);
  }
  CSA2_DEV bf16x8_t bf16_operand(int kk) const {
    return __builtin_bit_cast(bf16x8_t, (u32x4_t){w[kk][0], w[kk][1], w[kk][2], w[kk][3]});
  }
  CSA2_DEV void f16_operands(int kk, half8_t &hi, half8_t &lo) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = __uint_as_float(w[kk][i]);
      hi[i] = (_Float16)v;
      lo[i] = (_Float16)(v - (float)hi[i]);
    }
  }
};

// grid: (queries x (n_main_chunks + n_window_chunks) chunks, XCD-grouped
// (xcd_group), layers), 256 threads.  The arguments that the first loads
// need come first: they fit the 16 argument registers preloaded at launch.
// Thread (key = tid / 8, eighth = tid % 8) decodes dims eighth*D/8 .. of its
// key; wave w then takes head tiles w, w+4, ...: S = Q K^T over the chunk's
// two 16-key tiles (queries in registers, keys from LDS), logits, chunk
// statistics and the f16 p values.  The next tile's queries load while the
// current one computes; the first tile's load is issued with the key loads.
// ONE_TILE: at most 64 heads, one head tile per wave (its queries stay in
// registers across the workgroup's chunks, with no second tile's registers).
template <int D, bool QF32, bool ONE_TILE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ONE_TILE ? 4 : 1))) void k_attn_logits(int M, int K, int nmc, int nwc, const int32_t *__restrict__ q_seq,
                                                     const int32_t *__restrict__ q_pos,
                                                     const int64_t *__restrict__ seq_start,
                                                     const int32_t *__restrict__ seq_len,
                                                     const uint8_t *__restrict__ kv_codes,
                                                     const uint8_t *__restrict__ kv_scales, int ratio, int H,
                                                     float tau2, _Float16 *__restrict__ P, float2 *__restrict__ stats,
                                                     int32_t *__restrict__ lift, uint8_t *__restrict__ g_codes,
                                                     uint8_t *__restrict__ g_scales, uint8_t *__restrict__ g_win,
                                                     AttnBatch lb) {
  __shared__ __attribute__((aligned(16))) LogitLds<D> L;
  using Lds = LogitLds<D>;
  using QR = QRaw<D, QF32>;
  constexpr int NK = D / 32;
  constexpr int DP = D / 8;
  constexpr int QE = QF32 ? 4 : 2;
  const int nch = nmc + nwc, nkp = kChunk * nch, Kp = kChunk * nmc;
  int m, cp;   // query and chunk pair
  xcd_group(blockIdx.x, M, m, cp);
  const int li = blockIdx.y;
  const int tid = threadIdx.x, l = lane_id(), wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = l & 15, quad = l >> 4;
  const AttnLayer &ly = lb.l[li];
  const int32_t *topk = ly.topk;
  const int key = tid >> 3, d0 = (tid & 7) * DP;
  const rsrc_t r_topk = make_rsrc(K ? topk + (int64_t)m * K : nullptr, (uint32_t)(K * 4));
  // the chunk's key index (Top-K chunks; out of range otherwise)
  auto index_of = [&](int c) {
    const int slot = kChunk * c + key;
    return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_topk, (c < nmc && slot < K) ? slot * 4u : kOutOfRange, 0,
                                                         0);
  };
  // the index loads of the workgroup's Top-K chunks go out first, beside the
  // sequence lookup of query_rows (the row loads need both)
  int32_t jc[kLogitChunks];
#pragma unroll
  for (int cc = 0; cc < kLogitChunks; ++cc) jc[cc] = index_of(kLogitChunks * cp + cc);
  const QueryRows qr = query_rows(seq_start, seq_len, ratio, q_seq, q_pos, m);
  const rsrc_t rq = make_rsrc(static_cast<const char *>(ly.q) + (int64_t)m * H * D * QE, (uint32_t)(H * D * QE));
  // the wave's head tiles: wv + 4 it for it < ntw
  const int nht = (H + 15) / 16;
  const int ntw = (wv < nht) ? (nht - 1 - wv) / 4 + 1 : 0;
  auto q_load = [&](int it, QR &r) { r.load(rq, 16 * (wv + 4 * it) + row, H, quad, it < ntw); };
  QR qA;
  QR qB_store[ONE_TILE ? 1 : 2];
  QR &qB = qB_store[ONE_TILE ? 0 : 1];
  q_load(0, qA);
  // every Top-K chunk's key rows in flight at once (window chunks and slots
  // past the list or the visible entries read out of range): one round trip
  // to memory after the indices, not one per chunk
  const rsrc_t r_kc = make_rsrc(kv_codes + qr.row0 * (D / 2), (uint32_t)(qr.vis * (D / 2)));
  const rsrc_t r_ks = make_rsrc(kv_scales + qr.row0 * (D / 16), (uint32_t)(qr.vis * (D / 16)));
  Fp4Piece<D, DP> pcm[kLogitChunks];
  bool okm[kLogitChunks];
#pragma unroll
  for (int cc = 0; cc < kLogitChunks; ++cc) {
    const int c = kLogitChunks * cp + cc;
    okm[cc] = c < nmc && kChunk * c + key < K && jc[cc] >= 0 && jc[cc] < qr.vis;
    pcm[cc].load(r_kc, r_ks, okm[cc], (uint32_t)jc[cc], d0);
  }
  // the gathered copy of the Top-K rows: stores through a descriptor that
  // drops them unless this layer makes the copy (no branch around a store,
  // whose unknown count would make later waits wait for every store)
  const int64_t gr = ((int64_t)ly.list * M + m) * Kp;
  const rsrc_t r_gcw = make_rsrc(ly.gather ? g_codes + gr * (D / 2) : nullptr, ly.gather ? (uint32_t)(Kp * (D / 2)) : 0u);
  const rsrc_t r_gsw = make_rsrc(ly.gather ? g_scales + gr * (D / 16) : nullptr, ly.gather ? (uint32_t)(Kp * (D / 16)) : 0u);
  // ---- the workgroup's chunks, one after another: the queries of a wave
  // with one head tile stay in registers.  MODE 1: every chunk of the pair
  // is a Top-K chunk (one straight path, so the waits for the second
  // chunk's rows need not wait for the first chunk's stores); MODE 2: Top-K
  // or window chunks.  Returns false past the workgroup's last chunk ----
  auto run_chunk = [&](int cc, auto mode_tag) -> bool {
  constexpr int MODE = decltype(mode_tag)::value;
  const int c = kLogitChunks * cp + cc;
  if (c >= nch) return false;
  const bool main_chunk = MODE == 1 || c < nmc;
  if (!main_chunk && kChunk * (c - nmc) >= ly.window) return false;   // past this layer's window (as are later chunks)
  const int slot = kChunk * c + key;
  if (cc > 0) {
    __syncthreads();                 // the previous chunk's reads of the key tile are done
    if (!ONE_TILE && ntw > 1) q_load(0, qA);
  }

  // ---- the key row (its index issued earlier); decode the chunk's 32 keys
  // into LDS ----
  float ksv = 0.0f;
  auto put = [&](int u, const u32x4_t &v) {
    *reinterpret_cast<u32x4_t *>(&L.kt[key * Lds::KT + d0 + 8 * u]) = v;
  };
  if (main_chunk) {
    ksv = okm[cc] ? 1.0f : 0.0f;
    const Fp4Piece<D, DP> &pc = pcm[cc];
    pc.store(r_gcw, r_gsw, (uint32_t)slot, d0);   // zeros for empty slots
#pragma unroll
    for (int u = 0; u < DP / 8; ++u) put(u, QF32 ? __builtin_bit_cast(u32x4_t, pc.get(u)) : pc.get_bf16(u));
  } else {
    const int W = ly.window;
    const int wr = kChunk * (c - nmc) + key;
    const int wcount = max(0, min(ly.swa_count[m], W));
    const int64_t wstart = ly.swa_start[m];
    const bool ok = wr < wcount;
    // every row scale of the query's window (W <= 1024): the lift is shared
    // by all window chunks of the query
    const rsrc_t r_ws = make_rsrc(ly.swa_scale + wstart, (uint32_t)(wcount * 4));
    float rw = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      rw = fmaxf(rw, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_ws, (uint32_t)(tid + 256 * u) * 4u, 0, 0)));
    ksv = ok ? ly.swa_scale[wstart + wr] : 0.0f;
    Fp8Piece<DP> pc;
    pc.load(make_rsrc(ly.swa_codes + wstart * D, (uint32_t)(wcount * D)), ok, (uint32_t)wr, d0, D);
    // the gathered copy of the layer's window rows (zeros past the window)
    const int Wp = kChunk * nwc;
    pc.store(make_rsrc(g_win + ((int64_t)li * M + m) * Wp * D, (uint32_t)(Wp * D)), (uint32_t)wr, d0, D);
#pragma unroll
    for (int u = 0; u < DP / 8; ++u) put(u, QF32 ? __builtin_bit_cast(u32x4_t, pc.get(u)) : pc.get_bf16(u));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rw = fmaxf(rw, __shfl_xor(rw, o, 64));
    if (l == 0) L.rmax[wv] = rw;
  }
  if ((tid & 7) == 0) L.ks[key] = ksv;
  __syncthreads();
  // the window's lift: r_max * 2^e in [1, 2), the same for every chunk of the query's window
  int e = 0;
  if (!main_chunk) {
    const float rmax = fmaxf(fmaxf(L.rmax[0], L.rmax[1]), fmaxf(L.rmax[2], L.rmax[3]));
    (void)frexpf(rmax, &e);
    e = (rmax > 0.0f) ? 1 - e : 0;
  }
  const float ksr[2] = {L.ks[row], L.ks[16 + row]};
  if (!main_chunk && tid == 0) lift[((int64_t)li * M + m) * nch + c] = e;
  // stores through descriptors over the layer's [H] rows: heads past H fall
  // out of range and are dropped (no branch around a store)
  const int64_t lrow = ((int64_t)li * M + m) * H;
  const rsrc_t r_pw = make_rsrc(P + lrow * nkp, (uint32_t)(H * nkp * 2));
  const rsrc_t r_sw = make_rsrc(stats + lrow * nch, (uint32_t)(H * nch * 8));

  auto tile = [&](int it, const QR &cur, QR &nxt) {
    if constexpr (!ONE_TILE) q_load(it + 1, nxt);
    const int ht = wv + 4 * it;
    float4_t sacc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) sacc[i] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4_t b = *reinterpret_cast<const u32x4_t *>(&L.kt[(16 * i + row) * Lds::KT + 32 * kk + 8 * quad]);
        if constexpr (QF32) {
          half8_t qa, qb;
          cur.f16_operands(kk, qa, qb);
          const half8_t bh = __builtin_bit_cast(half8_t, b);
          sacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa, bh, sacc[i], 0, 0, 0);
          sacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qb, bh, sacc[i], 0, 0, 0);
        } else {
          sacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.bf16_operand(kk), __builtin_bit_cast(bf16x8_t, b),
                                                            sacc[i], 0, 0, 0);
        }
      }
    }
    // lane: key 16 i + row of the chunk, heads 16 ht + 4 quad + j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 16 * ht + 4 * quad + j;
      float z[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) z[i] = (ksr[i] != 0.0f) ? sacc[i][j] * tau2 * ksr[i] : -INFINITY;
      // the chunk's reference: its largest logit rounded up to an integer, so
      // that phase 2 rescales chunks by exact powers of two (p in (1/2, 1]
      // for the largest key)
      const float mc = ceilf(max16_lanes(fmaxf(z[0], z[1])));
      float p[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) p[i] = (z[i] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z[i] - mc);
      const float lc = sum16_lanes(p[0] + p[1]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)ldexpf(p[i] * ksr[i], e)), r_pw,
                                              (uint32_t)((h * nkp + kChunk * c + 16 * i + row) * 2), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64((u32x2_t){__float_as_uint(mc), __float_as_uint(lc)}, r_sw,
                                            row == 0 ? (uint32_t)((h * nch + c) * 8) : kOutOfRange, 0, 0);
    }
  };
  if constexpr (ONE_TILE) {
    // unconditional: a wave past the heads multiplies zeros and its stores
    // fall outside the descriptors (a branch here would leave the store count
    // unknown to the waits of the next chunk)
    tile(0, qA, qA);
  } else {
    for (int it = 0; it < ntw; it += 2) {
      tile(it, qA, qB);
      if (it + 1 < ntw) tile(it + 1, qB, qA);
    }
  }
  return true;
  };
  if (kLogitChunks * (cp + 1) <= nmc) {
#pragma unroll
    for (int cc = 0; cc < kLogitChunks; ++cc)
      if (!run_chunk(cc, std::integral_constant<int, 1>{})) break;
  } else {
#pragma unroll
    for (int cc = 0; cc < kLogitChunks; ++cc)
      if (!run_chunk(cc, std::integral_constant<int, 2>{})) break;
  }
}

template <int DS>
struct PvLds {
  static constexpr int VT = DS + 8;          // [key][dim] row stride of the decoded V slice (f16)
  _Float16 vt[kPvKeys * VT];
  _Float16 f[kMaxChunks * kPvHeads];         // [chunk][head]: 2^(m_c - M), the chunk's exact rescale
  float inv_l[kPvHeads];                     // per head: 1 / L
};

// grid: (queries x head groups of 64 x D / DS dim slices, XCD-grouped
// (xcd_group), layers), 256 threads.  The leading arguments fill the 16
// preloaded argument registers; every load of the first two blocks and of
// the statistics is addressed from them (the batch's largest window bounds
// them), so none waits for the layer's own arguments.
// Wave w owns heads 16 w .. 16 w + 15 of the workgroup's group; thread t
// decodes key slot t of each 256-slot block; Top-K and window slots both
// come from the gathered rows of phase 1.  A chunk's
// p values (f16) are rescaled by 2^(m_c - M) - exact, a power of two - and
// accumulated on MFMA: Top-K chunks in one accumulator, window chunks (whose
// p carry the lift 2^e) in another; O = (acc_main + 2^-e acc_win) / L.
// Blocks 0 and 1 are issued with the statistics.  NB = 3: block b + 2 is
// issued into a third register buffer before block b is multiplied (two
// waves per SIMD); NB = 2: block b + 2 goes into block b's registers once b
// is multiplied, so that three waves fit a SIMD (for grids of more than the
// 512 workgroups that are resident at once with NB = 3).
template <int D, int DS, int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NB == 2 ? 3 : 2))) void k_attn_pv(int M, int H, int nmc, int nwc, const _Float16 *__restrict__ P,
                                                 const float2 *__restrict__ stats, const int32_t *__restrict__ lift,
                                                 const uint8_t *__restrict__ g_codes,
                                                 const uint8_t *__restrict__ g_scales,
                                                 const uint8_t *__restrict__ g_win, AttnBatch lb) {
  __shared__ __attribute__((aligned(16))) PvLds<DS> L;
  using Lds = PvLds<DS>;
  constexpr int NDT = DS / 16;
  constexpr int NT = kPvKeys / kChunk;                       // k-steps per block
  constexpr int NS = D / DS;                                  // dim slices
  const int nhg = (H + kPvHeads - 1) / kPvHeads;
  int m, k;   // query and (head group, slice) member
  xcd_group(blockIdx.x, M, m, k);
  const int li = blockIdx.y, sl = k % NS, hb0 = (k / NS) * kPvHeads;
  const int tid = threadIdx.x, l = lane_id(), wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = l & 15, quad = l >> 4;
  const AttnLayer &ly = lb.l[li];
  const int W = ly.window;
  const int nchs = nmc + nwc, nkp = kChunk * nchs;          // strides of the phase-1 arrays
  const int nch = nmc + (W + kChunk - 1) / kChunk;          // this layer's chunks
  const int nslots = kChunk * nch, Kp = kChunk * nmc;
  const int hn = min(kPvHeads, H - hb0);
  const int Wp = kChunk * nwc;                               // gathered window rows of the batch
  const int64_t gr = ((int64_t)ly.list * M + m) * Kp;   // the layer's gathered Top-K rows
  const rsrc_t r_gc = make_rsrc(g_codes + gr * (D / 2), (uint32_t)(Kp * (D / 2)));
  const rsrc_t r_gs = make_rsrc(g_scales + gr * (D / 16), (uint32_t)(Kp * (D / 16)));
  const rsrc_t r_win = make_rsrc(g_win + ((int64_t)li * M + m) * Wp * D, (uint32_t)(Wp * D));
  const int64_t rows0 = ((int64_t)li * M + m) * H + hb0;    // first (layer, query, head) row of the group
  const rsrc_t r_p = make_rsrc(P + rows0 * nkp, (uint32_t)(hn * nkp * 2));
  const rsrc_t r_st = make_rsrc(stats + rows0 * nchs, (uint32_t)(hn * nchs * 8));

  struct Blk {
    Fp4Piece<D, DS> main;
    Fp8Piece<DS> win;
    half8_t pa[NT];   // P operands: lane (head row, quad) holds slots 32 t + 8 quad .. +7
  };
  const uint32_t prow = (uint32_t)((16 * wv + row) * nkp);
  // block b's rows and P operands; past the last block every offset is out
  // of range, so the loads return zeros and their number does not depend on b
  auto load_block = [&](int b, Blk &r) {
    const int slot = kPvKeys * b + tid;
    r.main.load(r_gc, r_gs, slot < Kp, (uint32_t)slot, sl * DS);
    // rows and p values past this layer's own slots (up to the batch's
    // largest window) are loaded but never multiplied
    const int wr = slot - Kp;
    r.win.load(r_win, slot >= Kp, (uint32_t)wr, sl * DS, D);
    const bool okp = kPvKeys * b < nkp;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      r.pa[t] = __builtin_bit_cast(
          half8_t, __builtin_amdgcn_raw_buffer_load_b128(
                       r_p, okp ? (prow + kPvKeys * b + kChunk * t + 8 * quad) * 2u : kOutOfRange, 0, 0));
  };

  // ---- issue: this thread's chunk statistics (head tid / 4; chunk groups
  // 4 g .. 4 g + 3 for g = tid % 4 + 4 k, two groups at a time), the
  // window's lift, blocks 0, 1 ----
  const int nblk = (nslots + kPvKeys - 1) / kPvKeys;
  const int hh = tid >> 2, q4 = tid & 3;
  const int kmax = (nchs + 15) / 16;                          // statistics groups per thread in use
  float2 sv[2][4];
  auto load_stats = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int g = q4 + 4 * (k0 + u);
      const uint32_t off = (k0 + u < kmax && hh < hn && 4 * g < nchs) ? (uint32_t)(hh * nchs + 4 * g) * 8u : kOutOfRange;
      const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r_st, off, 0, 0);
      const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(r_st, off == kOutOfRange ? off : off + 16u, 0, 0);
      sv[u][0] = make_float2(__uint_as_float(a[0]), __uint_as_float(a[1]));
      sv[u][1] = make_float2(__uint_as_float(a[2]), __uint_as_float(a[3]));
      sv[u][2] = make_float2(__uint_as_float(b[0]), __uint_as_float(b[1]));
      sv[u][3] = make_float2(__uint_as_float(b[2]), __uint_as_float(b[3]));
    }
  };
  load_stats(0);
  const int32_t ew_raw = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      make_rsrc(lift + ((int64_t)li * M + m) * nchs, (uint32_t)(nchs * 4)), nmc * 4u, 0, 0);
  Blk ba, bb, bc;   // bc: the third buffer of the NB = 3 ring
  load_block(0, ba);
  load_block(1, bb);
  // ---- per head: the largest reference M, the sum L, and each chunk's
  // rescale 2^(m_c - M) (0 below the f16 range).  The chunk maxima m_c are
  // integers; the thread keeps a running maximum and a sum rescaled by exact
  // powers of two, and parks its m_c in the V tile (free until the first
  // block is decoded) for the rescales ----
  float *const mpark = reinterpret_cast<float *>(L.vt);       // [chunk][head]
  static_assert(kMaxChunks * kPvHeads * 4 <= (int)sizeof(L.vt), "chunk maxima fit the V tile");
  float lse2;
  {
    float mx = -INFINITY, sum = 0.0f;
    auto fold = [&](int k0) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cc = 4 * (q4 + 4 * (k0 + u)) + i;
          const bool ok = hh < hn && cc < nch && sv[u][i].x != -INFINITY;
          if (cc < nch) mpark[cc * kPvHeads + hh] = ok ? sv[u][i].x : -INFINITY;
          if (ok) {
            const float mc = sv[u][i].x;
            if (mc > mx) {
              sum = (mx == -INFINITY) ? 0.0f : ldexpf(sum, (int)(mx - mc));
              mx = mc;
            }
            sum += ldexpf(sv[u][i].y, (int)(mc - mx));
          }
        }
    };
    fold(0);
    for (int k0 = 2; k0 < kmax; k0 += 2) {   // more than 32 chunks per layer
      load_stats(k0);
      fold(k0);
    }
    const float mx_own = mx;
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    sum = (mx_own == -INFINITY) ? 0.0f : ldexpf(sum, (int)(mx_own - mx));
    sum += __shfl_xor(sum, 1, 64);
    sum += __shfl_xor(sum, 2, 64);
    for (int k = 0; k < kmax; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cc = 4 * (q4 + 4 * k) + i;
        if (cc >= nch) continue;
        const float mc = mpark[cc * kPvHeads + hh];
        const int sh = (mc != -INFINITY) ? (int)(mc - mx) : -1000;   // an integer <= 0
        L.f[cc * kPvHeads + hh] = (sh >= -24) ? (_Float16)ldexpf(1.0f, sh) : (_Float16)0.0f;
      }
    if (q4 == 0) L.inv_l[hh] = (sum > 0.0f) ? 1.0f / sum : 0.0f;
    lse2 = (sum > 0.0f) ? mx + log2f(sum) : -INFINITY;
  }

  const int ew = (nch > nmc) ? ew_raw : 0;   // the window's lift (no window chunk: none)
  float4_t am[NDT], aw[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    am[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
    aw[t] = am[t];
  }
  const bool active = 16 * wv < hn;
  // block b: decode `cur` and multiply
  auto compute = [&](int b, const Blk &cur) {
    __syncthreads();      // the rescales (first block) or the previous block's V reads are done
    {
      // a wave's 64 slots are all Top-K or all window unless the list's end
      // falls inside them: the branch usually runs one decoder per wave
      _Float16 *vrow = &L.vt[tid * Lds::VT];
      if (kPvKeys * b + tid < Kp) {
#pragma unroll
        for (int u = 0; u < DS / 8; ++u) *reinterpret_cast<half8_t *>(vrow + 8 * u) = cur.main.get(u);
      } else {
#pragma unroll
        for (int u = 0; u < DS / 8; ++u) *reinterpret_cast<half8_t *>(vrow + 8 * u) = cur.win.get(u);
      }
    }
    __syncthreads();
    if (active) {
      const int nt = min(kPvKeys, nslots - kPvKeys * b) / kChunk;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= nt) break;
        const int cc = (kPvKeys * b) / kChunk + t;
        const _Float16 fc = L.f[cc * kPvHeads + 16 * wv + row];   // exact power of two (or 0)
        const half8_t a = cur.pa[t] * (half8_t){fc, fc, fc, fc, fc, fc, fc, fc};
        if (cc < nmc) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            am[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, v_operand_tr(L.vt, Lds::VT, kChunk * t, 16 * dt, row, quad),
                                                            am[dt], 0, 0, 0);
        } else {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            aw[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, v_operand_tr(L.vt, Lds::VT, kChunk * t, 16 * dt, row, quad),
                                                            aw[dt], 0, 0, 0);
        }
      }
    }
  };
  if constexpr (NB == 3) {
    // three buffers: block b + 2 is issued before block b is multiplied
    auto step = [&](int b, const Blk &cur, Blk &fut) {
      load_block(b + 2, fut);
      if (b < nblk) compute(b, cur);
    };
    for (int b = 0; b < nblk; b += 3) {
      step(b, ba, bc);
      step(b + 1, bb, ba);
      step(b + 2, bc, bb);
    }
  } else {
    // two buffers: block b + 2 goes into block b's registers once b is
    // multiplied (block b + 1's loads stay in flight meanwhile)
    auto step = [&](int b, Blk &cur) {
      if (b >= nblk) return;
      compute(b, cur);
      load_block(b + 2, cur);
    };
    for (int b = 0; b < nblk; b += 2) {
      step(b, ba);
      step(b + 1, bb);
    }
  }
  // ---- output: lane (dim row, quad) holds heads 16 w + 4 quad + j ----
  if (active) {
    const float4_t il = *reinterpret_cast<const float4_t *>(&L.inv_l[16 * wv + 4 * quad]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = hb0 + 16 * wv + 4 * quad + j;
      if (h >= H) continue;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        ly.out[((int64_t)m * H + h) * D + sl * DS + 16 * dt + row] = (am[dt][j] + ldexpf(aw[dt][j], -ew)) * il[j];
    }
  }
  if (sl == 0 && q4 == 0 && hh < hn && ly.lse) ly.lse[(int64_t)m * H + hb0 + hh] = lse2 * 0.6931471805599453f;
}

// ===========================================================================
// prefill schedule: one workgroup per (query, 64 heads), online softmax
// ===========================================================================

template <int D, bool QF32>
struct AttnLds {
  static constexpr int KT = D + 8;     // [key][dim] row stride (f16)
  static constexpr int PT = kKC + 8;   // [head][key] row stride of a wave's P tile
  _Float16 kt[kKC * KT];
  _Float16 p[4][16 * PT];
  float kscale[kKC];     // per key: r (window row scale) or 1; 0 = masked
  int64_t koff[kKC];     // per key: row of its FP4 codes (main) or FP8 row (window)
  float rmax;
};

template <int D, bool QF32>
__global__ __launch_bounds__(256) void k_attn(const void *__restrict__ q_any, int H,
                                              const uint8_t *__restrict__ kv_codes,
                                              const uint8_t *__restrict__ kv_scales,
                                              const int64_t *__restrict__ seq_start,
                                              const int32_t *__restrict__ seq_len, int ratio,
                                              const int32_t *__restrict__ q_seq, const int32_t *__restrict__ q_pos,
                                              const int32_t *__restrict__ topk, int K,
                                              const uint8_t *__restrict__ swa_codes,
                                              const float *__restrict__ swa_scale,
                                              const int32_t *__restrict__ swa_start,
                                              const int32_t *__restrict__ swa_count, int W, float tau2,
                                              float *__restrict__ out, float *__restrict__ lse) {
  __shared__ AttnLds<D, QF32> L;
  const int m = blockIdx.x, hb = blockIdx.y;
  const int tid = threadIdx.x, l = lane_id(), wv = tid >> 6;
  const int row = l & 15, quad = l >> 4;
  const int nk = K + W;
  const int h0 = hb * kHB + 16 * wv;        // first head of this wave
  const bool wave_active = h0 < H;

  const int s = q_seq[m];
  const int64_t lim = ((int64_t)q_pos[m] + 1) / ratio;
  const int64_t vis = max<int64_t>(0, min<int64_t>(seq_len[s], lim));
  const int64_t row0 = seq_start[s];
  // with no window the window arrays may be null
  const int wcount = (W > 0) ? min(swa_count[m], W) : 0;
  const int64_t wstart = (W > 0) ? swa_start[m] : 0;

  constexpr int NK = D / 32;
  half8_t qa[NK];
  half8_t qb[QF32 ? NK : 1];
  load_q_operands<D, QF32>(q_any, m, H, h0, row, quad, qa, qb);

  float m_run[4], l_run[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.0f; }
  constexpr int NCT = D / 16;  // 16-dim output tiles per wave
  float4_t o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o_acc[ct] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  int e_cur = 0;  // accumulator exponent: true O = o_acc * 2^-e_cur
  _Float16 *pw = L.p[wv];

  for (int sub = 0; sub < nk; sub += kKC) {
    __syncthreads();  // previous sub-chunk's LDS reads are done
    // ---- per-key validity, scale and source row (wave 0) ----
    if (tid < kKC) {
      const KeySrc src = key_source(sub + tid, m, K, nk, topk, vis, row0, wcount, wstart, swa_scale);
      L.kscale[tid] = src.ks;
      L.koff[tid] = src.row;
      float rm = src.ks;
      for (int o = 32; o > 0; o >>= 1) rm = fmaxf(rm, __shfl_xor(rm, o, 64));
      if (tid == 0) L.rmax = rm;
    }
    __syncthreads();
    decode_tile_to_lds<D>(L.kt, L.KT, L.kscale, L.koff, sub, K, kv_codes, kv_scales, swa_codes);
    __syncthreads();
    if (!wave_active) continue;

    float4_t sacc[4];
    qk_tile<D, QF32>(L.kt, L.KT, qa, qb, row, quad, sacc);
    // lane: key 16*t + row of each tile, heads 4*quad + j
    float z[4][4], ksc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) ksc[t] = L.kscale[16 * t + row];
    float cm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        z[t][j] = (ksc[t] != 0.0f) ? sacc[t][j] * tau2 * ksc[t] : -INFINITY;
        mx = fmaxf(mx, z[t][j]);
      }
      cm[j] = max16_lanes(mx);
    }
    int e_new = 0;
    (void)frexpf(L.rmax, &e_new);
    e_new = (L.rmax > 0.0f) ? 1 - e_new : 0;  // rmax * 2^e_new in [1, 2)
    float alpha[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float mnew = fmaxf(m_run[j], cm[j]);
      float psum = 0.0f;
      if (mnew == -INFINITY) {
        alpha[j] = 1.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) pw[(4 * quad + j) * L.PT + 16 * t + row] = (_Float16)0.0f;
      } else {
        alpha[j] = (m_run[j] == -INFINITY) ? 0.0f : exp2f(m_run[j] - mnew);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float p = (z[t][j] == -INFINITY) ? 0.0f : exp2f(z[t][j] - mnew);
          psum += p;
          pw[(4 * quad + j) * L.PT + 16 * t + row] = (_Float16)ldexpf(p * ksc[t], e_new);
        }
        m_run[j] = mnew;
      }
      l_run[j] = alpha[j] * l_run[j] + sum16_lanes(psum);
      alpha[j] = ldexpf(alpha[j], e_new - e_cur);
    }
    e_cur = e_new;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- O = alpha O + P V for 16 heads x D dims ----
    const half8_t pa0 = *reinterpret_cast<const half8_t *>(&pw[row * L.PT + 8 * quad]);
    const half8_t pa1 = *reinterpret_cast<const half8_t *>(&pw[row * L.PT + 32 + 8 * quad]);
    const bool first = sub == 0;   // accumulator still zero: no rescale
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (!first) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o_acc[ct][j] *= alpha[j];
      }
      o_acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa0, v_operand_tr(L.kt, L.KT, 0, 16 * ct, row, quad),
                                                         o_acc[ct], 0, 0, 0);
      o_acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa1, v_operand_tr(L.kt, L.KT, 32, 16 * ct, row, quad),
                                                         o_acc[ct], 0, 0, 0);
    }
  }

  if (!wave_active) return;
  // ---- write o (normalised) and lse ----
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = h0 + 4 * quad + j;
    if (h >= H) continue;
    const float inv = (l_run[j] > 0.0f) ? ldexpf(1.0f / l_run[j], -e_cur) : 0.0f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) out[((int64_t)m * H + h) * D + 16 * ct + row] = o_acc[ct][j] * inv;
    if (row == 0 && lse)
      lse[(int64_t)m * H + h] = (l_run[j] > 0.0f) ? (m_run[j] + log2f(l_run[j])) * 0.6931471805599453f : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// The decode schedule fills the chip when there are few queries; with many
// queries (prefill) the one-workgroup-per-query kernels already have a large
// grid and need no intermediates.
static bool use_decode_kernel(int m, int heads, int dim, int64_t max_len) {
  // its buffer descriptors span one sequence's rows: byte offsets must fit
  if (max_len * (dim / 2) >= kMaxRsrcBytes) return false;
  return (int64_t)m * ((heads + kHB - 1) / kHB) < 256;
}

// Decode-schedule workspace for a batch of `nl` layers over `nlists` Top-K
// lists: p values (f16) [layer][query][head][slot], chunk statistics (m_c,
// sum p) [layer][query][head][chunk], window-chunk lifts [layer][query]
// [chunk], the gathered Top-K rows [list][query][slot] (FP4 codes and scale
// bytes) and the gathered window rows [layer][query][row] (FP8 codes).
// Slots: the Top-K list padded to whole chunks, then the largest window of
// the batch.
struct DecodeWs {
  int nmc, nwc;
  size_t p, stats, lift, gcodes, gscales, gwin, total;
};
static DecodeWs decode_ws_layout(int m, int heads, int dim, int top_k, int max_window, int nl, int nlists) {
  DecodeWs w{};
  w.nmc = (top_k + kChunk - 1) / kChunk;
  w.nwc = (max_window + kChunk - 1) / kChunk;
  const size_t nch = (size_t)(w.nmc + w.nwc), rows = (size_t)nl * m * heads, kp = (size_t)kChunk * w.nmc;
  size_t off = 0;
  w.p = off;       off = align256(off + sizeof(_Float16) * rows * nch * kChunk);
  w.stats = off;   off = align256(off + sizeof(float2) * rows * nch);
  w.lift = off;    off = align256(off + sizeof(int32_t) * (size_t)nl * m * nch);
  w.gcodes = off;  off = align256(off + (size_t)nlists * m * kp * (dim / 2));
  w.gscales = off; off = align256(off + (size_t)nlists * m * kp * (dim / 16));
  w.gwin = off;    off = align256(off + (size_t)nl * m * (kChunk * w.nwc) * dim);
  w.total = off;
  return w;
}

size_t attn_ws_bytes(int m, int heads, int dim, int top_k, int max_window, int n_layers, int n_lists) {
  if (m < 1 || n_layers < 1 || !use_decode_kernel(m, heads, dim, 0)) return 256;
  const int nl = std::min(n_layers, kAttnBatch);
  return decode_ws_layout(m, heads, dim, top_k, max_window, nl, std::max(1, std::min(n_lists, nl))).total;
}

template <int D, bool QF32>
static int attn_layers_impl(const csa2_fp4_cache &kv, const csa2_queries &qs, int heads, int K,
                            const AttnLayer *layers, int n, float scale, void *ws, hipStream_t stream) {
  const float tau2 = scale * 1.4426950408889634f;  // log2-domain softmax: p = 2^(z - max)
  if (use_decode_kernel(qs.m, heads, D, kv.max_len)) {
    constexpr int DS = D < 64 ? D : 64;
    for (int b0 = 0; b0 < n; b0 += kAttnBatch) {
      const int nl = std::min(kAttnBatch, n - b0);
      AttnBatch lb{};
      int wmax = 0, nlists = 0;
      for (int i = 0; i < nl; ++i) {
        lb.l[i] = layers[b0 + i];
        wmax = std::max(wmax, layers[b0 + i].window);
        // one gathered copy per distinct list, written by its first layer
        int li = 0;
        while (li < i && lb.l[li].topk != lb.l[i].topk) ++li;
        lb.l[i].list = (li < i) ? lb.l[li].list : nlists++;
        lb.l[i].gather = li == i;
      }
      const DecodeWs L = decode_ws_layout(qs.m, heads, D, K, wmax, nl, nlists);
      char *base = static_cast<char *>(ws);
      _Float16 *P = reinterpret_cast<_Float16 *>(base + L.p);
      float2 *st = reinterpret_cast<float2 *>(base + L.stats);
      int32_t *lf = reinterpret_cast<int32_t *>(base + L.lift);
      uint8_t *gc = reinterpret_cast<uint8_t *>(base + L.gcodes);
      uint8_t *gs = reinterpret_cast<uint8_t *>(base + L.gscales);
      uint8_t *gw = reinterpret_cast<uint8_t *>(base + L.gwin);
      const dim3 g1(xcd_grid((L.nmc + L.nwc + kLogitChunks - 1) / kLogitChunks, qs.m), (unsigned)nl);
      if (heads <= 64)
        CSA2_TIMED_LAUNCH(kTimedAttn, (k_attn_logits<D, QF32, true>), g1, dim3(256), stream, qs.m, K, L.nmc, L.nwc,
                          qs.seq, qs.pos, kv.seq_start, kv.seq_len, kv.codes, kv.scales, kv.ratio, heads, tau2, P, st,
                          lf, gc, gs, gw, lb);
      else
        CSA2_TIMED_LAUNCH(kTimedAttn, (k_attn_logits<D, QF32, false>), g1, dim3(256), stream, qs.m, K, L.nmc, L.nwc,
                          qs.seq, qs.pos, kv.seq_start, kv.seq_len, kv.codes, kv.scales, kv.ratio, heads, tau2, P, st,
                          lf, gc, gs, gw, lb);
      const int nhg = (heads + kPvHeads - 1) / kPvHeads;
      const dim3 g2(xcd_grid((D / DS) * nhg, qs.m), (unsigned)nl);
      // up to 512 workgroups are resident at once with the three-buffer ring
      // (two waves per SIMD); beyond that the two-buffer ring lets three
      // fit a SIMD, so more of them run in the first round
      if ((int64_t)g2.x * g2.y <= 512)
        CSA2_TIMED_LAUNCH(kTimedAttn, (k_attn_pv<D, DS, 3>), g2, dim3(256), stream, qs.m, heads, L.nmc, L.nwc, P, st,
                          lf, gc, gs, gw, lb);
      else
        CSA2_TIMED_LAUNCH(kTimedAttn, (k_attn_pv<D, DS, 2>), g2, dim3(256), stream, qs.m, heads, L.nmc, L.nwc, P, st,
                          lf, gc, gs, gw, lb);
    }
    return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
  }
  for (int i = 0; i < n; ++i) {
    const AttnLayer &ly = layers[i];
    const csa2_swa swa{ly.swa_codes, ly.swa_scale, ly.swa_start, ly.swa_count, D, ly.window};
    if (attn_prefill_supported(kv, QF32 ? CSA2_F32 : CSA2_BF16, K)) {
      const int st = launch_attn_prefill(kv, qs, ly.q, heads, ly.topk, K, swa, scale, ly.out, ly.lse, stream);
      if (st != CSA2_OK) return st;
    } else {
      const dim3 grid(qs.m, (heads + kHB - 1) / kHB);
      CSA2_TIMED_LAUNCH(kTimedAttn, (k_attn<D, QF32>), grid, dim3(256), stream, ly.q, heads, kv.codes, kv.scales,
                        kv.seq_start, kv.seq_len, kv.ratio, qs.seq, qs.pos, ly.topk, K, ly.swa_codes, ly.swa_scale,
                        ly.swa_start, ly.swa_count, ly.window, tau2, ly.out, ly.lse);
    }
  }
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

int launch_attn_layers(const csa2_fp4_cache &kv, const csa2_queries &qs, int q_dtype, int heads, int top_k,
                       const AttnLayer *layers, int n_layers, float scale, void *ws, hipStream_t stream) {
  const bool f32 = q_dtype == CSA2_F32;
#define CSA2_ATTN(D, F) attn_layers_impl<D, F>(kv, qs, heads, top_k, layers, n_layers, scale, ws, stream)
  switch (kv.dim) {
    case 64: return f32 ? CSA2_ATTN(64, true) : CSA2_ATTN(64, false);
    case 128: return f32 ? CSA2_ATTN(128, true) : CSA2_ATTN(128, false);
    case 256: return f32 ? CSA2_ATTN(256, true) : CSA2_ATTN(256, false);
    case 512: return f32 ? CSA2_ERR_UNSUPPORTED : CSA2_ATTN(512, false);
    default: return CSA2_ERR_UNSUPPORTED;
  }
#undef CSA2_ATTN
}

}  // namespace csa2
