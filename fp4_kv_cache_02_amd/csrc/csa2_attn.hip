// CSA2 per-layer core attention: the selected FP4 main-KV entries
// concatenated with the layer's own FP8 window rows, one joint softmax (P5
// figure caption of the attention diagram: Selection / Top-K /
// Concatenation; P1 CSA2 section: each layer keeps its own query and window
// KV).  Keys double as values (MQA over the shared latent).  Key slots
// 0..K-1 are the Top-K list, K..K+W-1 the window rows.
//
// Two schedules compute the same thing:
//
// * Few queries (decode): k_attn_decode, one workgroup per (64 output dims,
//   query, 16 heads).  Its waves decode FP4 key rows straight into MFMA
//   operand registers, keep the logits in registers, and meet only for the
//   softmax statistics; the 64-dim V slice and P pass through LDS.  The
//   logits are recomputed by each output slice, which costs spare MFMA time
//   but makes one short kernel per layer: the grid covers the chip even for
//   four queries, with no workspace and no partial outputs to merge.
// * Many queries (prefill): k_attn, one workgroup per (query, 64 heads),
//   streams 64-key sub-chunks with an online softmax (flash style).
//
// A decoded key tile (flash) or V slice (decode) sits in LDS as row-major f16
// [key][dim]: S = Q K^T reads the tile as the MFMA B operand, and O = P V reads it through the gfx950
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
// decode schedule: key splits + merge
// ===========================================================================

constexpr int kSW = 4;                   // waves per split workgroup (one per SIMD)
constexpr int kSH = 16;                  // heads per split workgroup
constexpr int kSKeys = 128;              // key slots per split: 8 tiles of 16, two per wave
constexpr int kMaxSplits = (2048 + 1024) / kSKeys;   // Top-K <= 2048 slots, window <= 1024 rows

template <int D, bool QF32>
struct SplitLds {
  static constexpr int VT = D + 8;       // [key][dim] row stride of the decoded keys (f16)
  static constexpr int PT = kSKeys + 8;  // [head][key] row stride of P (f16)
  static constexpr int QT = D + 8;       // [head][dim] row stride of the staged queries (f16)
  _Float16 vt[kSKeys * VT];
  _Float16 p[kSH * PT];
  _Float16 q[(QF32 ? 2 : 1) * kSH * QT];  // hi parts, then lo parts (fp32 queries)
  float wmax[kSW][kSH];
  float wsum[kSW][kSH];
  float rm[kSW];
  float lsall[kMaxSplits * kSH];         // every split's lse (the merging workgroup)
  uint32_t prev;                         // arrival count seen by this workgroup
};

// Buffer loads (make_rsrc, kOutOfRange) make every load unconditional: empty,
// padded or invisible keys and heads beyond H are read at out-of-range
// offsets, which return zeros.
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

// The lane's share of one 16-key tile: lane (key row, quad) holds dims
// quad*(D/4) .. +D/4 of its key - D/8 FP4 code bytes plus D/64 E4M3 scale
// bytes of a Top-K row, or D/4 FP8 code bytes of a window row.
template <int D, bool MAIN>
struct KeyShare {
  uint32_t w[MAIN ? D / 32 : D / 16];
  uint32_t s[MAIN ? (D / 64 + 3) / 4 : 1];
};

// The f16 B operand of k-step kk (dims quad*(D/4) + 8*kk .. +7 of the lane's key).
template <int D, bool MAIN>
CSA2_DEV half8_t key_operand(const KeyShare<D, MAIN> &u, int kk) {
  if constexpr (MAIN) {
    const uint32_t sw = u.s[kk / 8] >> (8 * ((kk / 2) % 4));   // scale byte kk/2 of the lane's share
    return fp4x8_dequant_f16(u.w[kk], e4m3x2_to_f16(sw)[0]);
  } else {
    return e4m3x8_to_f16(u.w[2 * kk], u.w[2 * kk + 1]);
  }
}

// Partial outputs are kept in the MFMA accumulator layout: per (query, head
// block, split) a block of 4 waves x 64 lanes x (D/64 tiles x 4) floats, each
// lane's floats contiguous, so both the split kernel and the merge move them
// as 16-byte vectors.
template <int D>
CSA2_DEV int64_t part_offset(int64_t grp, int wave, int lane) {
  return ((grp * kSW + wave) * 64 + lane) * (D / 16);
}

// The workgroup's final output: lane (dim row, quad) of wave w holds heads
// 4*quad + j at dims w*(D/4) + 16*t + row; lse (natural log) from wave 0.
template <int D>
CSA2_DEV void store_output(const float4_t (&acc)[D / 64], const float (&ls2)[4], float *__restrict__ out,
                           float *__restrict__ lse, int H, int m, int hb, int wv, int row, int quad) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = hb * kSH + 4 * quad + j;
    if (h >= H) continue;
#pragma unroll
    for (int t = 0; t < D / 64; ++t) out[((int64_t)m * H + h) * D + wv * (D / 4) + 16 * t + row] = acc[t][j];
    if (lse && wv == 0 && row == 0) lse[(int64_t)m * H + h] = ls2[j] * 0.6931471805599453f;
  }
}

// One split: wave w owns tiles 2w and 2w+1 of the split's 128 key slots.
template <int D, bool QF32, bool MAIN>
CSA2_DEV void attn_split_body(SplitLds<D, QF32> &L, const void *__restrict__ q_any, int H,
                              const uint8_t *__restrict__ kv_codes, const uint8_t *__restrict__ kv_scales,
                              int64_t row0, int64_t vis, const int32_t *__restrict__ topk, int K, int sp0, int m,
                              int hb, const uint8_t *__restrict__ swa_codes, const float *__restrict__ swa_scale,
                              int64_t wstart, int wcount, float tau2, float *__restrict__ part_o,
                              float *__restrict__ part_lse, uint32_t *__restrict__ counters, int64_t grp, int sp,
                              int S, int HB, float *__restrict__ out, float *__restrict__ lse) {
  using Lds = SplitLds<D, QF32>;
  constexpr int NK = D / 32;             // MFMA k-steps per key
  constexpr int NDT = D / 64;            // 16-dim output tiles per wave
  constexpr int QE = QF32 ? 4 : 2;
  const int tid = threadIdx.x, l = lane_id(), wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = l & 15, quad = l >> 4;
  const rsrc_t r_codes = make_rsrc(kv_codes + row0 * (D / 2), (uint32_t)(vis * (D / 2)));
  const rsrc_t r_scales = make_rsrc(kv_scales + row0 * (D / 16), (uint32_t)(vis * (D / 16)));
  const rsrc_t r_win = make_rsrc(wcount ? swa_codes + wstart * D : nullptr, (uint32_t)(wcount * D));
  const rsrc_t r_wsc = make_rsrc(wcount ? swa_scale + wstart : nullptr, (uint32_t)(wcount * 4));
  const rsrc_t r_topk = make_rsrc(K ? topk + (int64_t)m * K : nullptr, (uint32_t)(K * 4));
  const rsrc_t r_q = make_rsrc(static_cast<const char *>(q_any) + (int64_t)m * H * D * QE, (uint32_t)(H * D * QE));

  // ---- the key slots of this lane's two tiles: index (or window scale) loads first ----
  const int slot0 = 128 * sp0 + 32 * wv + row;   // tile i: slot0 + 16 i
  int32_t jv[2];
  float rv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t so = (uint32_t)(slot0 + 16 * i) * 4u;
    if constexpr (MAIN) jv[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_topk, so, 0, 0);
    else rv[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_wsc, so, 0, 0));
  }
  // ---- the workgroup's 16 heads of queries, 8 dims per piece, loaded once ----
  constexpr int QPIECES = kSH * D / 8;
  constexpr int QPT = (QPIECES + 64 * kSW - 1) / (64 * kSW);   // pieces per thread
  uint32_t qraw[QPT][2 * QE];
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int pc = tid + 64 * kSW * u;
    const uint32_t off = (pc < QPIECES) ? (uint32_t)((hb * kSH * D + 8 * pc) * QE) : kOutOfRange;
    buffer_load_words<8 * QE>(qraw[u], r_q, off);
  }
  // ---- every key row of the lane's tiles ----
  float ks[2];
  KeyShare<D, MAIN> ku[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int slot = slot0 + 16 * i;
    if constexpr (MAIN) {
      const int32_t j = jv[i];
      const bool ok = slot < K && j >= 0 && j < vis;
      ks[i] = ok ? 1.0f : 0.0f;
      buffer_load_words<D / 8>(ku[i].w, r_codes, ok ? (uint32_t)j * (D / 2) + quad * (D / 8) : kOutOfRange);
      buffer_load_words<D / 64>(ku[i].s, r_scales, ok ? (uint32_t)j * (D / 16) + quad * (D / 64) : kOutOfRange);
    } else {
      ks[i] = (slot < wcount) ? rv[i] : 0.0f;   // rows past the window read as zeros
      buffer_load_words<D / 4>(ku[i].w, r_win, (uint32_t)slot * D + quad * (D / 4));
    }
  }
  // ---- queries to LDS as f16 [head][dim] (bf16 converts exactly in the f16
  // range; fp32 splits into hi + lo parts) ----
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int pc = tid + 64 * kSW * u;
    if (pc >= QPIECES) continue;
    const int h = pc / (D / 8), d = 8 * (pc % (D / 8));
    half8_t hi, lo;
    if constexpr (QF32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = __uint_as_float(qraw[u][i]);
        hi[i] = (_Float16)v;
        lo[i] = (_Float16)(v - (float)hi[i]);
      }
      *reinterpret_cast<half8_t *>(&L.q[(kSH + h) * Lds::QT + d]) = lo;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[2 * i] = (_Float16)__uint_as_float(qraw[u][i] << 16);
        hi[2 * i + 1] = (_Float16)__uint_as_float(qraw[u][i] & 0xFFFF0000u);
      }
    }
    *reinterpret_cast<half8_t *>(&L.q[h * Lds::QT + d]) = hi;
  }
  __syncthreads();
  // ---- S = Q K^T for the wave's two tiles: the query operands (lane (head
  // row, quad): dims quad*(D/4) + 8*kk) come from LDS all at once; the
  // decoded keys go to LDS for P V ----
  half8_t qa[NK];
  half8_t qb[QF32 ? NK : 1];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const int qo = row * Lds::QT + quad * (D / 4) + 8 * kk;
    qa[kk] = *reinterpret_cast<const half8_t *>(&L.q[qo]);
    if constexpr (QF32) qb[kk] = *reinterpret_cast<const half8_t *>(&L.q[kSH * Lds::QT + qo]);
  }
  float4_t sacc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) sacc[i] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  _Float16 *vrow = &L.vt[(32 * wv + row) * Lds::VT + quad * (D / 4)];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const half8_t b0 = key_operand<D, MAIN>(ku[0], kk);
    const half8_t b1 = key_operand<D, MAIN>(ku[1], kk);
    sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kk], b0, sacc[0], 0, 0, 0);
    sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kk], b1, sacc[1], 0, 0, 0);
    if constexpr (QF32) {
      sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qb[kk], b0, sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qb[kk], b1, sacc[1], 0, 0, 0);
    }
    *reinterpret_cast<half8_t *>(vrow + 8 * kk) = b0;
    *reinterpret_cast<half8_t *>(vrow + 16 * Lds::VT + 8 * kk) = b1;
  }
  // ---- split statistics: lane holds key (16*tile + row) of heads 4*quad + j ----
  float zz[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) zz[i][j] = (ks[i] != 0.0f) ? sacc[i][j] * tau2 * ks[i] : -INFINITY;
  // the window scale r enters P' = p * r * 2^e, with r * 2^e in [1, 2) for
  // the split's largest r (keeps small products out of the f16 subnormals)
  float rm = fmaxf(ks[0], ks[1]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) rm = fmaxf(rm, __shfl_xor(rm, o, 64));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float mx = max16_lanes(fmaxf(zz[0][j], zz[1][j]));
    if (row == 0) L.wmax[wv][4 * quad + j] = mx;
  }
  if (l == 0) L.rm[wv] = rm;
  __syncthreads();
  float mx[4];
  rm = 0.0f;
#pragma unroll
  for (int w = 0; w < kSW; ++w) rm = fmaxf(rm, L.rm[w]);
  int e = 0;
  (void)frexpf(rm, &e);
  e = (rm > 0.0f) ? 1 - e : 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSW; ++w) v = fmaxf(v, L.wmax[w][4 * quad + j]);
    mx[j] = v;
  }
  float lp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pr = (zz[i][j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(zz[i][j] - mx[j]);
      lp[j] += pr;
      L.p[(4 * quad + j) * Lds::PT + 32 * wv + 16 * i + row] = (_Float16)ldexpf(pr * ks[i], e);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float v = sum16_lanes(lp[j]);
    if (row == 0) L.wsum[wv][4 * quad + j] = v;
  }
  __syncthreads();
  // ---- O = P V for dims wv*(D/4) + 16*t over the split's 128 keys ----
  float4_t acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k0 = 0; k0 < kSKeys; k0 += 32) {
    const half8_t a = *reinterpret_cast<const half8_t *>(&L.p[row * Lds::PT + k0 + 8 * quad]);
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      const half8_t b = v_operand_tr(L.vt, Lds::VT, k0, wv * (D / 4) + 16 * t, row, quad);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[t], 0, 0, 0);
    }
  }
  // ---- normalised partial (accumulator layout) and its log2-domain lse ----
  float inv[4], ls[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = 4 * quad + j;
    float lt = 0.0f;
#pragma unroll
    for (int w = 0; w < kSW; ++w) lt += L.wsum[w][hh];
    inv[j] = (lt > 0.0f) ? ldexpf(1.0f / lt, -e) : 0.0f;
    ls[j] = (lt > 0.0f) ? mx[j] + log2f(lt) : -INFINITY;
  }
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] *= inv[j];
  if (S == 1) {
    store_output<D>(acc, ls, out, lse, H, m, hb, wv, row, quad);
    return;
  }
  // ---- key splits: this split's partial and lse go out through stores that
  // write through the caches (sc0 sc1), so every XCD reads them from memory;
  // they are complete (s_waitcnt) before the arrival is counted, and the last
  // split to arrive loads the others (again past the caches) only after it
  // has seen the count, then merges them by log-sum-exp ----
  const int64_t g0 = grp - sp;                       // split 0 of this (query, head block)
  const rsrc_t r_po = make_rsrc(part_o + part_offset<D>(g0, 0, 0), (uint32_t)(S * kSW * 64 * (D / 16) * 4));
  const rsrc_t r_pl = make_rsrc(part_lse + g0 * kSH, (uint32_t)(S * kSH * 4));
  constexpr int kThrough = 17;                       // cache policy sc0 | sc1: write through to memory
  const uint32_t slot_off = (uint32_t)(((sp * kSW + wv) * 64 + l) * (D / 16) * 4);
#pragma unroll
  for (int t = 0; t < NDT; ++t)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[t]), r_po, slot_off + 16 * t, 0,
                                           kThrough);
  if (wv == 0 && row == 0)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, (float4_t){ls[0], ls[1], ls[2], ls[3]}),
                                           r_pl, (uint32_t)((sp * kSH + 4 * quad) * 4), 0, kThrough);
  __builtin_amdgcn_s_waitcnt(0);                     // every store of this workgroup has completed
  __syncthreads();
  if (threadIdx.x == 0) L.prev = atomicInc(&counters[(int64_t)m * HB + hb], (uint32_t)S - 1u);  // wraps to 0
  __syncthreads();
  if (L.prev != (uint32_t)S - 1u) return;
  // every split's lse into LDS, then the maximum per head
  if (threadIdx.x < S * kSH)
    L.lsall[threadIdx.x] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_pl, threadIdx.x * 4u, 0, kThrough));
  __syncthreads();
  float mxs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) mxs[j] = ls[j];
  for (int s2 = 0; s2 < S; ++s2)
#pragma unroll
    for (int j = 0; j < 4; ++j) mxs[j] = fmaxf(mxs[j], L.lsall[s2 * kSH + 4 * quad + j]);
  // splits are added in split order whichever arrived last (this workgroup's
  // own partial comes from its registers), so the result is deterministic
  float wsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float4_t own[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) { own[t] = acc[t]; acc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f}; }
  for (int s2 = 0; s2 < S; ++s2) {
    float wt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float l2 = L.lsall[s2 * kSH + 4 * quad + j];
      wt[j] = (l2 == -INFINITY) ? 0.0f : exp2f(l2 - mxs[j]);
      wsum[j] += wt[j];
    }
    const uint32_t so = (uint32_t)(((s2 * kSW + wv) * 64 + l) * (D / 16) * 4);
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      float4_t v = own[t];
      if (s2 != sp)
        v = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(r_po, so + 16 * t, 0, kThrough));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[t][j] = fmaf(wt[j], v[j], acc[t][j]);
    }
  }
  float lsm[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float iw = (wsum[j] > 0.0f) ? 1.0f / wsum[j] : 0.0f;
#pragma unroll
    for (int t = 0; t < NDT; ++t) acc[t][j] *= iw;
    lsm[j] = (wsum[j] > 0.0f) ? mxs[j] + log2f(wsum[j]) : -INFINITY;
  }
  store_output<D>(acc, lsm, out, lse, H, m, hb, wv, row, quad);
}

// grid (key splits, queries, head blocks of 16), 4 waves.  Split s covers
// key slots 128s .. 128s+127 of the Top-K list (s < n_main) or window rows
// 128(s - n_main) .. of the query's window.  Wave w owns tiles 2w and 2w+1 of
// the split: it issues the Top-K index loads (or window scale loads), its
// share of the workgroup's 16 query heads (staged once in LDS as f16) and
// then every key row of its tiles at once; it computes S = Q K^T for its 32
// keys from registers (channels assigned to k-steps by quarter: lane quad q
// feeds dims q*(D/4) + 8*kk for both operands) and writes the decoded keys
// into an LDS tile for P V.  The split's softmax statistics meet in LDS; P
// (f16) goes to LDS; wave w computes O for dims w*(D/4) .. +D/4 over the
// split's 128 keys.  The normalised partial O and its log2-domain lse go to
// the workspace for k_attn_merge.
template <int D, bool QF32>
__global__ __launch_bounds__(64 * kSW) void k_attn_split(const void *__restrict__ q_any, int H,
                                                         const uint8_t *__restrict__ kv_codes,
                                                         const uint8_t *__restrict__ kv_scales,
                                                         const int64_t *__restrict__ seq_start,
                                                         const int32_t *__restrict__ seq_len, int ratio,
                                                         const int32_t *__restrict__ q_seq,
                                                         const int32_t *__restrict__ q_pos,
                                                         const int32_t *__restrict__ topk, int K, int n_main,
                                                         const uint8_t *__restrict__ swa_codes,
                                                         const float *__restrict__ swa_scale,
                                                         const int32_t *__restrict__ swa_start,
                                                         const int32_t *__restrict__ swa_count, int W, float tau2,
                                                         float *__restrict__ part_o, float *__restrict__ part_lse,
                                                         uint32_t *__restrict__ counters, float *__restrict__ out,
                                                         float *__restrict__ lse) {
  __shared__ __attribute__((aligned(16))) SplitLds<D, QF32> L;
  const int sp = blockIdx.x, m = blockIdx.y, hb = blockIdx.z;
  const int s = q_seq[m];
  const int64_t lim = ((int64_t)q_pos[m] + 1) / ratio;
  const int64_t vis = max<int64_t>(0, min<int64_t>(seq_len[s], lim));
  const int64_t row0 = seq_start[s];
  const int wcount = (W > 0) ? max(0, min(swa_count[m], W)) : 0;
  const int64_t wstart = (W > 0) ? swa_start[m] : 0;
  const int64_t grp = ((int64_t)m * gridDim.z + hb) * gridDim.x + sp;
  const int S = gridDim.x, HB = gridDim.z;
  if (sp < n_main)   // workgroup-uniform: Top-K keys or window rows
    attn_split_body<D, QF32, true>(L, q_any, H, kv_codes, kv_scales, row0, vis, topk, K, sp, m, hb, swa_codes,
                                   swa_scale, wstart, wcount, tau2, part_o, part_lse, counters, grp, sp, S, HB, out,
                                   lse);
  else
    attn_split_body<D, QF32, false>(L, q_any, H, kv_codes, kv_scales, row0, vis, topk, K, sp - n_main, m, hb,
                                    swa_codes, swa_scale, wstart, wcount, tau2, part_o, part_lse, counters, grp, sp,
                                    S, HB, out, lse);
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

// The split schedule fills the chip when there are few queries; with many
// queries (prefill) the flash kernel's one-workgroup-per-query grid is
// already large and needs no partial outputs.
static bool use_decode_kernel(int m, int heads, int dim, int64_t max_len) {
  // its buffer descriptors span one sequence's rows: byte offsets must fit
  if (max_len * (dim / 2) >= kMaxRsrcBytes) return false;
  return (int64_t)m * ((heads + kHB - 1) / kHB) < 256;
}

// Key splits of the decode schedule: 128 Top-K slots or window rows each.
static int split_main(int top_k) { return (top_k + kSKeys - 1) / kSKeys; }
static int split_count(int top_k, int window) { return split_main(top_k) + (window + kSKeys - 1) / kSKeys; }

// Decode-schedule workspace: arrival counters [query][head block] in a region
// of fixed size at offset 0 (zero before the first call, left zero by every
// call, never written by anything else: a later call of another shape finds
// its counters at the same place and still zero), normalised partial outputs
// [query][head block][split] in the accumulator layout, and their log2-domain
// lse.  The schedule's gate keeps m * ceil(heads/16) below 1024 counters.
struct AttnWs {
  size_t counters, part_o, part_lse, total;
};
static_assert(kAttnCounterBytes >= sizeof(uint32_t) * 1024, "counter region holds every decode-schedule counter");
static AttnWs attn_ws_layout(int m, int heads, int dim, int top_k, int window) {
  const size_t qh = (size_t)m * ((heads + kSH - 1) / kSH);
  const size_t groups = qh * split_count(top_k, window);
  AttnWs w{};
  size_t off = 0;
  w.counters = off; off = kAttnCounterBytes;
  w.part_o = off;   off = align256(off + sizeof(float) * groups * kSH * dim);
  w.part_lse = off; off = align256(off + sizeof(float) * groups * kSH);
  w.total = off;
  return w;
}

// Sized for the decode schedule whenever the query count may select it (a
// cache too long for it falls back to the flash kernel, which needs none).
size_t attn_ws_bytes(int m, int heads, int dim, int top_k, int window) {
  if (!use_decode_kernel(m, heads, dim, 0)) return 256;
  return attn_ws_layout(m, heads, dim, top_k, window).total;
}

template <int D, bool QF32>
static int attn_impl(const csa2_fp4_cache &kv, const csa2_queries &qs, const void *q, int heads,
                     const int32_t *topk, int K, const csa2_swa &swa, float scale, float *out, float *lse, void *ws,
                     hipStream_t stream) {
  const int W = swa.window;
  const float tau2 = scale * 1.4426950408889634f;  // log2-domain softmax: p = 2^(z - max)
  if (use_decode_kernel(qs.m, heads, D, kv.max_len)) {
    const AttnWs L = attn_ws_layout(qs.m, heads, D, K, W);
    char *base = static_cast<char *>(ws);
    uint32_t *ctr = reinterpret_cast<uint32_t *>(base + L.counters);
    float *po = reinterpret_cast<float *>(base + L.part_o);
    float *pl = reinterpret_cast<float *>(base + L.part_lse);
    const dim3 grid(split_count(K, W), qs.m, (heads + kSH - 1) / kSH);
    CSA2_TIMED_LAUNCH(kTimedAttn, (k_attn_split<D, QF32>), grid, dim3(64 * kSW), stream, q, heads, kv.codes,
                      kv.scales, kv.seq_start, kv.seq_len, kv.ratio, qs.seq, qs.pos, topk, K, split_main(K),
                      swa.codes, swa.scale, swa.start, swa.count, W, tau2, po, pl, ctr, out, lse);
  } else if (attn_prefill_supported(kv, QF32 ? CSA2_F32 : CSA2_BF16, K)) {
    return launch_attn_prefill(kv, qs, q, heads, topk, K, swa, scale, out, lse, stream);
  } else {
    const dim3 grid(qs.m, (heads + kHB - 1) / kHB);
    CSA2_TIMED_LAUNCH(kTimedAttn, (k_attn<D, QF32>), grid, dim3(256), stream, q, heads, kv.codes, kv.scales,
                      kv.seq_start, kv.seq_len, kv.ratio, qs.seq, qs.pos, topk, K, swa.codes, swa.scale, swa.start,
                      swa.count, W, tau2, out, lse);
  }
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

static int launch_attn_kernel(const csa2_fp4_cache &kv, const csa2_queries &qs, const void *q, int q_dtype,
                              int heads, const int32_t *topk, int top_k, const csa2_swa &swa, float scale, float *out,
                              float *lse, void *ws, hipStream_t stream) {
  const bool f32 = q_dtype == CSA2_F32;
#define CSA2_ATTN(D, F) attn_impl<D, F>(kv, qs, q, heads, topk, top_k, swa, scale, out, lse, ws, stream)
  switch (kv.dim) {
    case 64: return f32 ? CSA2_ATTN(64, true) : CSA2_ATTN(64, false);
    case 128: return f32 ? CSA2_ATTN(128, true) : CSA2_ATTN(128, false);
    case 256: return f32 ? CSA2_ATTN(256, true) : CSA2_ATTN(256, false);
    case 512: return f32 ? CSA2_ERR_UNSUPPORTED : CSA2_ATTN(512, false);
    default: return CSA2_ERR_UNSUPPORTED;
  }
#undef CSA2_ATTN
}

int launch_attn(const csa2_fp4_cache &kv, const csa2_queries &qs, const void *q, int q_dtype, int heads,
                const int32_t *topk, int top_k, const csa2_swa &swa, float scale, float *out, float *lse, void *ws,
                hipStream_t stream) {
  return launch_attn_kernel(kv, qs, q, q_dtype, heads, topk, top_k, swa, scale, out, lse, ws, stream);
}

}  // namespace csa2
