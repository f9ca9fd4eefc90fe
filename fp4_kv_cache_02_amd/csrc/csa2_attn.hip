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
// decode schedule: one fused kernel per layer
// ===========================================================================

constexpr int kDW = 8;                   // waves per decode workgroup
constexpr int kDH = 16;                  // heads per decode workgroup
constexpr int kDD = 64;                  // output dims per decode workgroup
constexpr int kDMainT = 4;               // Top-K tiles of 16 slots per wave and chunk
constexpr int kDTm = kDW * kDMainT;      // Top-K tiles per chunk (512 slots)
constexpr int kDTw = kDW;                // window tiles per chunk, one per wave (128 rows)
constexpr int kDSlots = 16 * (kDTm + kDTw);  // key slots per chunk (640)

struct DecLds {
  static constexpr int VT = kDD + 8;       // [key][dim] row stride of the V slice (f16)
  static constexpr int PT = kDSlots + 8;   // [head][key] row stride of P (f16)
  _Float16 vt[kDSlots * VT];
  _Float16 p[kDH * PT];
  float wmax[kDW][kDH];
  float wsum[kDW][kDH];
  float wr[kDW];
  float4_t ored[4][64];
};

// A lane's share of one key tile for S = Q K^T: the lane (key row, quad)
// holds dims quad*(D/4) .. +D/4 of its key.  Main rows: D/8 FP4 code bytes
// plus D/64 E4M3 scale bytes; window rows: D/4 FP8 code bytes.
template <int D>
struct MainUnit {
  uint32_t w[D / 32];
  uint32_t s[(D / 64 + 3) / 4];
};
template <int D>
struct WinUnit {
  uint32_t w[D / 16];
};

// Buffer loads (make_rsrc, kOutOfRange) make every load unconditional: the
// decode kernel reads empty, padded or invisible keys and heads beyond H at
// out-of-range offsets, which return zeros.
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

// S += Q K^T over every k-step of a main tile.  The B operand of step kk is
// dims quad*(D/4) + 8*kk .. +7 of the lane's key.  Called under wave-uniform
// conditions only: an MFMA reads the operands of every lane whatever the
// exec mask.
template <int D, bool QF32>
CSA2_DEV void score_main(const MainUnit<D> &u, const half8_t *qa, const half8_t *qb, float4_t &sa) {
  half2_t sc[(D / 64 + 1) / 2];
#pragma unroll
  for (int g = 0; g < (D / 64 + 1) / 2; ++g) sc[g] = e4m3x2_to_f16(u.s[g / 2] >> (16 * (g % 2)));
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const half8_t b = fp4x8_dequant_f16(u.w[kk], sc[kk / 4][(kk / 2) % 2]);
    sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kk], b, sa, 0, 0, 0);
    if constexpr (QF32) sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(qb[kk], b, sa, 0, 0, 0);
  }
}
template <int D, bool QF32>
CSA2_DEV void score_win(const WinUnit<D> &u, const half8_t *qa, const half8_t *qb, float4_t &sa) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const half8_t b = e4m3x8_to_f16(u.w[2 * kk], u.w[2 * kk + 1]);
    sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kk], b, sa, 0, 0, 0);
    if constexpr (QF32) sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(qb[kk], b, sa, 0, 0, 0);
  }
}

// The V slice of one key tile: lane (key n, part p) holds dims d0 + 16p ..
// +15 of key n (four parts cover the 64-dim slice), loaded apart from the
// scoring units (a cached re-read of 8 code bytes + 1 scale byte, or 16 FP8
// bytes) and stored as f16 into row n of the tile's LDS rows.
struct VPiece {
  uint32_t w[4];
};
CSA2_DEV void load_vpiece_main(VPiece &v, rsrc_t codes, rsrc_t scales, uint32_t code_off, uint32_t scale_off) {
  const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(codes, code_off, 0, 0);
  v.w[0] = x[0];
  v.w[1] = x[1];
  v.w[2] = __builtin_amdgcn_raw_buffer_load_b8(scales, scale_off, 0, 0);
  v.w[3] = 0u;
}
CSA2_DEV void load_vpiece_win(VPiece &v, rsrc_t win, uint32_t code_off) {
  const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(win, code_off, 0, 0);
  v.w[0] = x[0]; v.w[1] = x[1]; v.w[2] = x[2]; v.w[3] = x[3];
}
CSA2_DEV void store_vpiece(const VPiece &v, bool main, _Float16 *dst) {
  half8_t a, b;
  if (main) {
    const _Float16 sc = e4m3x2_to_f16(v.w[2])[0];
    a = fp4x8_dequant_f16(v.w[0], sc);
    b = fp4x8_dequant_f16(v.w[1], sc);
  } else {
    a = e4m3x8_to_f16(v.w[0], v.w[1]);
    b = e4m3x8_to_f16(v.w[2], v.w[3]);
  }
  *reinterpret_cast<half8_t *>(dst) = a;
  *reinterpret_cast<half8_t *>(dst + 8) = b;
}

// grid (D / 64 output slices, queries, head blocks of 16), 8 waves.
//
// A workgroup computes the logits of its 16 heads against every key of the
// query (replicated across the output slices: spare MFMA time buys a kernel
// with no partial outputs to merge) and P V for its 64 output dims.  Keys go
// in chunks of 32 Top-K tiles + 8 window tiles (one chunk for Top-512 + 128
// window rows): wave w owns Top-K tiles w, w+8, w+16, w+24 and window tile w
// of the chunk.  Every load of a chunk is issued before any key is scored, so
// a wave waits for memory once per chunk: the Top-K indices and window
// scales first, then (while they are in flight) the query operands straight
// into registers, then all key rows and V pieces.  Channels are assigned to
// MFMA k-steps by quarter (lane quad q feeds dims q*(D/4) + 8*kk .. +7 for
// both query and key), so a lane streams contiguous bytes of its key.  The
// chunk's softmax statistics meet in LDS; P (f16) and the 64-dim V slice
// pass through LDS; wave w multiplies P by V for dims 16*(w%4) .. +15 over
// every second 32-key step, the two halves being added at the end.  Chunks
// combine online.
template <int D, bool QF32>
__global__ __launch_bounds__(64 * kDW) void k_attn_decode(const void *__restrict__ q_any, int H,
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
  __shared__ DecLds L;
  constexpr int NK = D / 32;             // MFMA k-steps per key
  constexpr int DD = D < kDD ? D : kDD;  // dims of this workgroup's output slice
  constexpr int NT = kDMainT + 1;        // tiles per wave per chunk (Top-K tiles, then the window tile)
  const int m = blockIdx.y, hb = blockIdx.z;
  const int d0 = blockIdx.x * kDD;
  // the wave index as a scalar: per-tile conditions (and the descriptor choice)
  // are then wave-uniform branches, not exec-masked ones
  const int tid = threadIdx.x, l = lane_id(), wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = l & 15, quad = l >> 4;

  const int s = q_seq[m];
  const int64_t lim = ((int64_t)q_pos[m] + 1) / ratio;
  const int64_t vis = max<int64_t>(0, min<int64_t>(seq_len[s], lim));
  const int64_t row0 = seq_start[s];
  // with no window the window arrays may be null (their descriptors are empty)
  const int wcount = (W > 0) ? max(0, min(swa_count[m], W)) : 0;
  const int64_t wstart = (W > 0) ? swa_start[m] : 0;
  const int TM = (K + 15) / 16;        // Top-K tiles
  const int TW = (wcount + 15) / 16;   // window tiles of this query
  const int nchunk = max((TM + kDTm - 1) / kDTm, (TW + kDTw - 1) / kDTw);
  // descriptors: this query's visible rows, window rows, Top-K list and queries
  const rsrc_t r_codes = make_rsrc(kv_codes + row0 * (D / 2), (uint32_t)(vis * (D / 2)));
  const rsrc_t r_scales = make_rsrc(kv_scales + row0 * (D / 16), (uint32_t)(vis * (D / 16)));
  const rsrc_t r_win = make_rsrc(wcount ? swa_codes + wstart * D : nullptr, (uint32_t)(wcount * D));
  const rsrc_t r_wsc = make_rsrc(wcount ? swa_scale + wstart : nullptr, (uint32_t)(wcount * 4));
  const rsrc_t r_topk = make_rsrc(K ? topk + (int64_t)m * K : nullptr, (uint32_t)(K * 4));
  constexpr int QE = QF32 ? 4 : 2;  // query element bytes
  const rsrc_t r_q = make_rsrc(static_cast<const char *>(q_any) + (int64_t)m * H * D * QE, (uint32_t)(H * D * QE));

  half8_t qa[NK];
  half8_t qb[QF32 ? NK : 1];
  float m_run[4], l_part[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { m_run[j] = -INFINITY; l_part[j] = 0.0f; }
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  int e_cur = 0;                          // accumulator exponent: true O = acc * 2^-e_cur
  const int dt = wv & 3, khalf = wv >> 2;  // P V: dims 16*dt .., k-steps khalf, khalf + 2, ...

  for (int c = 0; c < nchunk; ++c) {
    const int nmc = max(0, min(kDTm, TM - kDTm * c));   // Top-K tiles of the chunk
    const int nwc = max(0, min(kDTw, TW - kDTw * c));   // window tiles of the chunk
    const int nme = (nmc + 1) & ~1, nwe = (nwc + 1) & ~1;  // rounded to whole 32-key steps
    if (c > 0) __syncthreads();           // the previous chunk's LDS reads are done
    // ---- sources of this wave's tiles: the index and window-scale loads go
    // first, the first chunk's query operands behind them ----
    int32_t jv[kDMainT];
#pragma unroll
    for (int i = 0; i < kDMainT; ++i) {
      const int slot = 16 * (kDTm * c + wv + kDW * i) + row;
      jv[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r_topk, (uint32_t)slot * 4u, 0, 0);
    }
    const int wi = 16 * (kDTw * c + wv) + row;   // window row of this lane (window tile)
    const float rv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_wsc, (uint32_t)wi * 4u, 0, 0));
    uint32_t qraw[QF32 ? D / 8 : D / 16];
    if (c == 0) {
      // lane (head row, quad): dims quad*(D/4) .. +D/4 of head hb*16 + row
      const uint32_t qoff = (uint32_t)(((hb * kDH + row) * D + quad * (D / 4)) * QE);
      buffer_load_words<(D / 4) * QE>(qraw, r_q, qoff);
    }
    // offsets (selects, not branches: a branch would pull each load down to its use)
    uint32_t coff[kDMainT], soff[kDMainT], vcoff[kDMainT], vsoff[kDMainT];
    float sks[NT];
    const int vd = d0 + 16 * quad;  // V piece of lane (key row, part quad): dims vd .. vd+15
#pragma unroll
    for (int i = 0; i < kDMainT; ++i) {
      const int slot = 16 * (kDTm * c + wv + kDW * i) + row;
      const int32_t j = jv[i];
      const bool ok = slot < K && j >= 0 && j < vis;
      coff[i] = ok ? (uint32_t)j * (D / 2) + quad * (D / 8) : kOutOfRange;
      soff[i] = ok ? (uint32_t)j * (D / 16) + quad * (D / 64) : kOutOfRange;
      vcoff[i] = ok ? (uint32_t)j * (D / 2) + vd / 2 : kOutOfRange;
      vsoff[i] = ok ? (uint32_t)j * (D / 16) + vd / 16 : kOutOfRange;
      sks[i] = ok ? 1.0f : 0.0f;
    }
    sks[kDMainT] = (wi < wcount) ? rv : 0.0f;
    // ---- every key load of the chunk (rows past the window read as zeros) ----
    MainUnit<D> mu[kDMainT];
    VPiece vp[NT];
#pragma unroll
    for (int i = 0; i < kDMainT; ++i) {
      if (wv + kDW * i < nme) {
        buffer_load_words<D / 8>(mu[i].w, r_codes, coff[i]);
        buffer_load_words<D / 64>(mu[i].s, r_scales, soff[i]);
        load_vpiece_main(vp[i], r_codes, r_scales, vcoff[i], vsoff[i]);
      }
    }
    WinUnit<D> wu;
    if (wv < nwe) {
      buffer_load_words<D / 4>(wu.w, r_win, (uint32_t)wi * D + quad * (D / 4));
      load_vpiece_win(vp[kDMainT], r_win, (uint32_t)wi * D + vd);
    }
    if (c == 0) {
      // queries as f16 MFMA A operands (bf16 converts exactly in the f16 range;
      // fp32 splits into hi + lo parts)
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        if constexpr (QF32) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float v = __uint_as_float(qraw[8 * kk + i]);
            const _Float16 hi = (_Float16)v;
            qa[kk][i] = hi;
            qb[kk][i] = (_Float16)(v - (float)hi);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t x = qraw[4 * kk + i];
            qa[kk][2 * i] = (_Float16)__uint_as_float(x << 16);
            qa[kk][2 * i + 1] = (_Float16)__uint_as_float(x & 0xFFFF0000u);
          }
        }
      }
    }
    // ---- S for this wave's tiles; V slices into LDS ----
    float4_t sacc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) sacc[i] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kDMainT; ++i) {
      const int lt = wv + kDW * i;
      if (lt < nmc) score_main<D, QF32>(mu[i], qa, qb, sacc[i]);
      if (lt < nme) store_vpiece(vp[i], true, &L.vt[(16 * lt + row) * DecLds::VT + 16 * quad]);
    }
    if (wv < nwc) score_win<D, QF32>(wu, qa, qb, sacc[kDMainT]);
    if (wv < nwe) store_vpiece(vp[kDMainT], false, &L.vt[(16 * (kDTm + wv) + row) * DecLds::VT + 16 * quad]);
    // ---- chunk statistics: lane holds key (16*tile + row) of heads 4*quad + j ----
    float zz[NT][4];
    float rm = 0.0f;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const bool live = (i < kDMainT) ? (wv + kDW * i < nmc) : (wv < nwc);
      const float ks = live ? sks[i] : 0.0f;
      rm = fmaxf(rm, ks);
#pragma unroll
      for (int j = 0; j < 4; ++j) zz[i][j] = (ks != 0.0f) ? sacc[i][j] * tau2 * ks : -INFINITY;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rm = fmaxf(rm, __shfl_xor(rm, o, 64));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < NT; ++i) mx = fmaxf(mx, zz[i][j]);
      mx = max16_lanes(mx);
      if (row == 0) L.wmax[wv][4 * quad + j] = mx;
    }
    if (l == 0) L.wr[wv] = rm;
    __syncthreads();
    float mnew[4], alpha[4];
    rm = 0.0f;
#pragma unroll
    for (int w = 0; w < kDW; ++w) rm = fmaxf(rm, L.wr[w]);
    int e_new = 0;
    (void)frexpf(rm, &e_new);
    e_new = (rm > 0.0f) ? 1 - e_new : 0;  // chunk's largest r * 2^e_new in [1, 2)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float cm = -INFINITY;
#pragma unroll
      for (int w = 0; w < kDW; ++w) cm = fmaxf(cm, L.wmax[w][4 * quad + j]);
      mnew[j] = fmaxf(m_run[j], cm);
      alpha[j] = (m_run[j] == -INFINITY) ? 0.0f : exp2f(m_run[j] - mnew[j]);
      m_run[j] = mnew[j];
    }
    // ---- P' = 2^(z - max) * r * 2^e_new as f16 into LDS [head][key] ----
    // the denominator sums 2^(z - max); the window scale r enters only P'
#pragma unroll
    for (int j = 0; j < 4; ++j) l_part[j] *= alpha[j];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int lt = (i < kDMainT) ? wv + kDW * i : kDTm + wv;
      const bool stored = (i < kDMainT) ? (wv + kDW * i < nme) : (wv < nwe);
      if (!stored) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pr = (zz[i][j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(zz[i][j] - mnew[j]);
        l_part[j] += pr;
        L.p[(4 * quad + j) * DecLds::PT + 16 * lt + row] = (_Float16)ldexpf(pr * sks[i], e_new);
      }
    }
    if (c > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] *= ldexpf(alpha[j], e_new - e_cur);
    }
    e_cur = e_new;
    __syncthreads();
    // ---- acc += P V for dims 16*dt .. over this wave's half of the 32-key
    // steps: the chunk's Top-K steps, then its window steps ----
    if (16 * dt < DD) {
      const int nsm = nme / 2, nst = nsm + nwe / 2;
      for (int st = khalf; st < nst; st += 2) {
        const int k0 = (st < nsm) ? 32 * st : 16 * kDTm + 32 * (st - nsm);
        const half8_t a = *reinterpret_cast<const half8_t *>(&L.p[row * DecLds::PT + k0 + 8 * quad]);
        const half8_t b = v_operand_tr(L.vt, DecLds::VT, k0, 16 * dt, row, quad);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
      }
    }
  }

  // ---- softmax denominators: lane partials -> rows -> waves; the two
  // k-step halves of each dim tile meet in LDS ----
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float v = sum16_lanes(l_part[j]);
    if (row == 0) L.wsum[wv][4 * quad + j] = v;
  }
  if (khalf == 1) L.ored[dt][l] = acc;
  __syncthreads();
  if (khalf == 1 || 16 * dt >= DD) return;
  acc += L.ored[dt][l];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = 4 * quad + j, h = hb * kDH + hh;
    float lt = 0.0f;
#pragma unroll
    for (int w = 0; w < kDW; ++w) lt += L.wsum[w][hh];
    if (h >= H) continue;
    out[((int64_t)m * H + h) * D + d0 + 16 * dt + row] = (lt > 0.0f) ? ldexpf(acc[j] / lt, -e_cur) : 0.0f;
    if (blockIdx.x == 0 && dt == 0 && row == 0 && lse)
      lse[(int64_t)m * H + h] = (lt > 0.0f) ? (m_run[j] + log2f(lt)) * 0.6931471805599453f : -INFINITY;
  }
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

// The fused decode kernel fills the chip when there are few queries; with
// many queries (prefill) the flash kernel's one-workgroup-per-query grid is
// already large and computes each logit once.
static bool use_decode_kernel(int m, int heads, int dim, int64_t max_len) {
  // its buffer descriptors span one sequence's rows: byte offsets must fit
  if (max_len * (dim / 2) >= kMaxRsrcBytes) return false;
  return (int64_t)m * ((heads + kHB - 1) / kHB) < 256;
}

// Neither schedule needs a workspace: the decode kernel keeps every key of a
// (query, head block) in one workgroup, so there are no partial outputs.
size_t attn_ws_bytes(int m, int heads, int dim, int top_k, int window) {
  (void)m; (void)heads; (void)dim; (void)top_k; (void)window;
  return 256;
}

template <int D, bool QF32>
static int attn_impl(const csa2_fp4_cache &kv, const csa2_queries &qs, const void *q, int heads,
                     const int32_t *topk, int K, const csa2_swa &swa, float scale, float *out, float *lse, void *ws,
                     hipStream_t stream) {
  const int W = swa.window;
  const float tau2 = scale * 1.4426950408889634f;  // log2-domain softmax: p = 2^(z - max)
  if (use_decode_kernel(qs.m, heads, D, kv.max_len)) {
    const dim3 grid((D + kDD - 1) / kDD, qs.m, (heads + kDH - 1) / kDH);
    CSA2_TIMED_LAUNCH(kTimedAttn, (k_attn_decode<D, QF32>), grid, dim3(64 * kDW), stream, q, heads, kv.codes,
                      kv.scales, kv.seq_start, kv.seq_len, kv.ratio, qs.seq, qs.pos, topk, K, swa.codes, swa.scale,
                      swa.start, swa.count, W, tau2, out, lse);
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
