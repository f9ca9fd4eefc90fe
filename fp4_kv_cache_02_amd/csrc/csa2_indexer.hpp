// Device-side pieces of the CSA2 indexer shared by the decode scan, the
// pool re-score and the multi-query prefill scorer (P1 section "Compressed
// Sparse Attention 2 (CSA2)"; P2 section 03; P4 section 二).
//
// Score s_j = sum_h w_h * max(0, q_h . k_j).  The dot products run on MFMA
// (v_mfma_f32_16x16x32_f16): rows = (query, head) pairs, columns = 16
// positions, k = channels.  FP4 keys decode exactly to f16 (e2m1 * e4m3 has
// <= 6 significant bits); each head's bf16 query is scaled by a power of two
// so its largest element lies in [2^14, 2^15) and converts exactly to f16,
// and the inverse power of two is folded into w_h.  Products are therefore
// exact and only the fp32 accumulation rounds.
#pragma once

#include "csa2_device.hpp"

namespace csa2 {

// ---------------------------------------------------------------------------
// per-wave query operands
// ---------------------------------------------------------------------------

template <int DI>
struct IdxQuery {
  half8_t a[DI / 32];  // A operand of MFMA t: lane (row m = l%16, quarter qq = l/16)
                       // holds channels qq*DI/4 + 8t .. +7 of head m
  float w[4];          // scaled weights of heads 4*qq + j (0 for missing heads)
};

CSA2_DEV float max_rows4(float v) {
  uint32_t u = __float_as_uint(v);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  float a = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  uint32_t ua = __float_as_uint(a);
  auto s16 = __builtin_amdgcn_permlane16_swap(ua, ua, false, false);
  return fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

// Query operands of one 16-row tile.  Row i (= lane % 16) is the bf16 vector
// `row` of DI channels with weight `wrow`, or a zero row when !valid.  Lane
// (i, qq) loads the DI/4 contiguous channels it feeds to MFMA with 16-byte
// loads; a[] receives them scaled exactly to f16 (row max into [2^14, 2^15)),
// w[j] the weight of row 4*qq + j with the inverse scale folded in.
template <int DI>
CSA2_DEV void load_query_rows(const uint16_t *__restrict__ row, bool valid, float wrow, half8_t a[DI / 32],
                              float w[4]) {
  const int l = lane_id();
  const int qq = l >> 4;
  constexpr int PER = DI / 4;
  float v[PER];
  float mx = 0.0f;
  const uint4 *src = reinterpret_cast<const uint4 *>(row + qq * PER);
#pragma unroll
  for (int k = 0; k < PER / 8; ++k) {
    const uint4 x = valid ? src[k] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t wds[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * k + 2 * i] = __uint_as_float(wds[i] << 16);
      v[8 * k + 2 * i + 1] = __uint_as_float(wds[i] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) mx = fmaxf(mx, fabsf(v[i]));
  mx = max_rows4(mx);
  int e = 0;
  (void)frexpf(mx, &e);
  const int kf = (mx > 0.0f) ? 15 - e : 0;  // row max scaled into [2^14, 2^15)
#pragma unroll
  for (int t = 0; t < DI / 32; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) a[t][i] = (_Float16)ldexpf(v[8 * t + i], kf);
  const float wv = valid ? wrow : 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * qq + j;
    w[j] = ldexpf(__shfl(wv, r, 64), -__shfl(kf, r, 64));
  }
}

// q: [H][DI] bf16 of this query, w: [H] fp32; row i of the tile is head i.
template <int DI>
CSA2_DEV void load_idx_query(const uint16_t *__restrict__ q, const float *__restrict__ w, int H,
                             IdxQuery<DI> &Q) {
  const int m = lane_id() & 15;
  const bool valid = m < H;
  load_query_rows<DI>(q + m * DI, valid, valid ? w[m] : 0.0f, Q.a, Q.w);
}

// ---------------------------------------------------------------------------
// one 16-position tile
// ---------------------------------------------------------------------------

// The codes this lane feeds into the tile: DI/8 bytes of one row.
template <int DI>
struct LaneCodes {
  uint32_t w[DI / 32];
  uint32_t s;  // DI/64 scale bytes (little-endian)
};

template <int DI>
CSA2_DEV void load_lane_codes(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, int64_t row,
                              int qq, LaneCodes<DI> &c) {
  const uint8_t *cp = codes + row * (DI / 2) + qq * (DI / 8);
  const uint8_t *sp = scales + row * (DI / 16) + qq * (DI / 64);
  if constexpr (DI == 64) {
    const uint2 x = *reinterpret_cast<const uint2 *>(cp);
    c.w[0] = x.x;
    c.w[1] = x.y;
    c.s = *sp;
  } else if constexpr (DI == 128) {
    const uint4 x = *reinterpret_cast<const uint4 *>(cp);
    c.w[0] = x.x;
    c.w[1] = x.y;
    c.w[2] = x.z;
    c.w[3] = x.w;
    c.s = *reinterpret_cast<const uint16_t *>(sp);
  } else {
    static_assert(DI == 256, "indexer dim");
    const uint4 x = reinterpret_cast<const uint4 *>(cp)[0];
    const uint4 y = reinterpret_cast<const uint4 *>(cp)[1];
    c.w[0] = x.x; c.w[1] = x.y; c.w[2] = x.z; c.w[3] = x.w;
    c.w[4] = y.x; c.w[5] = y.y; c.w[6] = y.z; c.w[7] = y.w;
    c.s = *reinterpret_cast<const uint32_t *>(sp);
  }
}

// max(x, 0) and max(a, b) as one v_med3_f32 each.  Scores are finite or
// -inf (never NaN), and for such values the median with FLT_MAX is exactly
// the maximum; fmaxf would add NaN canonicalisations (and a +inf bound is
// folded back into fmaxf by the compiler).
CSA2_DEV float relu_f(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.40282347e38f); }
CSA2_DEV float max_f(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, 3.40282347e38f); }

// max over the 8 lanes of each half-row (finite or -inf values)
CSA2_DEV float max8_scores(float v) {
  v = max_f(v, dpp_f<kDppXor1>(v));
  v = max_f(v, dpp_f<kDppXor2>(v));
  return max_f(v, dpp_f<kDppHalfMirror>(v));
}

// B operands of the DI/32 MFMAs of one tile: lane (column n = l%16, quarter
// qq = l/16) decodes the channels qq*DI/4 + 8t .. +7 of its position.
template <int DI>
CSA2_DEV void decode_keys(const LaneCodes<DI> &c, half8_t b[DI / 32]) {
  _Float16 sc[(DI / 64 > 0) ? DI / 64 : 1];
  if constexpr (DI == 64) {
    sc[0] = e4m3x2_to_f16(c.s)[0];
  } else if constexpr (DI == 128) {
    const half2_t s2 = e4m3x2_to_f16(c.s);
    sc[0] = s2[0];
    sc[1] = s2[1];
  } else {
    const half2_t s2 = e4m3x2_to_f16(c.s);
    const half2_t s3 = e4m3x2_to_f16(c.s >> 16);
    sc[0] = s2[0]; sc[1] = s2[1]; sc[2] = s3[0]; sc[3] = s3[1];
  }
#pragma unroll
  for (int t = 0; t < DI / 32; ++t) b[t] = fp4x8_dequant_f16(c.w[t], sc[t / 2]);
}

// This lane's weighted ReLU of the four rows 4*(lane/16) + j of an MFMA
// result, w[j] the rows' (scaled) weights.
CSA2_DEV float weighted_relu4(const float w[4], float4_t acc) {
  float part = w[0] * relu_f(acc[0]);
  part = fmaf(w[1], relu_f(acc[1]), part);
  part = fmaf(w[2], relu_f(acc[2]), part);
  part = fmaf(w[3], relu_f(acc[3]), part);
  return part;
}

// This lane's share of the score of position (lane % 16) of the tile: the
// weighted ReLU of its four heads 4*(lane/16) + j.  The score is the sum of
// the four quarters' shares, added as (q0 + q2) + (q1 + q3).
template <int DI>
CSA2_DEV float tile_partial(const IdxQuery<DI> &Q, const LaneCodes<DI> &c) {
  half8_t b[DI / 32];
  decode_keys<DI>(c, b);
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int t = 0; t < DI / 32; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Q.a[t], b[t], acc, 0, 0, 0);
  return weighted_relu4(Q.w, acc);
}

// Score of position (lane % 16) of the tile, returned in all four quarters.
template <int DI>
CSA2_DEV float tile_score(const IdxQuery<DI> &Q, const LaneCodes<DI> &c) {
  return sum_rows4(tile_partial<DI>(Q, c));
}

// Scores of four tiles from their lane shares p0..p3 with three lane swaps:
// row r (lanes 16r .. 16r+15) returns the 16 scores of tile row_tile(r).
// Same addition order as sum_rows4, so scores match tile_score bit for bit.
CSA2_DEV int row_tile(int row) { return ((row & 1) << 1) | (row >> 1); }  // rows hold tiles 0, 2, 1, 3
CSA2_DEV float tile_scores_x4(float p0, float p1, float p2, float p3) {
  // permlane32_swap(x, y): x keeps its low half and takes y's low half; y takes x's high half
  const auto a2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  const float a = __uint_as_float(a2[0]) + __uint_as_float(a2[1]);   // [t0 q0+q2, t0 q1+q3, t1 .., t1 ..]
  const auto b2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
  const float b = __uint_as_float(b2[0]) + __uint_as_float(b2[1]);   // same for tiles 2, 3
  // permlane16_swap(x, y): odd rows of x trade places with even rows of y
  const auto c2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(c2[0]) + __uint_as_float(c2[1]);
}

// Scores of two tiles whose rows hold two queries of 8 heads each (tile a:
// queries 2a, 2a+1 in rows 0-7, 8-15) from their lane shares pa, pb with one
// lane swap: row r of the result holds query row_tile(r) of the four
// {a0, a1, b0, b1} (rows hold a0, b0, a1, b1).
CSA2_DEV float tile_scores_x2(float pa, float pb) {
  const auto c2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
  return __uint_as_float(c2[0]) + __uint_as_float(c2[1]);
}

// Loads of one lane relative to a chunk: `row` counts from the chunk's first
// entry, so the offsets stay 32-bit and the bases stay scalar.  NT: the loads
// are non-temporal (streamed past the caches), for data read exactly once,
// which lifts the achievable HBM read rate; data that other workgroups read
// again takes plain loads.
template <int DI, bool NT = true>
CSA2_DEV void load_lane_codes_rel(const uint8_t *__restrict__ cbase, const uint8_t *__restrict__ sbase,
                                  uint32_t row, uint32_t qq, LaneCodes<DI> &c) {
  const uint32_t co = row * (DI / 2) + qq * (DI / 8);
  const uint32_t so = row * (DI / 16) + qq * (DI / 64);
  auto ld = [](const auto *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
  };
  if constexpr (DI == 64) {
    const u32x2_t x = ld(reinterpret_cast<const u32x2_t *>(cbase + co));
    c.w[0] = x[0];
    c.w[1] = x[1];
    c.s = ld(sbase + so);
  } else if constexpr (DI == 128) {
    const u32x4_t x = ld(reinterpret_cast<const u32x4_t *>(cbase + co));
    c.w[0] = x[0];
    c.w[1] = x[1];
    c.w[2] = x[2];
    c.w[3] = x[3];
    c.s = ld(reinterpret_cast<const uint16_t *>(sbase + so));
  } else {
    static_assert(DI == 256, "indexer dim");
    const u32x4_t x = ld(reinterpret_cast<const u32x4_t *>(cbase + co));
    const u32x4_t y = ld(reinterpret_cast<const u32x4_t *>(cbase + co + 16));
    c.w[0] = x[0]; c.w[1] = x[1]; c.w[2] = x[2]; c.w[3] = x[3];
    c.w[4] = y[0]; c.w[5] = y[1]; c.w[6] = y[2]; c.w[7] = y[3];
    c.s = ld(reinterpret_cast<const uint32_t *>(sbase + so));
  }
}

CSA2_DEV int64_t visible_entries(const int32_t *seq_len, const int32_t *q_seq, const int32_t *q_pos, int ratio,
                                 int m, int *s_out) {
  const int s = q_seq[m];
  *s_out = s;
  const int64_t lim = ((int64_t)q_pos[m] + 1) / ratio;
  const int64_t v = min<int64_t>((int64_t)seq_len[s], lim);
  return v > 0 ? v : 0;
}

}  // namespace csa2
