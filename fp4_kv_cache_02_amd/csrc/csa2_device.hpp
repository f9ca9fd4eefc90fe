// Device helpers shared by the CSA2 kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA2_DEV __device__ __forceinline__

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace csa2 {

constexpr int kWave = 64;
constexpr int kBlock = 8;          // positions per indexer block
constexpr int kGroup = 16;         // channels per FP4 scale
constexpr int kHistBits = 12;      // top bits of a score key used by the pool histogram
constexpr int kHistBins = 1 << kHistBits;

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------

// E4M3FN byte -> fp32, exact (NaN codes are not produced by the encoders).
CSA2_DEV float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = (e == 0) ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -v : v;
}

// Two E4M3FN bytes (the low 16 bits of `w`) -> two f16, exact (every finite
// E4M3 value is an f16 normal).  Hardware convert with unit scale.
CSA2_DEV half2_t e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

// The two E2M1 codes of byte `SEL` of `w` -> f16 pair (low nibble first), exact.
template <int SEL>
CSA2_DEV half2_t e2m1x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// 8 E2M1 codes of `w` (channels 0..7, channel 2k in the low nibble of byte k)
// times the f16 scale `s`: the exact products e2m1 * e4m3 (at most 6
// significant bits, magnitude within [2^-10, 2688]) are f16 numbers.
CSA2_DEV half8_t fp4x8_dequant_f16(uint32_t w, _Float16 s) {
  const half2_t ss = {s, s};
  half2_t p0 = e2m1x2_to_f16<0>(w) * ss;
  half2_t p1 = e2m1x2_to_f16<1>(w) * ss;
  half2_t p2 = e2m1x2_to_f16<2>(w) * ss;
  half2_t p3 = e2m1x2_to_f16<3>(w) * ss;
  half8_t r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

CSA2_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// ---------------------------------------------------------------------------
// LDS operand loads
// ---------------------------------------------------------------------------

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element (i%4)
// of the 8-byte chunks addressed by lanes i/4, i/4+4, i/4+8, i/4+12.
CSA2_DEV short4_t lds_read_tr16(const _Float16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_t *)((__attribute__((address_space(3))) char *)(p)));
}

// MFMA operand (16x16x32, A or B) of a product over 32 keys: the lane of
// row/column lane % 16 and k-quarter quad holds keys k0 + 8*quad .. +7 at
// dim d0 + (lane % 16) of a row-major [key][dim] f16 tile with row stride
// `stride` (the tile read down its columns, without a transposed copy).
CSA2_DEV half8_t v_operand_tr(const _Float16 *tile, int stride, int k0, int d0, int row, int quad) {
  const _Float16 *base = tile + (k0 + 8 * quad + (row >> 2)) * stride + d0 + 4 * (row & 3);
  const short4_t lo = lds_read_tr16(base);
  const short4_t hi = lds_read_tr16(base + 4 * stride);
  return __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Eight E4M3 codes (two little-endian words) as f16.
CSA2_DEV half8_t e4m3x8_to_f16(uint32_t a, uint32_t b) {
  const half2_t a0 = e4m3x2_to_f16(a), a1 = e4m3x2_to_f16(a >> 16);
  const half2_t a2 = e4m3x2_to_f16(b), a3 = e4m3x2_to_f16(b >> 16);
  return (half8_t){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

// ---------------------------------------------------------------------------
// exact encoders (write path)
// ---------------------------------------------------------------------------

// Non-negative finite E4M3 value of code k (0..126), fp32 exact.
CSA2_DEV float e4m3_pos_value(int k) { return e4m3_to_f32((uint32_t)k); }

// Code of the E4M3 value nearest to the exact quotient a / den (a >= 0, den
// in {1, 6}), ties to the even code, saturating at 448.  Midpoint m_i between
// codes i and i+1 is (v_i + v_{i+1}) / 2 and den * m_i is exact in fp32, so
// the comparisons below are exact.  `passed(i)` (a lies above midpoint i, or
// on it with i+1 even) is monotone in i; the code is the number of passed
// midpoints, found by binary search.
CSA2_DEV uint32_t e4m3_nearest_code(float a, float den) {
  int lo = 0, hi = 126;  // answer in [lo, hi]
  while (lo < hi) {
    const int i = (lo + hi) >> 1;  // test midpoint i (between i and i+1)
    const float t = den * 0.5f * (e4m3_pos_value(i) + e4m3_pos_value(i + 1));
    const bool passed = (a > t) || (a == t && ((i + 1) & 1) == 0);
    if (passed) lo = i + 1; else hi = i;
  }
  return (uint32_t)lo;
}

// E2M1 magnitude code of |x| for scale s > 0 (nearest to |x|/s, ties to even
// code, saturating at 6): thresholds m*s are exact fp32 products.
CSA2_DEV uint32_t e2m1_mag_code(float ax, float s) {
  uint32_t c = 0;
  c += ax > 0.25f * s;
  c += ax >= 0.75f * s;
  c += ax > 1.25f * s;
  c += ax >= 1.75f * s;
  c += ax > 2.5f * s;
  c += ax >= 3.5f * s;
  c += ax > 5.0f * s;
  return c;
}

// ---------------------------------------------------------------------------
// ordering keys
// ---------------------------------------------------------------------------

// Order-preserving map fp32 -> u32 (larger float -> larger key); -0 is
// folded onto +0 first so equal floats give equal keys.
CSA2_DEV uint32_t f2key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// raw buffer descriptors
// ---------------------------------------------------------------------------

// Raw buffer descriptor over `bytes` bytes (gfx9 data format word).  Loads
// at offsets past the end return zeros and stores there are dropped, without
// touching memory, so predicated accesses need no branch.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
CSA2_DEV rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// An offset past every descriptor used here, with room for per-access
// additions (< 2 GB - kMaxRsrcBytes) without wrapping: descriptors stay
// below kMaxRsrcBytes.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int64_t kMaxRsrcBytes = 0x7FFF0000;

// ---------------------------------------------------------------------------
// cross-lane helpers
// ---------------------------------------------------------------------------

// DPP move within rows of 16 lanes (row_mask / bank_mask all enabled).
template <int CTRL>
CSA2_DEV float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;       // lane i <-> 15-i within 16 lanes

// max over the 8 lanes of each half-row, result in all 8 lanes
CSA2_DEV float max8_lanes(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return v;
}
// max / sum over the 16 lanes of each row
CSA2_DEV float max16_lanes(float v) {
  v = max8_lanes(v);
  return fmaxf(v, dpp_f<kDppMirror>(v));
}
CSA2_DEV float sum16_lanes(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}

// Sum of v over the four 16-lane rows (lanes l, l^16, l^32, l^48), in every lane.
CSA2_DEV float sum_rows4(float v) {
  uint32_t u = __float_as_uint(v);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  float a = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  uint32_t ua = __float_as_uint(a);
  auto s16 = __builtin_amdgcn_permlane16_swap(ua, ua, false, false);
  return __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
}

CSA2_DEV int lane_id() { return __lane_id(); }

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active):
// Hillis-Steele steps inside each 16-lane row (row_shr 1, 2, 4, 8), then the
// row totals carried across rows with row_bcast 15 and row_bcast 31.  DPP
// moves take a few cycles where a shuffle is an LDS round trip.
CSA2_DEV int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive prefix sum of `v` over the threads of a block of NT threads
// (NT a multiple of 64, <= 1024); `scratch` holds NT/64 + 1 ints of LDS.
// Returns the prefix and writes the block total to *total.  Wave scans, then
// wave 0 scans the wave totals; the scratch is free again on return.
template <int NT>
CSA2_DEV int block_exclusive_scan(int v, int *scratch, int *total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int t = (lane < NW) ? scratch[lane] : 0;
    const int ti = wave_incl_scan(t);
    if (lane < NW) scratch[lane] = ti - t;
    if (lane == NW - 1) scratch[NW] = ti;
  }
  __syncthreads();
  const int res = scratch[wave] + incl - v;
  *total = scratch[NW];
  __syncthreads();
  return res;
}

}  // namespace csa2
