// CSA2 write path: FP4 quantise-on-write of main-KV rows with the indexer key
// derived from each written entry, FP8 window rows, and an FP4 decode probe.
//
// Format (P1 section "FP4 KV、Bounded Replay 及其他扩展"; P4 section 三; P5
// section "缓存精度与持久化分层"): E2M1 elements, one E4M3 scale per 16
// channels, no global scale; the window KV stays FP8.  The indexer key is
// projected from the main-KV entry (P4 section 二; P5 section "CSA2注意力").
#include "csa2_internal.hpp"

#include <algorithm>

namespace csa2 {

template <typename T>
CSA2_DEV float load_as_f32(const T *p);
template <>
CSA2_DEV float load_as_f32<float>(const float *p) { return *p; }
template <>
CSA2_DEV float load_as_f32<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

// Encode one 16-channel group held in v[16]; returns the 8 packed code bytes
// (little-endian in a uint2) and the scale byte.
CSA2_DEV void encode_group(const float v[16], uint2 *packed, uint8_t *scale_byte) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sc = e4m3_nearest_code(amax, 6.0f);
  const float s = e4m3_pos_value((int)sc);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t mag = (s == 0.0f) ? 0u : e2m1_mag_code(fabsf(v[i]), s);
    const uint32_t code = mag | ((__float_as_uint(v[i]) >> 31) << 3);
    if (i < 8) lo |= code << (4 * i); else hi |= code << (4 * (i - 8));
  }
  packed->x = lo;
  packed->y = hi;
  *scale_byte = (uint8_t)sc;
}

// Plain quantise: one thread per 16-channel group.
template <typename T>
__global__ __launch_bounds__(256) void k_quantize_fp4(const T *__restrict__ x, int64_t rows, int dim,
                                                       const int64_t *__restrict__ dst_row,
                                                       uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  const int gpr = dim / kGroup;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * gpr) return;
  const int64_t r = gid / gpr;
  const int g = (int)(gid - r * gpr);
  float v[16];
  const T *src = x + r * dim + g * kGroup;
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = load_as_f32<T>(src + i);
  uint2 packed;
  uint8_t sb;
  encode_group(v, &packed, &sb);
  const int64_t d = dst_row ? dst_row[r] : r;
  *reinterpret_cast<uint2 *>(codes + d * (dim / 2) + g * 8) = packed;
  scales[d * (dim / kGroup) + g] = sb;
}

// Quantise RB rows per workgroup and derive their indexer keys:
//   phase 1 encode every group, keep the exact decoded row in LDS;
//   phase 2 fp64 GEMV y = W_ik^T DQ4(row), summed in channel order from +0,
//           rounded once to fp32;
//   phase 3 encode y into the indexer-key planes.
constexpr int kDeriveLdsFloats = 4096;  // decoded rows per workgroup (16 KiB); needs idx_dim <= dim

// JM: row slots per thread in phase 2, at least ceil(rows per workgroup /
// (256 / idx_dim)) (at most 16, since idx_dim <= dim).
template <typename T, int JM>
__global__ __launch_bounds__(256) void k_quantize_fp4_derive(const T *__restrict__ x, int64_t rows, int dim,
                                                              const int64_t *__restrict__ dst_row,
                                                              uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                              const float *__restrict__ w_ik, int idx_dim,
                                                              uint8_t *__restrict__ ik_codes,
                                                              uint8_t *__restrict__ ik_scales) {
  __shared__ float dq[kDeriveLdsFloats];
  __shared__ float yk[kDeriveLdsFloats];
  const int rb = kDeriveLdsFloats / dim;  // rows per workgroup (dim <= 4096)
  const int64_t r0 = (int64_t)blockIdx.x * rb;
  const int nr = (int)min<int64_t>(rb, rows - r0);
  const int gpr = dim / kGroup;

  // phase 1
  for (int t = threadIdx.x; t < nr * gpr; t += blockDim.x) {
    const int rr = t / gpr, g = t - rr * gpr;
    float v[16];
    const T *src = x + (r0 + rr) * dim + g * kGroup;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = load_as_f32<T>(src + i);
    uint2 packed;
    uint8_t sb;
    encode_group(v, &packed, &sb);
    const int64_t d = dst_row ? dst_row[r0 + rr] : r0 + rr;
    *reinterpret_cast<uint2 *>(codes + d * (dim / 2) + g * 8) = packed;
    scales[d * gpr + g] = sb;
    const float s = e4m3_pos_value(sb);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = (i < 8) ? (packed.x >> (4 * i)) & 15u : (packed.y >> (4 * (i - 8))) & 15u;
      // E2M1 magnitude of code m: 0, .5, 1, 1.5 for m < 4, else 2^((m-2)/2) * (1 or 1.5)
      const uint32_t m = c & 7u;
      const float mag = (m < 4) ? 0.5f * (float)m : (float)(1u << ((m - 2) >> 1)) * ((m & 1u) ? 1.5f : 1.0f);
      const float val = mag * s;
      dq[rr * dim + g * kGroup + i] = (c & 8u) ? -val : val;
    }
  }
  __syncthreads();

  // phase 2: thread -> column i, rows rr = j*(256/idx_dim) + t/idx_dim
  const int col = threadIdx.x % idx_dim;
  const int rstep = blockDim.x / idx_dim;
  const int rfirst = threadIdx.x / idx_dim;
  // Channels go in ascending order (fp64 fma per channel), 16 at a time: the
  // 16 W_ik values of a block are loaded together, so the loop waits for
  // memory once per block, not once per channel (dim is a multiple of 16).
  double acc[JM];
#pragma unroll
  for (int j = 0; j < JM; ++j) acc[j] = 0.0;
  for (int c0 = 0; c0 < dim; c0 += kGroup) {
    float wv[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) wv[u] = w_ik[(int64_t)(c0 + u) * idx_dim + col];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const double w = (double)wv[u];
#pragma unroll
      for (int j = 0; j < JM; ++j) {
        const int rr = rfirst + j * rstep;
        if (rr < nr) acc[j] = fma((double)dq[rr * dim + c0 + u], w, acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < JM; ++j) {
    const int rr = rfirst + j * rstep;
    if (rr < nr) yk[rr * idx_dim + col] = (float)acc[j];
  }
  __syncthreads();

  // phase 3
  const int igpr = idx_dim / kGroup;
  for (int t = threadIdx.x; t < nr * igpr; t += blockDim.x) {
    const int rr = t / igpr, g = t - rr * igpr;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = yk[rr * idx_dim + g * kGroup + i];
    uint2 packed;
    uint8_t sb;
    encode_group(v, &packed, &sb);
    const int64_t d = dst_row ? dst_row[r0 + rr] : r0 + rr;
    *reinterpret_cast<uint2 *>(ik_codes + d * (idx_dim / 2) + g * 8) = packed;
    ik_scales[d * igpr + g] = sb;
  }
}

// Quantise rows and derive their indexer keys on the fp64 matrix cores, for
// dim <= 512.  The projection y = W_ik^T DQ4(row) is an fp64 product: every
// term DQ4(c) * w is exact in fp64 (at most 6 significant bits times fp32's
// 24), the sum is accumulated in fp64 by v_mfma_f64_16x16x4_f64 and rounded
// once to fp32, like the oracle's fp64 matrix product (whose summation
// order is not fixed either; fp64 sums in another order round to the same
// fp32 unless they straddle an fp32 rounding boundary within ~2^-50).
//
// grid (ceil(rows / 16), idx_dim / (16 CT)), 64 CT KS threads.  A workgroup
// encodes its 16 rows (codes and scales written by the workgroups of the
// first column group) and keeps their exact values in LDS as fp64; wave
// (ct, ks) multiplies them by the 16 key columns of tile ct over channel
// slice ks (W_ik loaded before the encode, so its latency overlaps it).  With
// KS > 1 (few rows: 8 waves per tile) the slices' partial tiles are added
// in slice order.  The 16 columns of a tile are one FP4 group of the key.
typedef double double4_t __attribute__((ext_vector_type(4)));
constexpr int kDeriveRows = 16;
constexpr int kDeriveMaxDim = 512;

//
// T = uint8_t derives the keys of rows already in the cache instead: their
// codes and scales are read from the destination rows (nothing is encoded or
// written to the main planes, x is unused).
//
// Workgroups with blockIdx.x past the row tiles clear zero[0 .. zero_n)
// (16-byte words) instead: a range the caller needs zeroed before its next
// launch, cleared here rather than by a launch of its own.
template <typename T, int CT, int KS>
__global__ __launch_bounds__(64 * CT * KS) void k_quantize_fp4_derive_mfma(
    const T *__restrict__ x, int64_t rows, int dim, const int64_t *__restrict__ dst_row, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ scales, const float *__restrict__ w_ik, int idx_dim, uint8_t *__restrict__ ik_codes,
    uint8_t *__restrict__ ik_scales, uint4 *__restrict__ zero, int64_t zero_n) {
  constexpr int NT = 64 * CT * KS;
  const int64_t row_tiles = (rows + kDeriveRows - 1) / kDeriveRows;
  if ((int64_t)blockIdx.x >= row_tiles) {
    const int64_t zb = ((int64_t)blockIdx.x - row_tiles) * gridDim.y + blockIdx.y;
    const int64_t zstride = ((int64_t)gridDim.x - row_tiles) * gridDim.y * NT;
    for (int64_t i = zb * NT + threadIdx.x; i < zero_n; i += zstride) zero[i] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  constexpr int DS = kDeriveMaxDim + 1;                 // fp64 row stride: rows fall in different banks
  constexpr int WPL = kDeriveMaxDim / 4 / KS;           // W_ik values per lane (one per k-step)
  __shared__ double dq[kDeriveRows * DS];
  __shared__ double part[KS > 1 ? KS * CT * 256 : 1];
  __shared__ float yk[CT * 256];
  const int64_t r0 = (int64_t)blockIdx.x * kDeriveRows;
  const int nr = (int)min<int64_t>(kDeriveRows, rows - r0);
  const int gpr = dim / kGroup;
  const int tid = threadIdx.x, l = lane_id(), wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ct = wv % CT, ks = wv / CT;
  const int col0 = (blockIdx.y * CT + ct) * kGroup;
  const int kper = dim / KS;                            // channels of this wave's slice
  const int c_begin = ks * kper;
  // ---- this lane's W_ik column entries: channel c_begin + 4 kk + l / 16 ----
  const rsrc_t r_w = make_rsrc(w_ik, (uint32_t)(dim * idx_dim * 4));
  float wreg[WPL];
#pragma unroll
  for (int kk = 0; kk < WPL; ++kk) {
    const int c = c_begin + 4 * kk + l / 16;
    const uint32_t off = (4 * kk < kper) ? (uint32_t)((c * idx_dim + col0 + l % 16) * 4) : kOutOfRange;
    wreg[kk] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_w, off, 0, 0));
  }
  // ---- encode the rows, exact values to LDS (rows past the end read as 0) ----
  for (int t = tid; t < kDeriveRows * gpr; t += NT) {
    const int rr = t / gpr, g = t - rr * gpr;
    double *dst = &dq[rr * DS + g * kGroup];
    if (rr >= nr) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[i] = 0.0;
      continue;
    }
    uint2 packed;
    uint8_t sb;
    if constexpr (__is_same(T, uint8_t)) {
      const int64_t d = dst_row ? dst_row[r0 + rr] : r0 + rr;
      packed = *reinterpret_cast<const uint2 *>(codes + d * (dim / 2) + g * 8);
      sb = scales[d * gpr + g];
    } else {
      float v[16];
      const T *src = x + (r0 + rr) * dim + g * kGroup;
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = load_as_f32<T>(src + i);
      encode_group(v, &packed, &sb);
      if (blockIdx.y == 0) {
        const int64_t d = dst_row ? dst_row[r0 + rr] : r0 + rr;
        *reinterpret_cast<uint2 *>(codes + d * (dim / 2) + g * 8) = packed;
        scales[d * gpr + g] = sb;
      }
    }
    const float sc = e4m3_pos_value(sb);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = (i < 8) ? (packed.x >> (4 * i)) & 15u : (packed.y >> (4 * (i - 8))) & 15u;
      // E2M1 magnitude of code m: 0, .5, 1, 1.5 for m < 4, else 2^((m-2)/2) * (1 or 1.5)
      const uint32_t m = c & 7u;
      const float mag = (m < 4) ? 0.5f * (float)m : (float)(1u << ((m - 2) >> 1)) * ((m & 1u) ? 1.5f : 1.0f);
      const float val = mag * sc;
      dst[i] = (double)((c & 8u) ? -val : val);
    }
  }
  __syncthreads();
  // ---- Y tile = DQ (16 rows x slice) x W (slice x 16 columns), fp64 ----
  double4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int kk = 0; kk < WPL; ++kk) {
    if (4 * kk >= kper) break;
    const double a = dq[(l % 16) * DS + c_begin + 4 * kk + l / 16];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, (double)wreg[kk], acc, 0, 0, 0);
  }
  // lane l holds rows l / 16 + 4 i of column l % 16
  if constexpr (KS > 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) part[((ks * CT + ct) * 64 + l) * 4 + i] = acc[i];
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double t = 0.0;
      for (int s2 = 0; s2 < KS; ++s2) t += part[((s2 * CT + ct) * 64 + l) * 4 + i];
      acc[i] = t;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) yk[ct * 256 + (l / 16 + 4 * i) * 16 + l % 16] = (float)(acc[i] + 0.0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // ---- encode each row's 16 key columns (one FP4 group) ----
  if (l < nr) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = yk[ct * 256 + l * 16 + i];
    uint2 packed;
    uint8_t sb;
    encode_group(v, &packed, &sb);
    const int64_t d = dst_row ? dst_row[r0 + l] : r0 + l;
    const int g = col0 / kGroup;
    *reinterpret_cast<uint2 *>(ik_codes + d * (idx_dim / 2) + g * 8) = packed;
    ik_scales[d * (idx_dim / kGroup) + g] = sb;
  }
}

// Indexer keys of many rows already in the cache, dim = 64 GQ (64, 128, 256
// or 512): the same fp64 product as k_quantize_fp4_derive_mfma with the work
// laid out for throughput.  A workgroup computes key columns 16 ct .. 16 ct
// + 15 (one FP4 group of the key) of 64 rows, wave w the 16-row tile w; its
// 16 W_ik columns are staged once in LDS and read by all four waves.  In a
// wave, k-slot q = l / 16 of the MFMA walks channels q dim/4 .. (q+1) dim/4
// - 1 in ascending order: lane l holds row l % 16's codes for those channels
// (GQ whole FP4 groups) and decodes them in registers, and reads column
// l % 16's weight at the same channel from LDS.  Four accumulators take the
// channels in turn and are added at the end (fp64 throughout, rounded once
// to fp32).
//
// 1-D grid of idx_dim / 16 * nq workgroups (nq = row quads rounded up to a
// multiple of 8), mapped so that the workgroups of one row quad run on one
// XCD (consecutive workgroups go to consecutive XCDs): they read the same
// rows, which then come from that XCD's L2.  Row quads past the last row exit.
// The two E2M1 codes of byte `sel` of `w` -> fp32 pair (low nibble first),
// exact (hardware convert with unit scale; sel is a constant after unrolling).
CSA2_DEV float2_t e2m1x2_to_f32(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

template <int GQ>
__global__ __launch_bounds__(256) void k_derive_tiles(int64_t rows, int dim, const int64_t *__restrict__ dst_row,
                                                      const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales,
                                                      const float *__restrict__ w_ik, int idx_dim,
                                                      uint8_t *__restrict__ ik_codes,
                                                      uint8_t *__restrict__ ik_scales) {
  constexpr int kq = GQ * kGroup;              // channels per k-slot
  __shared__ __attribute__((aligned(16))) float ws[kDeriveMaxDim * 16];   // [kk / 4][q][n][kk % 4]
  __shared__ float yk[4 * 256];
  const int cgs = idx_dim / kGroup;
  const uint32_t b = blockIdx.x;
  const int slot = (int)(b >> 3);
  const int ct = slot % cgs;
  const int64_t quad = (int64_t)(slot / cgs) * 8 + (b & 7);
  const int64_t r0 = quad * 64;
  if (r0 >= rows) return;
  const int tid = threadIdx.x, l = lane_id(), wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col0 = ct * kGroup;
  // ---- this workgroup's W_ik columns: 16 dim floats, 4 per load ----
  const rsrc_t r_w = make_rsrc(w_ik, (uint32_t)(dim * idx_dim * 4));
  u32x4_t wl[GQ];
#pragma unroll
  for (int i = 0; i < GQ; ++i) {
    const int c = tid + 256 * i, k = c >> 2, j = c & 3;
    wl[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                            r_w, (uint32_t)((k * idx_dim + col0 + 4 * j) * 4), 0, 0));
  }
  // ---- this lane's row: codes and scale values of its k-slot's groups ----
  const int64_t r = r0 + 16 * wv + (l % 16);
  const bool valid = r < rows;
  const int q = l / 16;
  const int64_t rc = valid ? r : rows - 1;     // a row in range (its codes are masked)
  const int64_t d = dst_row ? dst_row[rc] : rc;
  uint32_t cw[2 * GQ];
  float sf[GQ];
  const uint8_t *crow = codes + d * (dim / 2) + q * (kq / 2);
  const uint8_t *srow = scales + d * (dim / kGroup) + q * GQ;
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    const uint2 p = *reinterpret_cast<const uint2 *>(crow + 8 * g);
    cw[2 * g] = valid ? p.x : 0u;
    cw[2 * g + 1] = valid ? p.y : 0u;
    sf[g] = e4m3_pos_value(srow[g]);
  }
  // ---- W_ik columns to LDS as [kk / 4][q][n][kk % 4]: a lane reads 4 channels at once ----
#pragma unroll
  for (int i = 0; i < GQ; ++i) {
    const int c = tid + 256 * i, k = c >> 2, j = c & 3;
    const int qq = k / kq, kk = k - qq * kq;
    float *dst = &ws[(((kk >> 2) * 4 + qq) * 16 + 4 * j) * 4 + (kk & 3)];
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[4 * e] = __uint_as_float(wl[i][e]);
  }
  __syncthreads();
  if (r0 + 16 * wv >= rows) return;
  // ---- Y tile = DQ4 (16 rows x dim) x W (dim x 16 columns), fp64 ----
  // the next group's weights are read from LDS while the current group's
  // products run
  double4_t acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = (double4_t){0.0, 0.0, 0.0, 0.0};
  const float *wcol = ws + (q * 16 + (l % 16)) * 4;
  u32x4_t wn[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) wn[h] = *reinterpret_cast<const u32x4_t *>(wcol + h * 256);
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    u32x4_t w4[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) w4[h] = wn[h];
    if (g + 1 < GQ) {
#pragma unroll
      for (int h = 0; h < 4; ++h) wn[h] = *reinterpret_cast<const u32x4_t *>(wcol + (4 * (g + 1) + h) * 256);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {              // channels 16 g + 4 h .. + 3
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        // E2M1 pair (exact, unit scale) times the group's scale: exact in fp32
        const float2_t e = e2m1x2_to_f32(cw[2 * g + h / 2], 2 * (h % 2) + p);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const double a = (double)(e[u] * sf[g]);
          const double bw = (double)__uint_as_float(w4[h][2 * p + u]);
          acc[2 * p + u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bw, acc[2 * p + u], 0, 0, 0);
        }
      }
    }
  }
  // lane l holds rows l / 16 + 4 i of column l % 16
  float *yw = yk + wv * 256;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    yw[(l / 16 + 4 * i) * 16 + l % 16] = (float)(((acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i])) + 0.0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // ---- encode each row's 16 key columns (one FP4 group) ----
  if (l < 16 && valid) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = yw[l * 16 + i];
    uint2 packed;
    uint8_t sb;
    encode_group(v, &packed, &sb);
    *reinterpret_cast<uint2 *>(ik_codes + d * (idx_dim / 2) + ct * 8) = packed;
    ik_scales[d * cgs + ct] = sb;
  }
}

// Compressor (ratio r) fused with the FP4 write.  Entry j is fp32(W_c^T
// [x_rj; ...; x_rj+r-1]) (P4 section 二; P5 section "CSA2注意力": adjacent
// entries do not overlap and no position term is added).  The r token rows
// of entry j are row j of the token buffer viewed as [entries][K], K = r d_in,
// so the compressor is that bf16 matrix times W_c^T.  A product of two bf16
// values is exact in fp64 and v_mfma_f64_16x16x4_f64 accumulates in fp64; the
// sum is rounded once to fp32, like the fp64 product it restates.
//
// grid (ceil(entries / 16), dim / (16 CTC)), 64 KW threads.  A workgroup
// computes 16 entries x 16 CTC channels.  Its KW waves split K in KW slices;
// in a wave, k-slot q = l / 16 of the MFMA walks the q-th quarter of the
// slice in ascending k (8 values per 16-byte load), and lane l supplies the
// token value of row l % 16 and the weight of column l % 16 at that slot's k,
// so every slot pairs operands of the same k.  The slices' partial tiles are
// added in slice order in fp64 and rounded to fp32; each 16-channel column
// tile is one FP4 group, encoded and written to the entry's cache row.
constexpr int kCompressRound = 4;   // 16-byte chunks per operand loaded before use

CSA2_DEV double bf16_elem(const u32x4_t &v, int i) {
  const uint32_t w = v[i / 2];
  return (double)__uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

template <int CTC, int KW>
__global__ __launch_bounds__(64 * KW) void k_compress_fp4(const uint16_t *__restrict__ tokens, int64_t entries,
                                                          int K, const uint16_t *__restrict__ w_c, int dim,
                                                          const int64_t *__restrict__ dst_row,
                                                          uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  __shared__ double part[KW > 1 ? KW * CTC * 256 : 1];
  __shared__ float ent[kDeriveRows * 16 * CTC];
  const int64_t e0 = (int64_t)blockIdx.x * kDeriveRows;
  const int nr = (int)min<int64_t>(kDeriveRows, entries - e0);
  const int l = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = blockIdx.y * 16 * CTC;
  const int kq = K / (4 * KW);                    // k values per lane, a multiple of 8
  const int nch = kq / 8;
  const int kbase = wv * (K / KW) + (l / 16) * kq;
  // rows past the last entry lie outside the resource and read as 0
  const rsrc_t r_x = make_rsrc(tokens + e0 * K, (uint32_t)(nr * K * 2));
  const rsrc_t r_w = make_rsrc(w_c + (int64_t)c0 * K, (uint32_t)(16 * CTC * K * 2));
  const uint32_t xoff = (uint32_t)(((l % 16) * K + kbase) * 2);
  uint32_t woff[CTC];
#pragma unroll
  for (int t = 0; t < CTC; ++t) woff[t] = (uint32_t)(((16 * t + l % 16) * K + kbase) * 2);
  double4_t acc[CTC];
#pragma unroll
  for (int t = 0; t < CTC; ++t) acc[t] = (double4_t){0.0, 0.0, 0.0, 0.0};
  for (int ch0 = 0; ch0 < nch; ch0 += kCompressRound) {
    u32x4_t xa[kCompressRound], wb[kCompressRound][CTC];
#pragma unroll
    for (int c = 0; c < kCompressRound; ++c) {
      const bool in = ch0 + c < nch;
      xa[c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              r_x, in ? xoff + (uint32_t)(ch0 + c) * 16 : kOutOfRange, 0, 0));
#pragma unroll
      for (int t = 0; t < CTC; ++t)
        wb[c][t] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                   r_w, in ? woff[t] + (uint32_t)(ch0 + c) * 16 : kOutOfRange, 0, 0));
    }
    // chunks past the lane's range read as 0 and add +0 (no branch here,
    // so all the round's loads are in flight before the first product)
#pragma unroll
    for (int c = 0; c < kCompressRound; ++c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double a = bf16_elem(xa[c], i);
#pragma unroll
        for (int t = 0; t < CTC; ++t)
          acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bf16_elem(wb[c][t], i), acc[t], 0, 0, 0);
      }
    }
  }
  // lane l holds rows l / 16 + 4 i of column l % 16 of each tile
  constexpr int EW = 16 * CTC;                    // entry tile row stride (floats)
  if constexpr (KW > 1) {
#pragma unroll
    for (int t = 0; t < CTC; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[((wv * CTC + t) * 64 + l) * 4 + i] = acc[t][i];
    __syncthreads();
    for (int t = wv; t < CTC; t += KW) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        double s = 0.0;
        for (int ks = 0; ks < KW; ++ks) s += part[((ks * CTC + t) * 64 + l) * 4 + i];
        ent[(l / 16 + 4 * i) * EW + 16 * t + l % 16] = (float)(s + 0.0);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < CTC; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) ent[(l / 16 + 4 * i) * EW + 16 * t + l % 16] = (float)(acc[t][i] + 0.0);
  }
  __syncthreads();
  for (int u = threadIdx.x; u < nr * CTC; u += 64 * KW) {
    const int rr = u / CTC, g = u - rr * CTC;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = ent[rr * EW + 16 * g + i];
    uint2 packed;
    uint8_t sb;
    encode_group(v, &packed, &sb);
    const int64_t d = dst_row ? dst_row[e0 + rr] : e0 + rr;
    const int gg = c0 / kGroup + g;
    *reinterpret_cast<uint2 *>(codes + d * (dim / 2) + gg * 8) = packed;
    scales[d * (dim / kGroup) + gg] = sb;
  }
}

// FP8 window rows: one workgroup per row.
template <typename T>
__global__ __launch_bounds__(256) void k_quantize_fp8_rows(const T *__restrict__ x, int dim,
                                                            const int64_t *__restrict__ dst_row,
                                                            uint8_t *__restrict__ codes, float *__restrict__ scale) {
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const T *src = x + r * dim;
  float amax = 0.0f;
  for (int c = threadIdx.x; c < dim; c += blockDim.x) amax = fmaxf(amax, fabsf(load_as_f32<T>(src + c)));
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float rs = (amax == 0.0f) ? 1.0f : __fdiv_rn(amax, 448.0f);
  const int64_t d = dst_row ? dst_row[r] : r;
  for (int c = threadIdx.x; c < dim; c += blockDim.x) {
    const float v = load_as_f32<T>(src + c);
    const float y = __fdiv_rn(v, rs);
    const uint32_t code = e4m3_nearest_code(fabsf(y), 1.0f) | ((__float_as_uint(y) >> 31) << 7);
    codes[d * dim + c] = (uint8_t)code;
  }
  if (threadIdx.x == 0) scale[d] = rs;
}

// Decode probe: 8 channels per thread through the same f16 decode the
// indexer and attention kernels use, widened to fp32.
__global__ __launch_bounds__(256) void k_dequant_fp4(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales, int64_t rows, int dim,
                                                      float *__restrict__ out) {
  const int per_row = dim / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * per_row) return;
  const int64_t r = gid / per_row;
  const int k = (int)(gid - r * per_row);
  const uint32_t w = *reinterpret_cast<const uint32_t *>(codes + r * (dim / 2) + k * 4);
  const uint32_t sb = scales[r * (dim / kGroup) + k / 2];
  const _Float16 s = e4m3x2_to_f16(sb)[0];
  const half8_t h = fp4x8_dequant_f16(w, s);
  float4 a = {(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  float4 b = {(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
  float4 *dst = reinterpret_cast<float4 *>(out + r * dim + k * 8);
  dst[0] = a;
  dst[1] = b;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// The fp64-MFMA derive (dim <= kDeriveMaxDim); T = uint8_t: keys of rows already in the cache.
// Clear n16 16-byte words (one per thread).
__global__ __launch_bounds__(256) void k_zero16(uint4 *__restrict__ p, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

static void launch_zero16(uint32_t *zero, int64_t zero_words, hipStream_t stream) {
  const int64_t n16 = zero_words / 4;
  if (n16 > 0)
    hipLaunchKernelGGL(k_zero16, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<uint4 *>(zero), n16);
}

template <typename T>
void derive_mfma(const void *x, int64_t rows, int dim, const int64_t *dst_row, uint8_t *codes, uint8_t *scales,
                 const float *w_ik, int idx_dim, uint8_t *ik_codes, uint8_t *ik_scales, hipStream_t stream,
                 uint32_t *zero = nullptr, int64_t zero_words = 0) {
  // columns per workgroup: the largest tile count (up to 8) dividing the key's 16-column groups
  const int cgs = idx_dim / kGroup;
  const int ct = (cgs % 8 == 0) ? 8 : (cgs % 4 == 0) ? 4 : (cgs % 2 == 0) ? 2 : 1;
  // many rows (dim 64, 128, 256 or 512): the rows are encoded (T = float or
  // bf16) and their keys derived from the cache, 64 rows and one key group
  // per workgroup
  if (rows > 64 && (dim == 64 || dim == 128 || dim == 256 || dim == 512)) {
    if constexpr (!__is_same(T, uint8_t)) {
      const dim3 eg((unsigned)((rows * (dim / kGroup) + 255) / 256));
      CSA2_TIMED_LAUNCH(kTimedWrite, k_quantize_fp4<T>, eg, dim3(256), stream, (const T *)x, rows, dim, dst_row,
                        codes, scales);
    }
    const int64_t nq = ((rows + 63) / 64 + 7) / 8 * 8;
#define CSA2_TILES_LAUNCH(GQ)                                                                                  \
  CSA2_TIMED_LAUNCH(kTimedWrite, (k_derive_tiles<GQ>), dim3((unsigned)(nq * cgs)), dim3(256), stream, rows, dim, \
                    dst_row, codes, scales, w_ik, idx_dim, ik_codes, ik_scales)
    if (dim == 64) CSA2_TILES_LAUNCH(1);
    else if (dim == 128) CSA2_TILES_LAUNCH(2);
    else if (dim == 256) CSA2_TILES_LAUNCH(4);
    else CSA2_TILES_LAUNCH(8);
#undef CSA2_TILES_LAUNCH
    launch_zero16(zero, zero_words, stream);
    return;
  }
  // few rows: split the channels over 8 waves per tile instead (dim % 32 == 0)
  const bool few = rows <= 64 && dim % 32 == 0;
  // spare workgroups past the row tiles clear the zero range: about 32 KB each
  const unsigned gy = (unsigned)(few ? cgs : cgs / ct);
  const int64_t zero_n = zero ? zero_words / 4 : 0;
  const int64_t zx = zero_n > 0 ? std::max<int64_t>(1, zero_n / (2048 * (int64_t)gy)) : 0;
  const dim3 grid((unsigned)((rows + kDeriveRows - 1) / kDeriveRows + zx), gy);
  uint4 *zp = reinterpret_cast<uint4 *>(zero);
#define CSA2_MFMA_LAUNCH(CT, KS)                                                                              \
  CSA2_TIMED_LAUNCH(kTimedWrite, (k_quantize_fp4_derive_mfma<T, CT, KS>), grid, dim3(64 * CT * KS), stream, \
                    (const T *)x, rows, dim, dst_row, codes, scales, w_ik, idx_dim, ik_codes, ik_scales, zp, zero_n)
  if (few) CSA2_MFMA_LAUNCH(1, 8);
  else if (ct == 8) CSA2_MFMA_LAUNCH(8, 1);
  else if (ct == 4) CSA2_MFMA_LAUNCH(4, 1);
  else if (ct == 2) CSA2_MFMA_LAUNCH(2, 1);
  else CSA2_MFMA_LAUNCH(1, 1);
#undef CSA2_MFMA_LAUNCH
}

int launch_quantize_fp4(const void *x, int x_dtype, int64_t rows, int dim, const int64_t *dst_row,
                        uint8_t *codes, uint8_t *scales, const float *w_ik, int idx_dim, uint8_t *ik_codes,
                        uint8_t *ik_scales, hipStream_t stream, uint32_t *zero, int64_t zero_words) {
  if (rows == 0 || !w_ik || dim > kDeriveMaxDim) launch_zero16(zero, zero_words, stream);
  if (rows == 0) return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
  if (!w_ik) {
    const int64_t groups = rows * (dim / kGroup);
    const dim3 grid((unsigned)((groups + 255) / 256));
    if (x_dtype == CSA2_F32)
      CSA2_TIMED_LAUNCH(kTimedWrite, k_quantize_fp4<float>, grid, dim3(256), stream, (const float *)x, rows, dim, dst_row,
                         codes, scales);
    else
      CSA2_TIMED_LAUNCH(kTimedWrite, k_quantize_fp4<uint16_t>, grid, dim3(256), stream, (const uint16_t *)x, rows, dim,
                         dst_row, codes, scales);
  } else if (dim <= kDeriveMaxDim) {
    if (x_dtype == CSA2_F32)
      derive_mfma<float>(x, rows, dim, dst_row, codes, scales, w_ik, idx_dim, ik_codes, ik_scales, stream, zero,
                         zero_words);
    else
      derive_mfma<uint16_t>(x, rows, dim, dst_row, codes, scales, w_ik, idx_dim, ik_codes, ik_scales, stream, zero,
                            zero_words);
  } else {
    const int rb = kDeriveLdsFloats / dim;
    const dim3 grid((unsigned)((rows + rb - 1) / rb));
    const int jm = (rb + 256 / idx_dim - 1) / (256 / idx_dim);  // <= 16 since idx_dim <= dim
#define CSA2_DERIVE_LAUNCH(T, JM)                                                                            \
    CSA2_TIMED_LAUNCH(kTimedWrite, (k_quantize_fp4_derive<T, JM>), grid, dim3(256), stream, (const T *)x, rows, dim, \
                       dst_row, codes, scales, w_ik, idx_dim, ik_codes, ik_scales)
#define CSA2_DERIVE_JM(T)                                                                 \
    if (jm <= 1) CSA2_DERIVE_LAUNCH(T, 1); else if (jm <= 2) CSA2_DERIVE_LAUNCH(T, 2);    \
    else if (jm <= 4) CSA2_DERIVE_LAUNCH(T, 4); else if (jm <= 8) CSA2_DERIVE_LAUNCH(T, 8); \
    else CSA2_DERIVE_LAUNCH(T, 16)
    if (x_dtype == CSA2_F32) { CSA2_DERIVE_JM(float); } else { CSA2_DERIVE_JM(uint16_t); }
#undef CSA2_DERIVE_JM
#undef CSA2_DERIVE_LAUNCH
  }
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

int launch_compress_fp4(const uint16_t *tokens, int64_t entries, int ratio, int d_in, const uint16_t *w_c, int dim,
                        const int64_t *dst_row, uint8_t *codes, uint8_t *scales, const float *w_ik, int idx_dim,
                        uint8_t *ik_codes, uint8_t *ik_scales, hipStream_t stream) {
  if (entries == 0) return CSA2_OK;
  const int K = ratio * d_in;
  // few entries: one FP4 group per workgroup and 8 waves over K (more
  // workgroups and shorter chains); many: 4 groups per workgroup, 4 waves
  const bool few = entries <= 64;
  const int gpr = dim / kGroup;
  const int ctc = few ? 1 : (gpr % 4 == 0) ? 4 : (gpr % 2 == 0) ? 2 : 1;
  int kw = few ? 8 : 4;
  while (K % (32 * kw) != 0) kw /= 2;
  const dim3 grid((unsigned)((entries + kDeriveRows - 1) / kDeriveRows), (unsigned)(gpr / ctc));
#define CSA2_COMPRESS_LAUNCH(CTC, KW)                                                                      \
  CSA2_TIMED_LAUNCH(kTimedCompress, (k_compress_fp4<CTC, KW>), grid, dim3(64 * KW), stream, tokens, entries, K, \
                    w_c, dim, dst_row, codes, scales)
#define CSA2_COMPRESS_KW(CTC)                                                                    \
  if (kw == 8) CSA2_COMPRESS_LAUNCH(CTC, 8); else if (kw == 4) CSA2_COMPRESS_LAUNCH(CTC, 4);     \
  else if (kw == 2) CSA2_COMPRESS_LAUNCH(CTC, 2); else CSA2_COMPRESS_LAUNCH(CTC, 1)
  if (ctc == 4) { CSA2_COMPRESS_KW(4); } else if (ctc == 2) { CSA2_COMPRESS_KW(2); } else { CSA2_COMPRESS_KW(1); }
#undef CSA2_COMPRESS_KW
#undef CSA2_COMPRESS_LAUNCH
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_HIP;
  if (w_ik) derive_mfma<uint8_t>(nullptr, entries, dim, dst_row, codes, scales, w_ik, idx_dim, ik_codes, ik_scales,
                                 stream);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

int launch_quantize_fp8_rows(const void *x, int x_dtype, int64_t rows, int dim, const int64_t *dst_row,
                             uint8_t *codes, float *scale, hipStream_t stream) {
  if (rows == 0) return CSA2_OK;
  const dim3 grid((unsigned)rows);
  if (x_dtype == CSA2_F32)
    hipLaunchKernelGGL(k_quantize_fp8_rows<float>, grid, dim3(256), 0, stream, (const float *)x, dim, dst_row,
                       codes, scale);
  else
    hipLaunchKernelGGL(k_quantize_fp8_rows<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t *)x, dim,
                       dst_row, codes, scale);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

int launch_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int dim, float *out,
                       hipStream_t stream) {
  if (rows == 0) return CSA2_OK;
  const int64_t n = rows * (dim / 8);
  hipLaunchKernelGGL(k_dequant_fp4, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, codes, scales, rows,
                     dim, out);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

}  // namespace csa2
