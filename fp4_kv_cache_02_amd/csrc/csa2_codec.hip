// CSA2 write path: FP4 quantise-on-write of main-KV rows with the indexer key
// derived from each written entry, FP8 window rows, and an FP4 decode probe.
//
// Format (P1 section "FP4 KV、Bounded Replay 及其他扩展"; P4 section 三; P5
// section "缓存精度与持久化分层"): E2M1 elements, one E4M3 scale per 16
// channels, no global scale; the window KV stays FP8.  The indexer key is
// projected from the main-KV entry (P4 section 二; P5 section "CSA2注意力").
#include "csa2_internal.hpp"

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

// Quantise rows and derive their indexer keys for small batches (the decode
// write path): grid (rows, idx_dim / 16), one workgroup per (row, 16-column
// group of the indexer key), 16 * (1024 / idx_dim) threads: thread ->
// (column of the group, slice of PER channels); every W_ik value a thread
// needs is loaded before the fp64 dot products start, each slice sums from
// +0 in channel order and the slices are added in slice order.  Every
// workgroup of a row encodes the row (the exact decoded values feed its dot
// products); the first writes its codes.
constexpr int kRowThreads = 1024;   // (column, slice) pairs per row

template <typename T, int PER>
__global__ __launch_bounds__(512) void k_quantize_fp4_derive_row(const T *__restrict__ x, int dim,
                                                                          const int64_t *__restrict__ dst_row,
                                                                          uint8_t *__restrict__ codes,
                                                                          uint8_t *__restrict__ scales,
                                                                          const float *__restrict__ w_ik,
                                                                          int idx_dim, uint8_t *__restrict__ ik_codes,
                                                                          uint8_t *__restrict__ ik_scales) {
  __shared__ float dq[kDeriveLdsFloats];
  __shared__ double part[512];
  __shared__ float yk[kGroup];
  const int64_t r = blockIdx.x;
  const int cg = blockIdx.y;              // 16-column group of the indexer key
  const int64_t d = dst_row ? dst_row[r] : r;
  const int gpr = dim / kGroup;
  const int col = cg * kGroup + (int)(threadIdx.x % kGroup);
  const int nparts = kRowThreads / idx_dim;
  const int pidx = threadIdx.x / kGroup;
  const int c0 = pidx * PER;              // dim == PER * nparts (checked by the launcher)
  float wv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) wv[i] = w_ik[(int64_t)(c0 + i) * idx_dim + col];
  for (int g = threadIdx.x; g < gpr; g += blockDim.x) {
    float v[16];
    const T *src = x + r * dim + g * kGroup;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = load_as_f32<T>(src + i);
    uint2 packed;
    uint8_t sb;
    encode_group(v, &packed, &sb);
    if (cg == 0) {
      *reinterpret_cast<uint2 *>(codes + d * (dim / 2) + g * 8) = packed;
      scales[d * gpr + g] = sb;
    }
    const float s = e4m3_pos_value(sb);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = (i < 8) ? (packed.x >> (4 * i)) & 15u : (packed.y >> (4 * (i - 8))) & 15u;
      const uint32_t m = c & 7u;
      const float mag = (m < 4) ? 0.5f * (float)m : (float)(1u << ((m - 2) >> 1)) * ((m & 1u) ? 1.5f : 1.0f);
      const float val = mag * s;
      dq[g * kGroup + i] = (c & 8u) ? -val : val;
    }
  }
  __syncthreads();
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < PER; ++i) acc = fma((double)dq[c0 + i], (double)wv[i], acc);
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < kGroup) {
    double t = 0.0;
    for (int k = 0; k < nparts; ++k) t += part[k * kGroup + threadIdx.x];
    yk[threadIdx.x] = (float)t;
  }
  __syncthreads();
  const int igpr = idx_dim / kGroup;
  if (threadIdx.x == 0) {
    const int g = cg;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = yk[i];
    uint2 packed;
    uint8_t sb;
    encode_group(v, &packed, &sb);
    *reinterpret_cast<uint2 *>(ik_codes + d * (idx_dim / 2) + g * 8) = packed;
    ik_scales[d * igpr + g] = sb;
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

int launch_quantize_fp4(const void *x, int x_dtype, int64_t rows, int dim, const int64_t *dst_row,
                        uint8_t *codes, uint8_t *scales, const float *w_ik, int idx_dim, uint8_t *ik_codes,
                        uint8_t *ik_scales, hipStream_t stream) {
  if (rows == 0) return CSA2_OK;
  if (!w_ik) {
    const int64_t groups = rows * (dim / kGroup);
    const dim3 grid((unsigned)((groups + 255) / 256));
    if (x_dtype == CSA2_F32)
      CSA2_TIMED_LAUNCH(kTimedWrite, k_quantize_fp4<float>, grid, dim3(256), stream, (const float *)x, rows, dim, dst_row,
                         codes, scales);
    else
      CSA2_TIMED_LAUNCH(kTimedWrite, k_quantize_fp4<uint16_t>, grid, dim3(256), stream, (const uint16_t *)x, rows, dim,
                         dst_row, codes, scales);
  } else if (rows <= 1024 && dim % (kRowThreads / idx_dim) == 0 &&
             (dim / (kRowThreads / idx_dim) == 8 || dim / (kRowThreads / idx_dim) == 16 ||
              dim / (kRowThreads / idx_dim) == 32 || dim / (kRowThreads / idx_dim) == 64)) {
    const dim3 grid((unsigned)rows, (unsigned)(idx_dim / kGroup));
    const dim3 block((unsigned)(kGroup * (kRowThreads / idx_dim)));  // 64 .. 512
    const int per = dim / (kRowThreads / idx_dim);
#define CSA2_ROW_LAUNCH(T, PERV)                                                                                  \
    CSA2_TIMED_LAUNCH(kTimedWrite, (k_quantize_fp4_derive_row<T, PERV>), grid, block, stream, (const T *)x, dim,             \
                       dst_row, codes, scales, w_ik, idx_dim, ik_codes, ik_scales)
    if (x_dtype == CSA2_F32) {
      if (per == 8) CSA2_ROW_LAUNCH(float, 8); else if (per == 16) CSA2_ROW_LAUNCH(float, 16);
      else if (per == 32) CSA2_ROW_LAUNCH(float, 32); else CSA2_ROW_LAUNCH(float, 64);
    } else {
      if (per == 8) CSA2_ROW_LAUNCH(uint16_t, 8); else if (per == 16) CSA2_ROW_LAUNCH(uint16_t, 16);
      else if (per == 32) CSA2_ROW_LAUNCH(uint16_t, 32); else CSA2_ROW_LAUNCH(uint16_t, 64);
    }
#undef CSA2_ROW_LAUNCH
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
