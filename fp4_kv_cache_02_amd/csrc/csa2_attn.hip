// CSA2 per-layer core attention: the selected FP4 main-KV entries
// concatenated with the layer's own FP8 window rows, one joint softmax (P5
// figure caption of the attention diagram: Selection / Top-K /
// Concatenation; P1 CSA2 section: each layer keeps its own query and window
// KV).  Keys double as values (MQA over the shared latent).
//
// Workgroup = (key range, query, group of 16 heads), 4 waves.  Key slots
// 0..K-1 are the Top-K list, K..K+W-1 the window rows.  Each 64-key
// sub-chunk is decoded into LDS as f16 twice - [key][dim] for S = Q K^T and
// [dim][key] for O = P V - both products on v_mfma_f32_16x16x32_f16.
//
// Exactness: FP4 entries and E4M3 window codes are f16 numbers; each head's
// query is scaled by a power of two into f16 range (fp32 queries are split
// into hi + lo f16 parts) and the inverse power of two is folded into the
// softmax scale.  Window rows carry an fp32 row scale r: it multiplies the
// logits (z = tau * r * q.c) and the probabilities entering P V, where the
// sub-chunk's P is lifted by a power of two 2^S (undone on the accumulator)
// to keep small p * r values out of the f16 subnormal range.  P is rounded
// to f16 (relative error <= 2^-11); everything else accumulates in fp32.
// Several key ranges per query are combined by a log-sum-exp merge kernel.
#include "csa2_internal.hpp"

namespace csa2 {

constexpr int kKC = 64;    // keys per sub-chunk
constexpr int kHG = 16;    // heads per workgroup

template <int D, bool QF32>
struct AttnLds {
  static constexpr int KT = D + 8;     // [key][dim] row stride (f16)
  static constexpr int VT = kKC + 8;   // [dim][key] row stride
  static constexpr int QS = D + 8;
  _Float16 kt[kKC * KT];
  _Float16 vt[D * VT];
  _Float16 qh[kHG * QS];
  _Float16 ql[QF32 ? kHG * QS : 8];
  _Float16 p[kHG * VT];
  float kscale[kKC];     // per key: r (window row scale) or 1; 0 = masked
  float red[4][kHG];
  float tau[kHG];
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
                                              const int32_t *__restrict__ swa_count, int W, float softmax_scale,
                                              int span, float *__restrict__ out, float *__restrict__ lse) {
  __shared__ AttnLds<D, QF32> L;
  const int c = blockIdx.x, m = blockIdx.y, hg = blockIdx.z;
  const int NC = gridDim.x;
  const int tid = threadIdx.x, l = lane_id(), wv = tid >> 6;
  const int row = l & 15, quad = l >> 4;
  const int nk = K + W;
  const int slot_lo = c * span, slot_hi = min(nk, (c + 1) * span);

  int s;
  const int64_t lim = ((int64_t)q_pos[m] + 1) / ratio;
  s = q_seq[m];
  const int64_t vis = max<int64_t>(0, min<int64_t>(seq_len[s], lim));
  const int64_t row0 = seq_start[s];
  const int wcount = min(swa_count[m], W);
  const int64_t wstart = swa_start[m];

  // ---- queries: power-of-two scaling per head, into LDS as f16 ----
  {
    const int r = tid >> 4, part = tid & 15;  // 16 threads per head row
    const int h = hg * kHG + r;
    constexpr int PER = D / 16;
    float mx = 0.0f;
    if (h < H) {
      for (int i = 0; i < PER; ++i) {
        const int64_t off = ((int64_t)m * H + h) * D + part * PER + i;
        const float v = QF32 ? reinterpret_cast<const float *>(q_any)[off]
                             : bf16_to_f32(reinterpret_cast<const uint16_t *>(q_any)[off]);
        mx = fmaxf(mx, fabsf(v));
      }
    }
    mx = max16_lanes(mx);
    int e = 0;
    (void)frexpf(mx, &e);
    const int kf = (mx > 0.0f) ? 15 - e : 0;
    for (int i = 0; i < PER; ++i) {
      const int d = part * PER + i;
      float v = 0.0f;
      if (h < H) {
        const int64_t off = ((int64_t)m * H + h) * D + d;
        v = QF32 ? reinterpret_cast<const float *>(q_any)[off]
                 : bf16_to_f32(reinterpret_cast<const uint16_t *>(q_any)[off]);
      }
      const float vs = ldexpf(v, kf);
      const _Float16 hi = (_Float16)vs;
      L.qh[r * L.QS + d] = hi;
      if constexpr (QF32) L.ql[r * L.QS + d] = (_Float16)(vs - (float)hi);
    }
    if (part == 0) L.tau[r] = ldexpf(softmax_scale, -kf);
  }

  float m_run[4], l_run[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.0f; }
  constexpr int NCT = D / 64;  // 16-dim output tiles per wave
  float4_t o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o_acc[ct] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  int e_cur = 0;  // accumulator exponent: true O = o_acc * 2^-e_cur

  for (int sub = slot_lo; sub < slot_hi; sub += kKC) {
    __syncthreads();  // previous sub-chunk's LDS reads are done
    // ---- decode 64 keys into [key][dim] and [dim][key] ----
    if (tid < kKC) {
      const int slot = sub + tid;
      float ks = 0.0f;
      if (slot < slot_hi) {
        if (slot < K) {
          const int32_t j = topk[(int64_t)m * K + slot];
          ks = (j >= 0 && j < vis) ? 1.0f : 0.0f;
        } else {
          ks = (slot - K < wcount) ? swa_scale[wstart + (slot - K)] : 0.0f;
        }
      }
      L.kscale[tid] = ks;
    }
    __syncthreads();
    if (tid == 0) {
      float rm = 0.0f;
      for (int i = 0; i < kKC; ++i) rm = fmaxf(rm, L.kscale[i]);
      L.rmax = rm;
    }
    constexpr int G8 = D / 8;
    for (int item = tid; item < kKC * G8; item += 256) {
      const int key = item & (kKC - 1), g = item >> 6;
      const int slot = sub + key;
      half8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
      const float ks = L.kscale[key];
      if (ks != 0.0f) {
        if (slot < K) {
          const int64_t r = row0 + topk[(int64_t)m * K + slot];
          const uint32_t w = *reinterpret_cast<const uint32_t *>(kv_codes + r * (D / 2) + g * 4);
          const uint32_t sb = kv_scales[r * (D / 16) + (g >> 1)];
          v = fp4x8_dequant_f16(w, e4m3x2_to_f16(sb)[0]);
        } else {
          const int64_t r = wstart + (slot - K);
          const uint2 w = *reinterpret_cast<const uint2 *>(swa_codes + r * D + g * 8);
          const half2_t a0 = e4m3x2_to_f16(w.x), a1 = e4m3x2_to_f16(w.x >> 16);
          const half2_t a2 = e4m3x2_to_f16(w.y), a3 = e4m3x2_to_f16(w.y >> 16);
          v = (half8_t){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
        }
      }
      *reinterpret_cast<half8_t *>(&L.kt[key * L.KT + g * 8]) = v;
#pragma unroll
      for (int i = 0; i < 8; ++i) L.vt[(g * 8 + i) * L.VT + key] = v[i];
    }
    __syncthreads();

    // ---- S = Q K^T for keys 16*wv .. +15 ----
    float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
    const int kcol = 16 * wv + row;
#pragma unroll 4
    for (int kk = 0; kk < D / 32; ++kk) {
      const half8_t b = *reinterpret_cast<const half8_t *>(&L.kt[kcol * L.KT + 32 * kk + 8 * quad]);
      const half8_t a = *reinterpret_cast<const half8_t *>(&L.qh[row * L.QS + 32 * kk + 8 * quad]);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, sacc, 0, 0, 0);
      if constexpr (QF32) {
        const half8_t a2 = *reinterpret_cast<const half8_t *>(&L.ql[row * L.QS + 32 * kk + 8 * quad]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, b, sacc, 0, 0, 0);
      }
    }
    // lane: key column kcol, head rows 4*quad + j
    const float kscale = L.kscale[kcol];
    float z[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = (kscale != 0.0f) ? sacc[j] * L.tau[4 * quad + j] * kscale : -INFINITY;
    float cm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cm[j] = max16_lanes(z[j]);
    if (row == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) L.red[wv][4 * quad + j] = cm[j];
    }
    __syncthreads();
    float mnew[4], alpha[4], p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * quad + j;
      const float cmax = fmaxf(fmaxf(L.red[0][h], L.red[1][h]), fmaxf(L.red[2][h], L.red[3][h]));
      mnew[j] = fmaxf(m_run[j], cmax);
      if (mnew[j] == -INFINITY) {
        alpha[j] = 1.0f;
        p[j] = 0.0f;
      } else {
        alpha[j] = expf(m_run[j] - mnew[j]);
        p[j] = (z[j] == -INFINITY) ? 0.0f : expf(z[j] - mnew[j]);
      }
    }
    __syncthreads();  // everyone read L.red
    float ps[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ps[j] = sum16_lanes(p[j]);
    if (row == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) L.red[wv][4 * quad + j] = ps[j];
    }
    // P' = p * r * 2^S into LDS [head][key]
    int e_new = 0;
    (void)frexpf(L.rmax, &e_new);
    e_new = (L.rmax > 0.0f) ? 1 - e_new : 0;  // rmax * 2^e_new in [1, 2)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      L.p[(4 * quad + j) * L.VT + kcol] = (_Float16)ldexpf(p[j] * kscale, e_new);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * quad + j;
      const float tot = L.red[0][h] + L.red[1][h] + L.red[2][h] + L.red[3][h];
      l_run[j] = alpha[j] * l_run[j] + tot;
      m_run[j] = mnew[j];
      alpha[j] = ldexpf(alpha[j], e_new - e_cur);
    }
    e_cur = e_new;

    // ---- O += P V for dims [wv*D/4, (wv+1)*D/4) ----
    const half8_t pa0 = *reinterpret_cast<const half8_t *>(&L.p[row * L.VT + 8 * quad]);
    const half8_t pa1 = *reinterpret_cast<const half8_t *>(&L.p[row * L.VT + 32 + 8 * quad]);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int dcol = wv * (D / 4) + 16 * ct + row;
#pragma unroll
      for (int j = 0; j < 4; ++j) o_acc[ct][j] *= alpha[j];
      const half8_t b0 = *reinterpret_cast<const half8_t *>(&L.vt[dcol * L.VT + 8 * quad]);
      const half8_t b1 = *reinterpret_cast<const half8_t *>(&L.vt[dcol * L.VT + 32 + 8 * quad]);
      o_acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa0, b0, o_acc[ct], 0, 0, 0);
      o_acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa1, b1, o_acc[ct], 0, 0, 0);
    }
  }

  // ---- write o (normalised) and lse for this key range ----
  const int64_t obase = (NC == 1) ? (int64_t)m * H : ((int64_t)m * NC + c) * H;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = hg * kHG + 4 * quad + j;
    if (h >= H) continue;
    const float inv = (l_run[j] > 0.0f) ? ldexpf(1.0f / l_run[j], -e_cur) : 0.0f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int d = wv * (D / 4) + 16 * ct + row;
      out[(obase + h) * D + d] = o_acc[ct][j] * inv;
    }
    if (row == 0 && wv == 0 && lse)
      lse[obase + h] = (l_run[j] > 0.0f) ? m_run[j] + logf(l_run[j]) : -INFINITY;
  }
}

// Log-sum-exp merge of NC partial results: grid (m, heads), D threads.
template <int D>
__global__ __launch_bounds__(D) void k_attn_merge(const float *__restrict__ po, const float *__restrict__ plse,
                                                  int NC, int H, float *__restrict__ out, float *__restrict__ lse) {
  const int m = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  float mx = -INFINITY;
  for (int c = 0; c < NC; ++c) mx = fmaxf(mx, plse[((int64_t)m * NC + c) * H + h]);
  float acc = 0.0f, wsum = 0.0f;
  if (mx > -INFINITY) {
    for (int c = 0; c < NC; ++c) {
      const float lc = plse[((int64_t)m * NC + c) * H + h];
      const float wc = (lc == -INFINITY) ? 0.0f : expf(lc - mx);
      wsum += wc;
      acc = fmaf(wc, po[(((int64_t)m * NC + c) * H + h) * D + d], acc);
    }
  }
  out[((int64_t)m * H + h) * D + d] = (wsum > 0.0f) ? acc / wsum : 0.0f;
  if (d == 0 && lse) lse[(int64_t)m * H + h] = (wsum > 0.0f) ? mx + logf(wsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static int attn_splits(int m, int heads, int top_k, int window) {
  const int nsub = (top_k + window + kKC - 1) / kKC;
  const int base = m * ((heads + kHG - 1) / kHG);
  int nc = (512 + base - 1) / base;
  if (nc > nsub) nc = nsub;
  if (nc < 1) nc = 1;
  return nc;
}

size_t attn_ws_bytes(int m, int heads, int dim, int top_k, int window) {
  const int nc = attn_splits(m, heads, top_k, window);
  if (nc == 1) return 256;
  return align256(sizeof(float) * (size_t)m * nc * heads * dim) + align256(sizeof(float) * (size_t)m * nc * heads);
}

template <int D, bool QF32>
static int attn_impl(const csa2_fp4_cache &kv, const csa2_queries &qs, const void *q, int heads,
                     const int32_t *topk, int K, const csa2_swa &swa, float scale, float *out, float *lse, void *ws,
                     hipStream_t stream) {
  const int W = swa.window;
  const int nc = attn_splits(qs.m, heads, K, W);
  const int nsub = (K + W + kKC - 1) / kKC;
  const int span = ((nsub + nc - 1) / nc) * kKC;
  const int ncu = (K + W + span - 1) / span;  // ranges actually used
  const dim3 grid(ncu, qs.m, (heads + kHG - 1) / kHG);
  float *po = out, *pl = lse;
  if (ncu > 1) {
    po = static_cast<float *>(ws);
    pl = reinterpret_cast<float *>(static_cast<char *>(ws) + align256(sizeof(float) * (size_t)qs.m * ncu * heads * D));
  }
  hipLaunchKernelGGL((k_attn<D, QF32>), grid, dim3(256), 0, stream, q, heads, kv.codes, kv.scales, kv.seq_start,
                     kv.seq_len, kv.ratio, qs.seq, qs.pos, topk, K, swa.codes, swa.scale, swa.start, swa.count, W,
                     scale, span, po, pl);
  if (ncu > 1)
    hipLaunchKernelGGL(k_attn_merge<D>, dim3(qs.m, heads), dim3(D), 0, stream, po, pl, ncu, heads, out, lse);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

int launch_attn(const csa2_fp4_cache &kv, const csa2_queries &qs, const void *q, int q_dtype, int heads,
                const int32_t *topk, int top_k, const csa2_swa &swa, float scale, float *out, float *lse, void *ws,
                hipStream_t stream) {
  const bool f32 = q_dtype == CSA2_F32;
  switch (kv.dim) {
    case 64: return f32 ? attn_impl<64, true>(kv, qs, q, heads, topk, top_k, swa, scale, out, lse, ws, stream)
                        : attn_impl<64, false>(kv, qs, q, heads, topk, top_k, swa, scale, out, lse, ws, stream);
    case 128: return f32 ? attn_impl<128, true>(kv, qs, q, heads, topk, top_k, swa, scale, out, lse, ws, stream)
                         : attn_impl<128, false>(kv, qs, q, heads, topk, top_k, swa, scale, out, lse, ws, stream);
    case 256: return f32 ? attn_impl<256, true>(kv, qs, q, heads, topk, top_k, swa, scale, out, lse, ws, stream)
                         : attn_impl<256, false>(kv, qs, q, heads, topk, top_k, swa, scale, out, lse, ws, stream);
    case 512: return f32 ? CSA2_ERR_UNSUPPORTED
                         : attn_impl<512, false>(kv, qs, q, heads, topk, top_k, swa, scale, out, lse, ws, stream);
    default: return CSA2_ERR_UNSUPPORTED;
  }
}

}  // namespace csa2
