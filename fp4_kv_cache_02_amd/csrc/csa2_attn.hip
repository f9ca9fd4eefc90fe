// CSA2 per-layer core attention: the selected FP4 main-KV entries
// concatenated with the layer's own FP8 window rows, one joint softmax (P5
// figure caption of the attention diagram: Selection / Top-K /
// Concatenation; P1 CSA2 section: each layer keeps its own query and window
// KV).  Keys double as values (MQA over the shared latent).
//
// Workgroup = (key range, query, block of 64 heads), 4 waves; wave w owns
// heads 16w..16w+15, so the softmax of a head never leaves its wave.  Key
// slots 0..K-1 are the Top-K list, K..K+W-1 the window rows.  Each 64-key
// sub-chunk is decoded once into LDS as a row-major f16 tile [key][dim]:
// S = Q K^T reads it as the MFMA B operand, and O = P V reads it through the
// gfx950 transposing LDS load (ds_read_b64_tr_b16), which hands each lane four
// consecutive keys of one dimension - the B operand of the P V product -
// without a transposed copy.  Both products run on v_mfma_f32_16x16x32_f16.
//
// Exactness: FP4 entries and E4M3 window codes are f16 numbers; bf16 queries
// convert to f16 exactly inside the f16 normal range (|q| in [2^-14, 65504];
// smaller values round to f16 subnormals, larger ones are outside the
// supported input range) and fp32 queries are split into hi + lo f16 parts.
// Window rows carry an fp32 row scale r: it multiplies the
// logits (z = tau * r * q.c) and the probabilities entering P V, where the
// sub-chunk's P is lifted by a power of two 2^S (undone on the accumulator)
// to keep small p * r values out of the f16 subnormal range.  P is rounded
// to f16 (relative error <= 2^-11); everything else accumulates in fp32.
// Several key ranges per query are combined by a log-sum-exp merge kernel.
#include "csa2_internal.hpp"

namespace csa2 {

constexpr int kKC = 64;    // keys per sub-chunk
constexpr int kHB = 64;    // heads per workgroup (4 waves x 16)

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element (i%4)
// of the 8-byte chunks addressed by lanes i/4, i/4+4, i/4+8, i/4+12.
CSA2_DEV short4_t lds_read_tr16(const _Float16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_t *)((__attribute__((address_space(3))) char *)(p)));
}

template <int D, bool QF32>
struct AttnLds {
  static constexpr int KT = D + 8;     // [key][dim] row stride (f16)
  static constexpr int PT = kKC + 8;   // [head][key] row stride of a wave's P tile
  _Float16 kt[kKC * KT];
  _Float16 p[4][16 * PT];
  float kscale[kKC];     // per key: r (window row scale) or 1; 0 = masked
  int64_t koff[kKC];     // per key: byte offset of its FP4 codes (main) or FP8 row (window)
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
  const int c = blockIdx.x, m = blockIdx.y, hb = blockIdx.z;
  const int NC = gridDim.x;
  const int tid = threadIdx.x, l = lane_id(), wv = tid >> 6;
  const int row = l & 15, quad = l >> 4;
  const int nk = K + W;
  const int slot_lo = c * span, slot_hi = min(nk, (c + 1) * span);
  const int h0 = hb * kHB + 16 * wv;        // first head of this wave
  const bool wave_active = h0 < H;

  const int s = q_seq[m];
  const int64_t lim = ((int64_t)q_pos[m] + 1) / ratio;
  const int64_t vis = max<int64_t>(0, min<int64_t>(seq_len[s], lim));
  const int64_t row0 = seq_start[s];
  const int wcount = min(swa_count[m], W);
  const int64_t wstart = swa_start[m];

  // ---- this wave's queries as MFMA A operands (registers) ----
  // lane (head row, quad) holds dims 32*kk + 8*quad .. +7 for kk = 0 .. D/32-1.
  // bf16 queries convert to f16 directly (exact inside the f16 normal range);
  // fp32 queries are split into hi + lo f16 parts.
  constexpr int NK = D / 32;
  half8_t qa[NK];
  half8_t qb[QF32 ? NK : 1];
  // log2-domain softmax: z2 = log2(e) * tau * q.k, p = 2^(z2 - max)
  const float tau2 = softmax_scale * 1.4426950408889634f;
  {
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

  float m_run[4], l_run[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.0f; }
  constexpr int NCT = D / 16;  // 16-dim output tiles per wave
  float4_t o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o_acc[ct] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  int e_cur = 0;  // accumulator exponent: true O = o_acc * 2^-e_cur
  _Float16 *pw = L.p[wv];

  for (int sub = slot_lo; sub < slot_hi; sub += kKC) {
    __syncthreads();  // previous sub-chunk's LDS reads are done
    // ---- per-key validity, scale and source offset (wave 0) ----
    if (tid < kKC) {
      const int slot = sub + tid;
      float ks = 0.0f;
      int64_t off = 0;
      if (slot < slot_hi) {
        if (slot < K) {
          const int32_t j = topk[(int64_t)m * K + slot];
          if (j >= 0 && j < vis) { ks = 1.0f; off = row0 + j; }
        } else if (slot - K < wcount) {
          off = wstart + (slot - K);
          ks = swa_scale[off];
        }
      }
      L.kscale[tid] = ks;
      L.koff[tid] = off;
      float rm = ks;
      for (int o = 32; o > 0; o >>= 1) rm = fmaxf(rm, __shfl_xor(rm, o, 64));
      if (tid == 0) L.rmax = rm;
    }
    __syncthreads();
    // ---- decode 64 keys into kt[key][dim]; a wave covers contiguous groups of one row ----
    constexpr int G8 = D / 8;
    constexpr int ITEMS = kKC * G8 / 256;
    constexpr int BATCH = ITEMS < 8 ? ITEMS : 8;   // loads in flight per thread
#pragma unroll
    for (int i0 = 0; i0 < ITEMS; i0 += BATCH) {
      half8_t vals[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int item = tid + 256 * (i0 + u);
        const int key = item / G8, g = item % G8;
        const int slot = sub + key;
        const float ks = L.kscale[key];
        const int64_t r = L.koff[key];
        half8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (ks != 0.0f) {
          if (slot < K) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(kv_codes + r * (D / 2) + g * 4);
            const uint32_t sb = kv_scales[r * (D / 16) + (g >> 1)];
            v = fp4x8_dequant_f16(w, e4m3x2_to_f16(sb)[0]);
          } else {
            const uint2 w = *reinterpret_cast<const uint2 *>(swa_codes + r * D + g * 8);
            const half2_t a0 = e4m3x2_to_f16(w.x), a1 = e4m3x2_to_f16(w.x >> 16);
            const half2_t a2 = e4m3x2_to_f16(w.y), a3 = e4m3x2_to_f16(w.y >> 16);
            v = (half8_t){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
          }
        }
        vals[u] = v;
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int item = tid + 256 * (i0 + u);
        const int key = item / G8, g = item % G8;
        *reinterpret_cast<half8_t *>(&L.kt[key * L.KT + g * 8]) = vals[u];
      }
    }
    __syncthreads();
    if (!wave_active) continue;

    // ---- S = Q K^T for 16 heads x 64 keys (4 key tiles) ----
    float4_t sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) sacc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const half8_t b = *reinterpret_cast<const half8_t *>(&L.kt[(16 * t + row) * L.KT + 32 * kk + 8 * quad]);
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kk], b, sacc[t], 0, 0, 0);
        if constexpr (QF32) sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qb[kk], b, sacc[t], 0, 0, 0);
      }
    }
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
    // transposing-read addresses: lane i of the quad group supplies key 8*quad + 4*h + i/4, dims 4*(i%4)..
    const int tr_key = 8 * quad + (row >> 2);
    const int tr_dim = 4 * (row & 3);
    const bool first = sub == slot_lo;   // accumulator still zero: no rescale
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (!first) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o_acc[ct][j] *= alpha[j];
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const _Float16 *base = &L.kt[(32 * kk + tr_key) * L.KT + 16 * ct + tr_dim];
        const short4_t lo = lds_read_tr16(base);
        const short4_t hi = lds_read_tr16(base + 4 * L.KT);
        const short8_t s8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const half8_t b = __builtin_bit_cast(half8_t, s8);
        o_acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kk ? pa1 : pa0, b, o_acc[ct], 0, 0, 0);
      }
    }
  }

  if (!wave_active) return;
  // ---- write o (normalised) and lse for this key range ----
  const int64_t obase = (NC == 1) ? (int64_t)m * H : ((int64_t)m * NC + c) * H;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = h0 + 4 * quad + j;
    if (h >= H) continue;
    const float inv = (l_run[j] > 0.0f) ? ldexpf(1.0f / l_run[j], -e_cur) : 0.0f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) out[(obase + h) * D + 16 * ct + row] = o_acc[ct][j] * inv;
    if (row == 0 && lse)
      lse[obase + h] = (l_run[j] > 0.0f) ? (m_run[j] + log2f(l_run[j])) * 0.6931471805599453f : -INFINITY;
  }
}

// Log-sum-exp merge of NC partial results: grid (m, heads), D threads.  All
// partial values are loaded before they are combined.
constexpr int kMaxSplits = 32;

template <int D>
__global__ __launch_bounds__(D) void k_attn_merge(const float *__restrict__ po, const float *__restrict__ plse,
                                                  int NC, int H, float *__restrict__ out, float *__restrict__ lse) {
  const int m = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  float lc[kMaxSplits], oc[kMaxSplits];
#pragma unroll
  for (int c = 0; c < kMaxSplits; ++c) {
    if (c < NC) {
      lc[c] = plse[((int64_t)m * NC + c) * H + h];
      oc[c] = po[(((int64_t)m * NC + c) * H + h) * D + d];
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < kMaxSplits; ++c)
    if (c < NC) mx = fmaxf(mx, lc[c]);
  float acc = 0.0f, wsum = 0.0f;
  if (mx > -INFINITY) {
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c) {
      if (c < NC) {
        const float wc = (lc[c] == -INFINITY) ? 0.0f : expf(lc[c] - mx);
        wsum += wc;
        acc = fmaf(wc, oc[c], acc);
      }
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
  const int base = m * ((heads + kHB - 1) / kHB);
  int nc = (512 + base - 1) / base;
  if (nc > nsub) nc = nsub;
  if (nc > kMaxSplits) nc = kMaxSplits;
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
  const dim3 grid(ncu, qs.m, (heads + kHB - 1) / kHB);
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
