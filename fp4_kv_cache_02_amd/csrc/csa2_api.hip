// C ABI of the CSA2 hot path: host-side validation, workspace sizing and
// dispatch.  Every check runs before anything is enqueued.
#include "csa2_internal.hpp"

#include <vector>

using namespace csa2;

// ---------------------------------------------------------------------------
// kernel timing records: first scans and attention launches
// ---------------------------------------------------------------------------
namespace csa2 {
namespace {
struct Timing {
  bool on = false;
  std::vector<hipEvent_t> events;   // begin/end pairs in launch order
};
Timing g_timing[2];                 // 0: first scan, 1: attention

void clear_events(Timing &t) {
  for (hipEvent_t e : t.events) (void)hipEventDestroy(e);
  t.events.clear();
}
int read_events(Timing &t, double *total_ms, int64_t *launches) {
  if (!total_ms || !launches) return CSA2_ERR_NULL_ARG;
  double tot = 0.0;
  int64_t n = 0;
  for (size_t i = 0; i + 1 < t.events.size(); i += 2) {
    if (hipEventSynchronize(t.events[i + 1]) != hipSuccess) return CSA2_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, t.events[i], t.events[i + 1]) != hipSuccess) return CSA2_ERR_HIP;
    tot += ms;
    ++n;
  }
  clear_events(t);
  *total_ms = tot;
  *launches = n;
  return CSA2_OK;
}
}  // namespace

void timing_events(int which, hipEvent_t *start, hipEvent_t *stop) {
  *start = *stop = nullptr;
  Timing &t = g_timing[which];
  if (!t.on) return;
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess) return;
  if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
  t.events.push_back(a);
  t.events.push_back(b);
  *start = a;
  *stop = b;
}
}  // namespace csa2

namespace {

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_cache(const csa2_fp4_cache *c, bool need_dim32) {
  if (!c) return CSA2_ERR_NULL_ARG;
  if (!c->codes || !c->scales || !c->seq_start || !c->seq_len) return CSA2_ERR_NULL_ARG;
  if (c->n_seq <= 0 || c->dim <= 0 || c->max_len < 0 || c->ratio < 1) return CSA2_ERR_BAD_SHAPE;
  if (need_dim32 && c->dim % 32 != 0) return CSA2_ERR_BAD_SHAPE;
  if (!aligned(c->codes, 16)) return CSA2_ERR_MISALIGNED;
  return CSA2_OK;
}

int check_queries(const csa2_queries *q) {
  if (!q) return CSA2_ERR_NULL_ARG;
  if (q->m < 0) return CSA2_ERR_BAD_SHAPE;
  if (q->m > 0 && (!q->seq || !q->pos)) return CSA2_ERR_NULL_ARG;
  if (q->m > 65535) return CSA2_ERR_UNSUPPORTED;
  return CSA2_OK;
}

int check_index_common(const csa2_fp4_cache *idx, const csa2_queries *qs, const uint16_t *q_idx,
                       const float *w_idx, int heads, int top_k, const int32_t *topk_out) {
  int st = check_cache(idx, true);
  if (st) return st;
  if ((st = check_queries(qs))) return st;
  if (qs->m > 0 && (!q_idx || !w_idx || !topk_out)) return CSA2_ERR_NULL_ARG;
  if (heads < 1 || top_k < 1) return CSA2_ERR_BAD_SHAPE;
  if (heads > 16 || top_k > 2048) return CSA2_ERR_UNSUPPORTED;
  if (idx->dim != 64 && idx->dim != 128 && idx->dim != 256) return CSA2_ERR_UNSUPPORTED;
  return CSA2_OK;
}

size_t index_bytes(const csa2_fp4_cache *idx, int m, int pool_blocks, int top_k) {
  if (pool_blocks == 0) return flat_ws_bytes(idx->max_len, m, top_k);
  return index_ws_layout(idx->max_len, m, pool_blocks, top_k).total;
}

int check_swa(const csa2_swa *swa, int dim) {
  if (!swa) return CSA2_ERR_NULL_ARG;
  if (swa->window < 0) return CSA2_ERR_BAD_SHAPE;
  if (swa->window > 1024) return CSA2_ERR_UNSUPPORTED;
  if (swa->window > 0) {
    if (!swa->codes || !swa->scale || !swa->start || !swa->count) return CSA2_ERR_NULL_ARG;
    if (swa->dim != dim) return CSA2_ERR_BAD_SHAPE;
    if (!aligned(swa->codes, 16)) return CSA2_ERR_MISALIGNED;
  }
  return CSA2_OK;
}

}  // namespace

extern "C" {

int32_t csa2_abi_version(void) { return CSA2_ABI_VERSION; }

const char *csa2_status_string(int32_t status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL_ARG: return "null argument";
    case CSA2_ERR_BAD_SHAPE: return "bad shape";
    case CSA2_ERR_BAD_DTYPE: return "bad dtype";
    case CSA2_ERR_MISALIGNED: return "misaligned pointer";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_UNSUPPORTED: return "unsupported configuration";
    case CSA2_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int32_t csa2_quantize_fp4(const void *x, int32_t x_dtype, int64_t rows, int32_t dim, const int64_t *dst_row,
                          uint8_t *codes, uint8_t *scales, const float *w_ik, int32_t idx_dim, uint8_t *ik_codes,
                          uint8_t *ik_scales, void *stream) {
  if (rows < 0 || dim <= 0 || dim % 32 != 0 || dim > 4096) return CSA2_ERR_BAD_SHAPE;
  if (x_dtype != CSA2_F32 && x_dtype != CSA2_BF16) return CSA2_ERR_BAD_DTYPE;
  if (rows == 0) return CSA2_OK;
  if (!x || !codes || !scales) return CSA2_ERR_NULL_ARG;
  if (!aligned(codes, 8)) return CSA2_ERR_MISALIGNED;
  if (w_ik) {
    if (!ik_codes || !ik_scales) return CSA2_ERR_NULL_ARG;
    if (idx_dim != 32 && idx_dim != 64 && idx_dim != 128 && idx_dim != 256) return CSA2_ERR_UNSUPPORTED;
    if (idx_dim > dim) return CSA2_ERR_UNSUPPORTED;
    if (!aligned(ik_codes, 8)) return CSA2_ERR_MISALIGNED;
  }
  return launch_quantize_fp4(x, x_dtype, rows, dim, dst_row, codes, scales, w_ik, idx_dim, ik_codes, ik_scales,
                             (hipStream_t)stream);
}

int32_t csa2_quantize_fp8_rows(const void *x, int32_t x_dtype, int64_t rows, int32_t dim, const int64_t *dst_row,
                               uint8_t *codes, float *scale, void *stream) {
  if (rows < 0 || dim <= 0 || dim % 16 != 0) return CSA2_ERR_BAD_SHAPE;
  if (x_dtype != CSA2_F32 && x_dtype != CSA2_BF16) return CSA2_ERR_BAD_DTYPE;
  if (rows == 0) return CSA2_OK;
  if (rows > 0x7FFFFFFF) return CSA2_ERR_UNSUPPORTED;
  if (!x || !codes || !scale) return CSA2_ERR_NULL_ARG;
  return launch_quantize_fp8_rows(x, x_dtype, rows, dim, dst_row, codes, scale, (hipStream_t)stream);
}

int32_t csa2_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int32_t dim, float *out,
                         void *stream) {
  if (rows < 0 || dim <= 0 || dim % 32 != 0) return CSA2_ERR_BAD_SHAPE;
  if (rows == 0) return CSA2_OK;
  if (!codes || !scales || !out) return CSA2_ERR_NULL_ARG;
  if (!aligned(codes, 4) || !aligned(out, 16)) return CSA2_ERR_MISALIGNED;
  return launch_dequant_fp4(codes, scales, rows, dim, out, (hipStream_t)stream);
}

int32_t csa2_index_workspace_size(const csa2_fp4_cache *idx, int32_t m, int32_t pool_blocks, int32_t top_k,
                                  size_t *bytes) {
  if (!idx || !bytes) return CSA2_ERR_NULL_ARG;
  if (m < 0 || pool_blocks < 0 || top_k < 1 || idx->max_len < 0) return CSA2_ERR_BAD_SHAPE;
  if (pool_blocks > 4096 || top_k > 2048) return CSA2_ERR_UNSUPPORTED;
  *bytes = index_bytes(idx, m, pool_blocks, top_k);
  return CSA2_OK;
}

int32_t csa2_index_full(const csa2_fp4_cache *idx, const csa2_queries *qs, const uint16_t *q_idx,
                        const float *w_idx, int32_t idx_heads, int32_t pool_blocks, int32_t top_k,
                        int32_t *pool_out, int32_t *pool_count, int32_t *topk_out, float *topk_score,
                        void *workspace, size_t ws_bytes, void *stream) {
  int st = check_index_common(idx, qs, q_idx, w_idx, idx_heads, top_k, topk_out);
  if (st) return st;
  if (pool_blocks < 0) return CSA2_ERR_BAD_SHAPE;
  if (pool_blocks > 4096) return CSA2_ERR_UNSUPPORTED;
  if (pool_blocks > 0 && qs->m > 0 && (!pool_out || !pool_count)) return CSA2_ERR_NULL_ARG;
  if (qs->m == 0) return CSA2_OK;
  if (!workspace || ws_bytes < index_bytes(idx, qs->m, pool_blocks, top_k)) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_MISALIGNED;
  if (pool_blocks == 0)
    return launch_index_flat(*idx, *qs, q_idx, w_idx, idx_heads, top_k, topk_out, topk_score, workspace,
                             (hipStream_t)stream);
  return launch_index_full(*idx, *qs, q_idx, w_idx, idx_heads, pool_blocks, top_k, pool_out, pool_count, topk_out,
                           topk_score, workspace, (hipStream_t)stream);
}

int32_t csa2_reindex(const csa2_fp4_cache *idx, const csa2_queries *qs, const uint16_t *q_idx, const float *w_idx,
                     int32_t idx_heads, const int32_t *pool_in, const int32_t *pool_count, int32_t pool_blocks,
                     int32_t top_k, int32_t *topk_out, float *topk_score, void *workspace, size_t ws_bytes,
                     void *stream) {
  int st = check_index_common(idx, qs, q_idx, w_idx, idx_heads, top_k, topk_out);
  if (st) return st;
  if (pool_blocks < 1) return CSA2_ERR_BAD_SHAPE;
  if (pool_blocks > 4096) return CSA2_ERR_UNSUPPORTED;
  if (qs->m > 0 && (!pool_in || !pool_count)) return CSA2_ERR_NULL_ARG;
  if (qs->m == 0) return CSA2_OK;
  if (!workspace || ws_bytes < index_bytes(idx, qs->m, pool_blocks, top_k)) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_MISALIGNED;
  return launch_reindex(*idx, *qs, q_idx, w_idx, idx_heads, pool_in, pool_count, pool_blocks, top_k, topk_out,
                        topk_score, workspace, (hipStream_t)stream);
}

int32_t csa2_attn_workspace_size(int32_t m, int32_t heads, int32_t dim, int32_t top_k, int32_t window,
                                 size_t *bytes) {
  if (!bytes) return CSA2_ERR_NULL_ARG;
  if (m < 0 || heads < 1 || dim <= 0 || top_k < 0 || window < 0) return CSA2_ERR_BAD_SHAPE;
  *bytes = (m == 0) ? 256 : attn_ws_bytes(m, heads, dim, top_k, window);
  return CSA2_OK;
}

int32_t csa2_sparse_swa_attn(const csa2_fp4_cache *kv, const csa2_queries *qs, const void *q, int32_t q_dtype,
                             int32_t heads, const int32_t *topk, int32_t top_k, const csa2_swa *swa,
                             float softmax_scale, float *out, float *lse, void *workspace, size_t ws_bytes,
                             void *stream) {
  int st = check_cache(kv, true);
  if (st) return st;
  if ((st = check_queries(qs))) return st;
  if ((st = check_swa(swa, kv->dim))) return st;
  if (q_dtype != CSA2_F32 && q_dtype != CSA2_BF16) return CSA2_ERR_BAD_DTYPE;
  if (heads < 1 || top_k < 0) return CSA2_ERR_BAD_SHAPE;
  if (heads > 256 || top_k > 2048) return CSA2_ERR_UNSUPPORTED;
  if (kv->dim != 64 && kv->dim != 128 && kv->dim != 256 && kv->dim != 512) return CSA2_ERR_UNSUPPORTED;
  if (kv->dim == 512 && q_dtype == CSA2_F32) return CSA2_ERR_UNSUPPORTED;
  if (top_k + swa->window == 0) return CSA2_ERR_BAD_SHAPE;
  if (qs->m == 0) return CSA2_OK;
  if (!q || !out) return CSA2_ERR_NULL_ARG;
  if (top_k > 0 && !topk) return CSA2_ERR_NULL_ARG;
  const size_t need = attn_ws_bytes(qs->m, heads, kv->dim, top_k, swa->window);
  if (need > 256 && (!workspace || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 256)) return CSA2_ERR_MISALIGNED;
  return launch_attn(*kv, *qs, q, q_dtype, heads, topk, top_k, *swa, softmax_scale, out, lse, workspace,
                     (hipStream_t)stream);
}

// Group workspace: the indexer's region, then the attention region (whose
// arrival counters must keep their zeros between calls, so the indexer never
// writes there).
static size_t group_attn_offset(const csa2_group_desc *g) {
  return align256(index_bytes(&g->idx, g->qs.m, g->pool_blocks, g->top_k));
}

int32_t csa2_group_workspace_size(const csa2_group_desc *g, size_t *bytes) {
  if (!g || !bytes) return CSA2_ERR_NULL_ARG;
  if (g->qs.m < 0 || g->n_layers < 1 || g->heads < 1 || g->top_k < 1 || g->pool_blocks < 0)
    return CSA2_ERR_BAD_SHAPE;
  if (g->pool_blocks > 4096 || g->top_k > 2048) return CSA2_ERR_UNSUPPORTED;
  size_t b = 256;
  for (int i = 0; i < g->n_layers; ++i) {
    const int w = g->swa ? g->swa[i].window : 0;
    const size_t x = attn_ws_bytes(g->qs.m > 0 ? g->qs.m : 1, g->heads, g->kv.dim, g->top_k, w);
    if (x > b) b = x;
  }
  *bytes = group_attn_offset(g) + b;
  return CSA2_OK;
}

int32_t csa2_group_step(const csa2_group_desc *g, void *workspace, size_t ws_bytes, void *stream) {
  if (!g) return CSA2_ERR_NULL_ARG;
  if (g->first_mode != CSA2_MODE_FULL && g->first_mode != CSA2_MODE_REINDEX) return CSA2_ERR_BAD_SHAPE;
  if (g->n_layers < 1 || g->n_layers > 64) return CSA2_ERR_BAD_SHAPE;
  if (!g->q || !g->swa || !g->out) return CSA2_ERR_NULL_ARG;
  if (g->first_mode == CSA2_MODE_REINDEX && g->pool_blocks < 1) return CSA2_ERR_BAD_SHAPE;
  if (g->first_mode == CSA2_MODE_FULL && g->new_rows < 0) return CSA2_ERR_BAD_SHAPE;
  int st;
  size_t need = 0;
  if ((st = csa2_group_workspace_size(g, &need))) return st;
  if (!workspace || ws_bytes < need) return CSA2_ERR_WORKSPACE;
  // validate every call before enqueueing anything
  if ((st = check_index_common(&g->idx, &g->qs, g->q_idx, g->w_idx, g->idx_heads, g->top_k, g->topk))) return st;
  if ((st = check_cache(&g->kv, true))) return st;
  if (g->kv.dim != 64 && g->kv.dim != 128 && g->kv.dim != 256 && g->kv.dim != 512) return CSA2_ERR_UNSUPPORTED;
  if (g->q_dtype != CSA2_F32 && g->q_dtype != CSA2_BF16) return CSA2_ERR_BAD_DTYPE;
  if (g->kv.dim == 512 && g->q_dtype == CSA2_F32) return CSA2_ERR_UNSUPPORTED;
  if (g->heads > 256) return CSA2_ERR_UNSUPPORTED;
  if (g->pool_blocks > 0 && (!g->pool || !g->pool_count)) return CSA2_ERR_NULL_ARG;
  for (int i = 0; i < g->n_layers; ++i) {
    if ((st = check_swa(&g->swa[i], g->kv.dim))) return st;
    if (g->qs.m > 0 && (!g->q[i] || !g->out[i])) return CSA2_ERR_NULL_ARG;
  }
  if (g->first_mode == CSA2_MODE_FULL && g->new_rows > 0) {
    if (!g->new_kv || !g->w_ik || !g->new_dst_row) return CSA2_ERR_NULL_ARG;
    if (g->new_kv_dtype != CSA2_F32 && g->new_kv_dtype != CSA2_BF16) return CSA2_ERR_BAD_DTYPE;
    if (g->idx.dim > g->kv.dim) return CSA2_ERR_UNSUPPORTED;
  }
  if (g->qs.m == 0) return CSA2_OK;
  hipStream_t s = (hipStream_t)stream;
  if (g->first_mode == CSA2_MODE_FULL && g->new_rows > 0) {
    st = launch_quantize_fp4(g->new_kv, g->new_kv_dtype, g->new_rows, g->kv.dim, g->new_dst_row, g->kv.codes,
                             g->kv.scales, g->w_ik, g->idx.dim, g->idx.codes, g->idx.scales, s);
    if (st) return st;
  }
  if (g->first_mode == CSA2_MODE_FULL) {
    if (g->pool_blocks == 0)
      st = launch_index_flat(g->idx, g->qs, g->q_idx, g->w_idx, g->idx_heads, g->top_k, g->topk, g->topk_score,
                             workspace, s);
    else
      st = launch_index_full(g->idx, g->qs, g->q_idx, g->w_idx, g->idx_heads, g->pool_blocks, g->top_k, g->pool,
                             g->pool_count, g->topk, g->topk_score, workspace, s);
  } else {
    st = launch_reindex(g->idx, g->qs, g->q_idx, g->w_idx, g->idx_heads, g->pool, g->pool_count, g->pool_blocks,
                        g->top_k, g->topk, g->topk_score, workspace, s);
  }
  if (st) return st;
  for (int i = 0; i < g->n_layers; ++i) {
    st = launch_attn(g->kv, g->qs, g->q[i], g->q_dtype, g->heads, g->topk, g->top_k, g->swa[i], g->softmax_scale,
                     g->out[i], g->lse ? g->lse[i] : nullptr,
                     static_cast<char *>(workspace) + group_attn_offset(g), s);
    if (st) return st;
  }
  return CSA2_OK;
}

int32_t csa2_profile_scan(int32_t enable) {
  clear_events(g_timing[0]);
  g_timing[0].on = enable != 0;
  return CSA2_OK;
}

int32_t csa2_profile_scan_read(double *total_ms, int64_t *launches) {
  return read_events(g_timing[0], total_ms, launches);
}

int32_t csa2_profile_attn(int32_t enable) {
  clear_events(g_timing[1]);
  g_timing[1].on = enable != 0;
  return CSA2_OK;
}

int32_t csa2_profile_attn_read(double *total_ms, int64_t *launches) {
  return read_events(g_timing[1], total_ms, launches);
}

}  // extern "C"
