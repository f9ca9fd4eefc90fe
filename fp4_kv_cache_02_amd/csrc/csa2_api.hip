// C ABI of the CSA2 hot path: host-side validation, workspace sizing and
// dispatch.  Every check runs before anything is enqueued.
#include "csa2_internal.hpp"

#include <mutex>
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
Timing g_timing[4];                 // 0: first scan, 1: attention, 2: quantise-on-write, 3: compressor

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
  if (q->m < 0 || q->run < 0) return CSA2_ERR_BAD_SHAPE;
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

// The flat (pool_blocks == 0) indexer keeps every query's block maxima for its
// block select: at most kBlockSelectMax blocks per sequence.
int check_flat_limits(const csa2_fp4_cache *idx, int pool_blocks) {
  if (pool_blocks == 0 && (idx->max_len + kBlock - 1) / kBlock > kBlockSelectMax) return CSA2_ERR_UNSUPPORTED;
  return CSA2_OK;
}

size_t index_bytes(const csa2_fp4_cache *idx, int m, int pool_blocks, int top_k, int n_sets = 1) {
  if (pool_blocks == 0) return flat_ws_bytes(idx->max_len, m, top_k);
  return index_ws_layout(idx->max_len, m, pool_blocks, top_k, n_sets).total;
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

int32_t csa2_compress_fp4(const uint16_t *tokens, int64_t entries, int32_t ratio, int32_t d_in, const uint16_t *w_c,
                          int32_t dim, const int64_t *dst_row, uint8_t *codes, uint8_t *scales, const float *w_ik,
                          int32_t idx_dim, uint8_t *ik_codes, uint8_t *ik_scales, void *stream) {
  if (entries < 0 || ratio < 1 || ratio > 16 || d_in <= 0 || d_in % 32 != 0 || d_in > 8192 ||
      (int64_t)ratio * d_in > 16384 || dim <= 0 || dim % 32 != 0)
    return CSA2_ERR_BAD_SHAPE;
  if (dim > 512) return CSA2_ERR_UNSUPPORTED;
  if (entries == 0) return CSA2_OK;
  if (entries > ((int64_t)1 << 31)) return CSA2_ERR_UNSUPPORTED;
  if (!tokens || !w_c || !codes || !scales) return CSA2_ERR_NULL_ARG;
  if (!aligned(tokens, 16) || !aligned(w_c, 16) || !aligned(codes, 8)) return CSA2_ERR_MISALIGNED;
  if (w_ik) {
    if (!ik_codes || !ik_scales) return CSA2_ERR_NULL_ARG;
    if (idx_dim != 32 && idx_dim != 64 && idx_dim != 128 && idx_dim != 256) return CSA2_ERR_UNSUPPORTED;
    if (idx_dim > dim) return CSA2_ERR_UNSUPPORTED;
    if (!aligned(ik_codes, 8)) return CSA2_ERR_MISALIGNED;
  }
  return launch_compress_fp4(tokens, entries, ratio, d_in, w_c, dim, dst_row, codes, scales, w_ik, idx_dim, ik_codes,
                             ik_scales, (hipStream_t)stream);
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
  if ((st = check_flat_limits(idx, pool_blocks))) return st;
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
  *bytes = (m == 0) ? 256 : attn_ws_bytes(m, heads, dim, top_k, window, 1, 1);
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
  const size_t need = attn_ws_bytes(qs->m, heads, kv->dim, top_k, swa->window, 1, 1);
  if (need > 256 && (!workspace || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 256)) return CSA2_ERR_MISALIGNED;
  const AttnLayer layer{q, swa->codes, swa->scale, swa->start, swa->count, swa->window, out, lse, topk, 0, 0};
  return launch_attn_layers(*kv, *qs, q_dtype, heads, top_k, &layer, 1, softmax_scale, workspace,
                            (hipStream_t)stream);
}

static_assert(kAttnBatch >= 1, "attention batches");

// Group workspace: the attention region (its layers' intermediates), then the
// indexer's region.  Neither needs initial contents.
static int group_max_window(const csa2_group_desc *g) {
  int w = 0;
  for (int i = 0; i < g->n_layers; ++i) w = std::max(w, g->swa ? g->swa[i].window : 0);
  return w;
}
static size_t group_index_offset(const csa2_group_desc *g) {
  const size_t a = attn_ws_bytes(g->qs.m > 0 ? g->qs.m : 1, g->heads, g->kv.dim, g->top_k, group_max_window(g),
                                 g->n_layers, 1);
  return align256(std::max<size_t>(256, a));
}

int32_t csa2_group_workspace_size(const csa2_group_desc *g, size_t *bytes) {
  if (!g || !bytes) return CSA2_ERR_NULL_ARG;
  if (g->qs.m < 0 || g->n_layers < 1 || g->heads < 1 || g->top_k < 1 || g->pool_blocks < 0)
    return CSA2_ERR_BAD_SHAPE;
  if (g->pool_blocks > 4096 || g->top_k > 2048) return CSA2_ERR_UNSUPPORTED;
  *bytes = group_index_offset(g) + align256(index_bytes(&g->idx, g->qs.m, g->pool_blocks, g->top_k));
  return CSA2_OK;
}

// Every check of a group step except the workspace's, before anything is enqueued.
static int check_group(const csa2_group_desc *g) {
  if (!g) return CSA2_ERR_NULL_ARG;
  if (g->first_mode != CSA2_MODE_FULL && g->first_mode != CSA2_MODE_REINDEX) return CSA2_ERR_BAD_SHAPE;
  if (g->n_layers < 1 || g->n_layers > 64) return CSA2_ERR_BAD_SHAPE;
  if (!g->q || !g->swa || !g->out) return CSA2_ERR_NULL_ARG;
  if (g->first_mode == CSA2_MODE_REINDEX && g->pool_blocks < 1) return CSA2_ERR_BAD_SHAPE;
  if (g->first_mode == CSA2_MODE_FULL && g->new_rows < 0) return CSA2_ERR_BAD_SHAPE;
  int st;
  size_t need = 0;
  if ((st = csa2_group_workspace_size(g, &need))) return st;
  if ((st = check_index_common(&g->idx, &g->qs, g->q_idx, g->w_idx, g->idx_heads, g->top_k, g->topk))) return st;
  if (g->first_mode == CSA2_MODE_FULL && (st = check_flat_limits(&g->idx, g->pool_blocks))) return st;
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
  return CSA2_OK;
}

// A Full group's write path.  When the group's pool comes from the first
// scan, the write launch also clears the index workspace's histograms and
// counters (which the scan needs zeroed), so the index path skips its own
// fill launch; returns whether it did.
static int enqueue_group_write(const csa2_group_desc *g, void *iws, hipStream_t s, bool *cleared) {
  *cleared = false;
  if (g->first_mode != CSA2_MODE_FULL || g->new_rows <= 0) return CSA2_OK;
  uint32_t *zero = nullptr;
  int64_t words = 0;
  if (g->pool_blocks > 0 && g->qs.m > 0) {
    const IndexWs L = index_ws_layout(g->idx.max_len, g->qs.m, g->pool_blocks, g->top_k);
    zero = reinterpret_cast<uint32_t *>(static_cast<char *>(iws) + L.hist);
    words = (int64_t)((L.sure - L.hist) / sizeof(uint32_t));
  }
  const int st = launch_quantize_fp4(g->new_kv, g->new_kv_dtype, g->new_rows, g->kv.dim, g->new_dst_row,
                                     g->kv.codes, g->kv.scales, g->w_ik, g->idx.dim, g->idx.codes, g->idx.scales, s,
                                     zero, words);
  *cleared = st == CSA2_OK && zero != nullptr;
  return st;
}

// The group's write path and its first layer's indexer (m > 0).
static int enqueue_group_index(const csa2_group_desc *g, void *iws, hipStream_t s) {
  bool cleared = false;
  int st = enqueue_group_write(g, iws, s, &cleared);
  if (st) return st;
  if (g->first_mode == CSA2_MODE_FULL) {
    if (g->pool_blocks == 0)
      st = launch_index_flat(g->idx, g->qs, g->q_idx, g->w_idx, g->idx_heads, g->top_k, g->topk, g->topk_score,
                             iws, s);
    else if ((st = launch_index_pool(g->idx, g->qs, g->q_idx, g->w_idx, g->idx_heads, g->pool_blocks, g->top_k,
                                     g->pool, g->pool_count, iws, s, cleared)) == CSA2_OK) {
      const IndexWs L = index_ws_layout(g->idx.max_len, g->qs.m, g->pool_blocks, g->top_k);
      const SelSet set{g->q_idx, g->w_idx, g->topk, g->topk_score};
      st = launch_rescore_select(g->idx, g->qs, g->idx_heads, g->pool, g->pool_count, g->pool_blocks, g->top_k,
                                 &set, 1, reinterpret_cast<float *>(static_cast<char *>(iws) + L.pscore), s);
    }
  } else {
    st = launch_reindex(g->idx, g->qs, g->q_idx, g->w_idx, g->idx_heads, g->pool, g->pool_count, g->pool_blocks,
                        g->top_k, g->topk, g->topk_score, iws, s);
  }
  return st;
}

static void group_layers(const csa2_group_desc *g, AttnLayer *out) {
  for (int i = 0; i < g->n_layers; ++i) {
    const csa2_swa &w = g->swa[i];
    out[i] = AttnLayer{g->q[i], w.codes, w.scale, w.start, w.count, w.window, g->out[i],
                       g->lse ? g->lse[i] : nullptr, g->topk, 0, 0};
  }
}

int32_t csa2_group_step(const csa2_group_desc *g, void *workspace, size_t ws_bytes, void *stream) {
  int st = check_group(g);
  if (st) return st;
  size_t need = 0;
  if ((st = csa2_group_workspace_size(g, &need))) return st;
  if (!workspace || ws_bytes < need) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_MISALIGNED;
  if (g->qs.m == 0) return CSA2_OK;
  hipStream_t s = (hipStream_t)stream;
  if ((st = enqueue_group_index(g, static_cast<char *>(workspace) + group_index_offset(g), s))) return st;
  AttnLayer layers[64];
  group_layers(g, layers);
  return launch_attn_layers(g->kv, g->qs, g->q_dtype, g->heads, g->top_k, layers, g->n_layers, g->softmax_scale,
                            workspace, s);
}

// ---------------------------------------------------------------------------
// csa2_group_steps: several groups, their attention batched across groups
// ---------------------------------------------------------------------------
// Consecutive groups whose layers can share one attention launch: the same
// main cache, queries, query format, heads, Top-K length and softmax scale.
static bool same_attention(const csa2_group_desc *a, const csa2_group_desc *b) {
  const csa2_fp4_cache &x = a->kv, &y = b->kv;
  return x.codes == y.codes && x.scales == y.scales && x.seq_start == y.seq_start && x.seq_len == y.seq_len &&
         x.n_seq == y.n_seq && x.dim == y.dim && x.max_len == y.max_len && x.ratio == y.ratio &&
         a->qs.seq == b->qs.seq && a->qs.pos == b->qs.pos && a->qs.m == b->qs.m && a->q_dtype == b->q_dtype &&
         a->heads == b->heads && a->top_k == b->top_k && a->softmax_scale == b->softmax_scale;
}

constexpr int kMaxGroups = 32;

// Workspace: the attention region (any batch of the call), then the region
// the groups' indexers use one after another.
static size_t steps_index_offset(const csa2_group_desc *groups, int n) {
  int wmax = 0, layers = 0;
  for (int i = 0; i < n; ++i) {
    wmax = std::max(wmax, group_max_window(&groups[i]));
    layers += groups[i].n_layers;
  }
  size_t a = 256;
  for (int i = 0; i < n; ++i) {
    const csa2_group_desc *g = &groups[i];
    a = std::max(a, attn_ws_bytes(g->qs.m > 0 ? g->qs.m : 1, g->heads, g->kv.dim, g->top_k, wmax, layers, n));
  }
  return align256(a);
}

// A REINDEX group that can join the query sets re-scored and selected
// together with the groups before it (the first of which is `head`): the
// same pool, indexer cache, queries and pool / Top-K sizes.
static bool same_pool(const csa2_group_desc *head, const csa2_group_desc *g) {
  const csa2_fp4_cache &x = head->idx, &y = g->idx;
  return g->first_mode == CSA2_MODE_REINDEX && head->pool_blocks > 0 && g->pool == head->pool &&
         g->pool_count == head->pool_count && g->pool_blocks == head->pool_blocks && g->top_k == head->top_k &&
         g->idx_heads == head->idx_heads && x.codes == y.codes && x.scales == y.scales &&
         x.seq_start == y.seq_start && x.seq_len == y.seq_len && x.n_seq == y.n_seq && x.dim == y.dim &&
         x.max_len == y.max_len && x.ratio == y.ratio && g->qs.seq == head->qs.seq && g->qs.pos == head->qs.pos &&
         g->qs.m == head->qs.m && g->qs.run == head->qs.run;
}

// Query-set families: each group starts one unless it joins the previous
// family; fam[i] = index of the first group of group i's family.
static void pool_families(const csa2_group_desc *groups, int n, int *fam) {
  for (int i = 0; i < n; ++i) {
    fam[i] = i;
    if (i > 0) {
      const int h = fam[i - 1];
      if (i - h < kSelSets && same_pool(&groups[h], &groups[i])) fam[i] = h;
    }
  }
}

int32_t csa2_group_steps_workspace_size(const csa2_group_desc *groups, int32_t n_groups, size_t *bytes) {
  if (!groups || !bytes) return CSA2_ERR_NULL_ARG;
  if (n_groups < 1 || n_groups > kMaxGroups) return CSA2_ERR_BAD_SHAPE;
  int fam[kMaxGroups];
  pool_families(groups, n_groups, fam);
  size_t idx = 0;
  for (int i = 0; i < n_groups; ++i) {
    size_t one = 0;
    const int st = csa2_group_workspace_size(&groups[i], &one);
    if (st) return st;
    if (groups[i].n_layers > 64) return CSA2_ERR_BAD_SHAPE;
    // a family's last group sizes the re-score buffer of all its query sets
    idx = std::max(idx, align256(index_bytes(&groups[i].idx, groups[i].qs.m, groups[i].pool_blocks,
                                             groups[i].top_k, i - fam[i] + 1)));
  }
  *bytes = steps_index_offset(groups, n_groups) + idx;
  return CSA2_OK;
}

int32_t csa2_group_steps(const csa2_group_desc *groups, int32_t n_groups, void *workspace, size_t ws_bytes,
                         void *stream) {
  if (!groups) return CSA2_ERR_NULL_ARG;
  if (n_groups < 1 || n_groups > kMaxGroups) return CSA2_ERR_BAD_SHAPE;
  int st;
  for (int i = 0; i < n_groups; ++i)
    if ((st = check_group(&groups[i]))) return st;
  size_t need = 0;
  if ((st = csa2_group_steps_workspace_size(groups, n_groups, &need))) return st;
  if (!workspace || ws_bytes < need) return CSA2_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return CSA2_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  void *iws = static_cast<char *>(workspace) + steps_index_offset(groups, n_groups);
  std::vector<AttnLayer> layers;
  // the attention of groups [a, b), one launch sequence per run of groups
  // that can share it
  auto flush = [&](int a, int b) -> int {
    for (int i = a; i < b;) {
      int j = i + 1;
      while (j < b && same_attention(&groups[i], &groups[j])) ++j;
      const csa2_group_desc *g = &groups[i];
      if (g->qs.m > 0) {
        layers.clear();
        for (int k = i; k < j; ++k) {
          const size_t at = layers.size();
          layers.resize(at + groups[k].n_layers);
          group_layers(&groups[k], layers.data() + at);
        }
        const int r = launch_attn_layers(g->kv, g->qs, g->q_dtype, g->heads, g->top_k, layers.data(),
                                         (int)layers.size(), g->softmax_scale, workspace, s);
        if (r) return r;
      }
      i = j;
    }
    return CSA2_OK;
  };
  int fam[kMaxGroups];
  pool_families(groups, n_groups, fam);
  // the re-score and select of family [h, e): one launch pair for all its query sets
  auto select = [&](int h, int e) -> int {
    const csa2_group_desc *g = &groups[h];
    if (g->qs.m == 0) return CSA2_OK;
    SelSet sets[kSelSets];
    for (int k = h; k < e; ++k) sets[k - h] = SelSet{groups[k].q_idx, groups[k].w_idx, groups[k].topk,
                                                       groups[k].topk_score};
    const IndexWs L = index_ws_layout(g->idx.max_len, g->qs.m, g->pool_blocks, g->top_k, e - h);
    return launch_rescore_select(g->idx, g->qs, g->idx_heads, g->pool, g->pool_count, g->pool_blocks, g->top_k,
                                 sets, e - h, reinterpret_cast<float *>(static_cast<char *>(iws) + L.pscore), s);
  };
  int pending = 0;   // first group whose attention has not been enqueued
  for (int i = 0; i < n_groups; ++i) {
    const csa2_group_desc *g = &groups[i];
    // a group that writes into a main cache which pending attention still
    // reads runs after that attention, as it would group by group
    if (g->first_mode == CSA2_MODE_FULL && g->new_rows > 0) {
      for (int k = pending; k < i; ++k)
        if (groups[k].kv.codes == g->kv.codes || groups[k].kv.scales == g->kv.scales) {
          if ((st = flush(pending, i))) return st;
          pending = i;
          break;
        }
    }
    if (g->qs.m > 0) {
      bool cleared = false;
      if ((st = enqueue_group_write(g, iws, s, &cleared))) return st;
      if (g->first_mode == CSA2_MODE_FULL && g->pool_blocks == 0) {
        st = launch_index_flat(g->idx, g->qs, g->q_idx, g->w_idx, g->idx_heads, g->top_k, g->topk, g->topk_score,
                               iws, s);
      } else if (g->first_mode == CSA2_MODE_FULL) {
        st = launch_index_pool(g->idx, g->qs, g->q_idx, g->w_idx, g->idx_heads, g->pool_blocks, g->top_k, g->pool,
                               g->pool_count, iws, s, cleared);
      }
      if (st) return st;
    }
    // a family ends where the next group does not join it: its query sets
    // are re-scored and selected before anything of the next group runs
    const bool flat = g->first_mode == CSA2_MODE_FULL && g->pool_blocks == 0;
    if (!flat && (i + 1 == n_groups || fam[i + 1] != fam[i]) && (st = select(fam[i], i + 1))) return st;
  }
  return flush(pending, n_groups);
}

// ---------------------------------------------------------------------------
// csa2_group_step_static: the group step on a library-owned scratch array
// ---------------------------------------------------------------------------
// One copy per GPU, held until the process ends.  In host code `scratch` is a
// host-side stand-in for the device symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) uint8_t scratch[CSA2_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device

int static_scratch(void **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CSA2_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CSA2_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA2_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return CSA2_OK;
}
}  // namespace

int32_t csa2_group_step_static(const csa2_group_desc *g, void *stream) {
  if (!g) return CSA2_ERR_NULL_ARG;
  size_t need = 0;
  int st = csa2_group_workspace_size(g, &need);
  if (st) return st;
  if (need > (size_t)CSA2_STATIC_SCRATCH_BYTES) return CSA2_ERR_WORKSPACE;
  void *p = nullptr;
  if ((st = static_scratch(&p))) return st;
  // no call needs initial scratch contents
  return csa2_group_step(g, p, (size_t)CSA2_STATIC_SCRATCH_BYTES, stream);
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

int32_t csa2_profile_write(int32_t enable) {
  clear_events(g_timing[2]);
  g_timing[2].on = enable != 0;
  return CSA2_OK;
}

int32_t csa2_profile_write_read(double *total_ms, int64_t *launches) {
  return read_events(g_timing[2], total_ms, launches);
}

int32_t csa2_profile_compress(int32_t enable) {
  clear_events(g_timing[3]);
  g_timing[3].on = enable != 0;
  return CSA2_OK;
}

int32_t csa2_profile_compress_read(double *total_ms, int64_t *launches) {
  return read_events(g_timing[3], total_ms, launches);
}

}  // extern "C"
