// Internal declarations shared by the CSA2 translation units.
#pragma once

#include "../../include/csa2.h"
#include "csa2_device.hpp"

#include <hip/hip_ext.h>

namespace csa2 {

// ---- write path (csa2_codec.hip) ----
int launch_quantize_fp4(const void *x, int x_dtype, int64_t rows, int dim, const int64_t *dst_row,
                        uint8_t *codes, uint8_t *scales, const float *w_ik, int idx_dim, uint8_t *ik_codes,
                        uint8_t *ik_scales, hipStream_t stream);
int launch_quantize_fp8_rows(const void *x, int x_dtype, int64_t rows, int dim, const int64_t *dst_row,
                             uint8_t *codes, float *scale, hipStream_t stream);
int launch_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int dim, float *out,
                       hipStream_t stream);

// ---- indexer (csa2_index.hip) ----
// Workspace layout of the indexer calls, all offsets 256-byte aligned.
struct IndexWs {
  size_t bmax, hist, counters, sure, tie, pscore, total;
  int64_t nb_max;       // block slots per query
  int32_t slots;        // 8 * pool_blocks
  int32_t hist_rep;     // first-scan histogram replicas per query
};
IndexWs index_ws_layout(int64_t max_len, int m, int pool_blocks, int top_k);

int launch_index_full(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                      const float *w_idx, int heads, int pool_blocks, int top_k, int32_t *pool_out,
                      int32_t *pool_count, int32_t *topk_out, float *topk_score, void *ws, hipStream_t stream);
int launch_reindex(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx, const float *w_idx,
                   int heads, const int32_t *pool_in, const int32_t *pool_count, int pool_blocks, int top_k,
                   int32_t *topk_out, float *topk_score, void *ws, hipStream_t stream);

// Stages shared with the flat indexer.  Block select: the pool of the top P
// blocks per query straight from the block maxima bmax[m * nb_stride + b]
// (nb_max >= every query's block count, at most kBlockSelectMax).  Re-score
// and select: the Top-K positions of the given pools, pscore holding 8P
// floats per query.
constexpr int64_t kBlockSelectMax = 1024 * 64;
int launch_block_select(const float *bmax, int64_t nb_stride, int64_t nb_max, const csa2_fp4_cache &idx,
                        const csa2_queries &qs, int P, int32_t *pool_out, int32_t *pool_count, hipStream_t stream);
int launch_rescore_select(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                          const float *w_idx, int heads, const int32_t *pool, const int32_t *pool_count, int P, int K,
                          int32_t *topk_out, float *topk_score, float *pscore, hipStream_t stream);

// ---- flat (prefill) indexer (csa2_prefill.hip) ----
size_t flat_ws_bytes(int64_t max_len, int m, int top_k);
int launch_index_flat(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                      const float *w_idx, int heads, int top_k, int32_t *topk_out, float *topk_score, void *ws,
                      hipStream_t stream);

// ---- attention (csa2_attn.hip) ----
// workspace of an attention call; its first bytes hold arrival counters that must be
// zero before the first call with that workspace (every call leaves them zero)
size_t attn_ws_bytes(int m, int heads, int dim, int top_k, int window);
int launch_attn(const csa2_fp4_cache &kv, const csa2_queries &qs, const void *q, int q_dtype, int heads,
                const int32_t *topk, int top_k, const csa2_swa &swa, float scale, float *out, float *lse, void *ws,
                hipStream_t stream);

// Prefill schedule for the 512-channel latent with bf16 queries
// (csa2_attn_prefill.hip); needs top_k % 16 == 0 and no workspace.
bool attn_prefill_supported(const csa2_fp4_cache &kv, int q_dtype, int top_k);
int launch_attn_prefill(const csa2_fp4_cache &kv, const csa2_queries &qs, const void *q, int heads,
                        const int32_t *topk, int top_k, const csa2_swa &swa, float scale, float *out, float *lse,
                        hipStream_t stream);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- kernel timing (csa2_api.hip) ----
// Timed kernels: the first scan of an index call (decode scan or prefill
// scoring) and each attention launch.  timing_events hands out a fresh
// start/stop pair when that timing is on (both null otherwise); launched with
// hipExtLaunchKernelGGL, the pair takes the dispatch's own start and end
// times, so no marker packets sit between the events and the kernel.
enum TimedKernel { kTimedScan = 0, kTimedAttn = 1 };
void timing_events(int which, hipEvent_t *start, hipEvent_t *stop);

#define CSA2_TIMED_LAUNCH(which, kernel, grid, block, stream, ...)                                  \
  do {                                                                                              \
    hipEvent_t csa2_t0_, csa2_t1_;                                                                  \
    ::csa2::timing_events(which, &csa2_t0_, &csa2_t1_);                                             \
    if (csa2_t0_)                                                                                   \
      hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, csa2_t0_, csa2_t1_, 0, __VA_ARGS__);    \
    else                                                                                            \
      hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);                              \
  } while (0)

}  // namespace csa2
