// Internal declarations shared by the CSA2 translation units.
#pragma once

#include "../../include/csa2.h"
#include "csa2_device.hpp"

#include <hip/hip_ext.h>

namespace csa2 {

// ---- write path (csa2_codec.hip) ----
// zero / zero_words: a 16-byte aligned range (zero_words % 4 == 0) that the
// launch also clears - in spare workgroups of the write kernel when the rows
// take the few-row kernel (the decode write), else with a fill kernel - so a
// decode step's index workspace needs no fill launch of its own.
int launch_quantize_fp4(const void *x, int x_dtype, int64_t rows, int dim, const int64_t *dst_row,
                        uint8_t *codes, uint8_t *scales, const float *w_ik, int idx_dim, uint8_t *ik_codes,
                        uint8_t *ik_scales, hipStream_t stream, uint32_t *zero = nullptr, int64_t zero_words = 0);
// Compressor fused with the FP4 write (and the indexer keys of the written
// rows when w_ik is given); dim <= 512, (ratio * d_in) % 32 == 0.
int launch_compress_fp4(const uint16_t *tokens, int64_t entries, int ratio, int d_in, const uint16_t *w_c, int dim,
                        const int64_t *dst_row, uint8_t *codes, uint8_t *scales, const float *w_ik, int idx_dim,
                        uint8_t *ik_codes, uint8_t *ik_scales, hipStream_t stream);
int launch_quantize_fp8_rows(const void *x, int x_dtype, int64_t rows, int dim, const int64_t *dst_row,
                             uint8_t *codes, float *scale, hipStream_t stream);
int launch_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int dim, float *out,
                       hipStream_t stream);

// ---- indexer (csa2_index.hip) ----
// Workspace layout of the indexer calls, all offsets 256-byte aligned.
struct IndexWs {
  size_t bmax, hist, counters, fine, sure, tie, pscore, total;
  int64_t nb_max;       // block slots per query
  int32_t slots;        // 8 * pool_blocks
  int32_t hist_rep;     // first-scan histogram replicas per query
};
// n_sets: query sets (groups) re-scored and selected together over one pool.
IndexWs index_ws_layout(int64_t max_len, int m, int pool_blocks, int top_k, int n_sets = 1);

int launch_index_full(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                      const float *w_idx, int heads, int pool_blocks, int top_k, int32_t *pool_out,
                      int32_t *pool_count, int32_t *topk_out, float *topk_score, void *ws, hipStream_t stream);
// The first part of launch_index_full alone: the scan and the pool (no Top-K).
// ws_cleared: the workspace's [hist, sure) range (histograms, counters) is
// already zero in stream order (cleared by the step's write launch).
int launch_index_pool(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx, const float *w_idx,
                      int heads, int pool_blocks, int top_k, int32_t *pool_out, int32_t *pool_count, void *ws,
                      hipStream_t stream, bool ws_cleared = false);
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
// One query set of a batched re-score and select: its indexer queries and
// head weights, and its outputs.
struct SelSet {
  const uint16_t *q_idx;
  const float *w_idx;
  int32_t *topk;
  float *score;
};
constexpr int kSelSets = 8;   // query sets per launch
// Re-score and select for n_sets query sets over the same pools (pscore:
// n_sets * m * 8P floats).
int launch_rescore_select(const csa2_fp4_cache &idx, const csa2_queries &qs, int heads, const int32_t *pool,
                          const int32_t *pool_count, int P, int K, const SelSet *sets, int n_sets, float *pscore,
                          hipStream_t stream);

// ---- multi-query scoring (csa2_prefill.hip) ----
// Block maxima bmax[m * nb_stride + b] of every query's visible entries from
// the multi-query MFMA kernel (each streamed indexer entry scored against all
// the queries of its sequence in a workgroup's query block).
int launch_score_blocks(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                        const float *w_idx, int heads, float *bmax, int64_t nb_stride, hipStream_t stream);

// ---- flat (prefill) indexer (csa2_prefill.hip) ----
size_t flat_ws_bytes(int64_t max_len, int m, int top_k);
int launch_index_flat(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                      const float *w_idx, int heads, int top_k, int32_t *topk_out, float *topk_score, void *ws,
                      hipStream_t stream);

// ---- attention (csa2_attn.hip) ----
// One layer's attention inputs and outputs (window fields as in csa2_swa).
struct AttnLayer {
  const void *q;
  const uint8_t *swa_codes;
  const float *swa_scale;
  const int32_t *swa_start;
  const int32_t *swa_count;
  int32_t window;
  float *out;
  float *lse;
  const int32_t *topk;   // the layer's Top-K list [m][top_k]
  // set by launch_attn_layers: which gathered copy of a Top-K list the layer
  // reads in its batch, and whether it writes that copy
  int32_t list;
  int32_t gather;
};
constexpr int kAttnBatch = 24;  // layers per launch of the decode schedule
// Workspace of launch_attn_layers over n_layers layers whose largest window
// is max_window and that use at most n_lists distinct Top-K lists (no
// initial contents needed).
size_t attn_ws_bytes(int m, int heads, int dim, int top_k, int max_window, int n_layers, int n_lists);
// Attention of n_layers layers that share the main cache and the queries;
// each layer has its own Top-K list pointer (layers of one group share it).
int launch_attn_layers(const csa2_fp4_cache &kv, const csa2_queries &qs, int q_dtype, int heads, int top_k,
                       const AttnLayer *layers, int n_layers, float scale, void *ws, hipStream_t stream);

// Prefill schedule for the 512-channel latent with bf16 queries
// (csa2_attn_prefill.hip); needs top_k % 16 == 0 and no workspace.
bool attn_prefill_supported(const csa2_fp4_cache &kv, int q_dtype, int top_k);
int launch_attn_prefill(const csa2_fp4_cache &kv, const csa2_queries &qs, const void *q, int heads,
                        const int32_t *topk, int top_k, const csa2_swa &swa, float scale, float *out, float *lse,
                        hipStream_t stream);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- kernel timing (csa2_api.hip) ----
// Timed kernels: the first scan of an index call (decode scan or prefill
// scoring), each attention launch, each quantise-on-write launch and each
// compressor launch.  timing_events hands out a fresh
// start/stop pair when that timing is on (both null otherwise); launched with
// hipExtLaunchKernelGGL, the pair takes the dispatch's own start and end
// times, so no marker packets sit between the events and the kernel.
enum TimedKernel { kTimedScan = 0, kTimedAttn = 1, kTimedWrite = 2, kTimedCompress = 3 };
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
