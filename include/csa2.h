/*
 * csa2.h - C ABI of the CSA2 (Compressed Sparse Attention 2) hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * Source pages (cited by key):
 *   P1 "DeepSeek-V4.1-Flash 发布：100 万上下文 + FP4 KV Cache + 跨层注意力复用"
 *      (feinterview.poetries.top)
 *   P2 "DeepSeek V4.1 Flash 发布，百万上下文开始算缓存这笔账" (cnblogs.com/OpenCSG)
 *   P4 DeepSeek V4.1-Flash CED / CSA2 paper notes (yomxxx.com, 2026-09-14)
 *   P5 "V4.1 Flash 内测登场：40 天改架构、调用价不变" (tucaod.com)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every function returns an int32_t status (CSA2_OK = 0, errors < 0).
 * - Pointers marked "device" must point to GPU memory of the current HIP
 *   device; pointers marked "host" to host memory.  The caller owns every
 *   buffer; the library never allocates or frees device memory on these
 *   calls.  Scratch memory is the caller's `workspace` (size from the
 *   matching *_workspace_size call, alignment 256 bytes).
 * - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *   enqueue work on it; none synchronises with the host.
 * - All argument validation happens on the host before anything is
 *   enqueued, so errors leave device memory untouched.  A kernel fault
 *   surfaces at the caller's next synchronisation.  CSA2_ERR_HIP reports a
 *   failed launch (hipGetLastError after enqueueing).
 * - Data-dependent conditions are defined behaviour, not errors: a Top-K or
 *   pool entry < 0 or >= the query's visible count is skipped; fewer
 *   candidates than K pad the output with -1; an empty key set yields
 *   o = 0 and lse = -inf.
 * - Calls that share a workspace must be ordered on one stream.
 *
 * Storage formats (P1 section "FP4 KV、Bounded Replay 及其他扩展"; P4 section
 * 三; P5 section "缓存精度与持久化分层")
 * ----------------------------------------------------------------------
 * FP4 row of `dim` channels: `dim/2` code bytes - byte k
 * holds channel 2k in its low nibble and 2k+1 in its high nibble, each an
 * E2M1 code (sign bit 3, magnitudes 0,.5,1,1.5,2,3,4,6) - plus `dim/16`
 * scale bytes, scale g being an OCP E4M3FN value for channels 16g..16g+15.
 * Codes and scales live in two planes, [rows][dim/2] and [rows][dim/16].
 * Value = e2m1(code) * e4m3(scale); no global scale.  The format itself
 * needs dim % 16 == 0 (whole scale groups); this library takes FP4 rows
 * with dim % 32 == 0 (its kernels move whole 16-byte code words, 32
 * channels) and rejects other widths with BAD_SHAPE; 512-channel latents
 * and 128- or 64-channel indexer keys qualify.
 * FP8 window row: `dim` OCP E4M3FN codes plus one fp32 row scale; value =
 * e4m3(code) * scale.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 2

enum csa2_status {
  CSA2_OK = 0,
  CSA2_ERR_NULL_ARG = -1,      /* a required pointer is NULL */
  CSA2_ERR_BAD_SHAPE = -2,     /* a size is negative, inconsistent or out of range */
  CSA2_ERR_BAD_DTYPE = -3,     /* unknown dtype code */
  CSA2_ERR_MISALIGNED = -4,    /* a pointer lacks the alignment the layout needs */
  CSA2_ERR_WORKSPACE = -5,     /* workspace NULL or smaller than required */
  CSA2_ERR_UNSUPPORTED = -6,   /* valid but not implemented (e.g. dim or head count) */
  CSA2_ERR_HIP = -7            /* a HIP launch failed */
};

enum csa2_dtype { CSA2_F32 = 0, CSA2_BF16 = 1 };

enum csa2_mode { CSA2_MODE_FULL = 0, CSA2_MODE_REINDEX = 1 };

/* One FP4 cache (main latent KV or indexer keys) holding `n_seq` sequences.
 * Entry j of sequence s is row seq_start[s] + j; seq_len[s] entries exist.
 * At compression ratio `ratio`, entry j summarises tokens j*r .. j*r+r-1 and
 * is visible to token t iff (j+1)*r - 1 <= t (P4 section 二; P1 CSA2
 * section: the encoder caches at ratio 2, the decoder at ratio 1). */
typedef struct csa2_fp4_cache {
  uint8_t *codes;             /* device [rows][dim/2], 16-byte aligned, dim/2 % 16 == 0 */
  uint8_t *scales;            /* device [rows][dim/16] */
  const int64_t *seq_start;   /* device [n_seq] first row of each sequence */
  const int32_t *seq_len;     /* device [n_seq] entries of each sequence */
  int32_t n_seq;
  int32_t dim;                /* channels per entry, multiple of 32 */
  int32_t max_len;            /* host upper bound of seq_len[] (sizes grids and workspace) */
  int32_t ratio;              /* compression ratio r >= 1 */
} csa2_fp4_cache;

/* The queries of one call: query i belongs to sequence seq[i] and is token
 * pos[i] of it.  Visible entries: vis = min(seq_len, floor((pos+1)/ratio)).
 * `run` is a host-side schedule hint: the queries come in runs of `run`
 * consecutive entries of one sequence (several tokens of one sequence decoded
 * together, P5 section "其他架构扩展" on parallel draft positions; a replayed
 * window of tokens, P1 section "FP4 KV、Bounded Replay 及其他扩展").  With
 * run >= 2 the indexers score each streamed indexer entry against all the
 * queries of its sequence at once.  0 or 1 promises nothing; results never
 * depend on it. */
typedef struct csa2_queries {
  const int32_t *seq;         /* device [m] */
  const int32_t *pos;         /* device [m] */
  int32_t m;
  int32_t run;                /* host: queries per run of one sequence (0/1: no promise) */
} csa2_queries;

/* Sliding-window KV of one layer: query i attends to rows start[i] ..
 * start[i]+count[i]-1 (0 <= count[i] <= window).  Each layer keeps its own
 * window rows in every mode (P1 CSA2 section; P4 section 二). */
typedef struct csa2_swa {
  const uint8_t *codes;       /* device [rows][dim] E4M3FN, 16-byte aligned */
  const float *scale;         /* device [rows] */
  const int32_t *start;       /* device [m] */
  const int32_t *count;       /* device [m] */
  int32_t dim;
  int32_t window;             /* upper bound of count[] */
} csa2_swa;

int32_t csa2_abi_version(void);
const char *csa2_status_string(int32_t status);

/* ---------------------------------------------------------------------
 * csa2_quantize_fp4 - quantise-on-write of main-KV rows, optionally with the
 * indexer key derived from each written entry.
 *
 * P1 section "FP4 KV、Bounded Replay 及其他扩展" / P4 section 三: main KV is
 * E2M1 with one E4M3 scale per 16 channels and no global scale.  P4 section
 * 二 / P5 section "CSA2注意力": a Full layer projects its indexer key from its
 * own main-KV entry.
 *
 * x        device [rows][dim], fp32 or bf16 (x_dtype), row-major, dense.
 * dst_row  device [rows] int64: cache row that input row i is written to;
 *          NULL writes row i to cache row i.
 * codes/scales  device FP4 planes of the main cache (see header comment).
 * Group scale = E4M3 nearest to the exact amax/6 (ties to even code);
 * element = E2M1 nearest to the exact |x|/scale (ties to even, saturating at
 * 6), sign bit kept.  NaN/Inf inputs give unspecified codes.
 * w_ik     device [dim][idx_dim] fp32 or NULL.  When given, the indexer key
 *          fp32(W_ik^T DQ4(written row)) (fp64 accumulation, one rounding; a
 *          zero sum is +0) is FP4-encoded into ik_codes/ik_scales at the
 *          same row.  idx_dim % 32 == 0, idx_dim <= 256.
 * Errors: NULL_ARG, BAD_SHAPE (rows < 0, dim % 32 != 0, dim > 4096),
 *         BAD_DTYPE, MISALIGNED, UNSUPPORTED (idx_dim), HIP.
 * ------------------------------------------------------------------- */
int32_t csa2_quantize_fp4(const void *x, int32_t x_dtype, int64_t rows, int32_t dim,
                          const int64_t *dst_row, uint8_t *codes, uint8_t *scales,
                          const float *w_ik, int32_t idx_dim, uint8_t *ik_codes,
                          uint8_t *ik_scales, void *stream);

/* ---------------------------------------------------------------------
 * csa2_compress_fp4 - the compressor at ratio r fused with quantise-on-write
 * and the indexer-key derivation.
 *
 * P4 section 二 / P5 section "CSA2注意力": CSA2's compressor has no overlap
 * between adjacent compressed entries and no absolute position embedding,
 * and the indexer key is projected from the main-KV entry.  Entry j is a
 * linear map of its own r token rows only:
 *     c_j = fp32(W_c^T [x_{r j}; x_{r j + 1}; ...; x_{r j + r - 1}]),
 * every bf16 x bf16 product exact, accumulated in fp64, rounded once to fp32
 * (a zero sum is +0).  c_j is then written exactly as csa2_quantize_fp4
 * writes an fp32 row (same FP4 rounding, same indexer key).
 *
 * tokens   device bf16 [entries * ratio][d_in], row-major, dense: token rows
 *          in sequence order; entry j reads rows ratio*j .. ratio*j+ratio-1.
 * w_c      device bf16 [dim][ratio * d_in], row-major: row c holds output
 *          channel c's weights over the concatenated rows (x_{rj} first).
 * dst_row  device [entries] int64: cache row entry j is written to; NULL
 *          writes entry j to row j.
 * codes/scales, w_ik, idx_dim, ik_codes/ik_scales  as in csa2_quantize_fp4
 *          (w_ik NULL: no indexer keys).
 * Enqueues two kernels on the stream: the compressor with the FP4 write,
 * then (w_ik given) the key derivation, which reads the rows just written.
 * tokens, w_c and the cache planes must not overlap.
 * Errors: BAD_SHAPE (entries < 0, ratio outside 1..16, d_in % 32 != 0,
 *         d_in > 8192, ratio * d_in > 16384, dim % 32 != 0), UNSUPPORTED
 *         (dim > 512, entries > 2^31, idx_dim), NULL_ARG, MISALIGNED (tokens
 *         or w_c not 16-byte aligned, codes or ik_codes not 8-byte aligned),
 *         HIP.
 * ------------------------------------------------------------------- */
int32_t csa2_compress_fp4(const uint16_t *tokens, int64_t entries, int32_t ratio, int32_t d_in,
                          const uint16_t *w_c, int32_t dim, const int64_t *dst_row, uint8_t *codes,
                          uint8_t *scales, const float *w_ik, int32_t idx_dim, uint8_t *ik_codes,
                          uint8_t *ik_scales, void *stream);

/* ---------------------------------------------------------------------
 * csa2_quantize_fp8_rows - window-KV write (P2 section 03 / P5 section
 * "缓存精度与持久化分层": the sliding-window KV stays FP8).
 *
 * Row scale r = fp32(amax/448) (1 for an all-zero row); code = E4M3 nearest
 * to fp32(x/r) (ties to even, saturating at 448); both divisions correctly
 * rounded fp32.  x device [rows][dim] fp32|bf16; dst_row as above; codes
 * device [.][dim]; scale device [.].
 * Errors: NULL_ARG, BAD_SHAPE (rows < 0, dim <= 0, dim % 16 != 0), BAD_DTYPE, HIP.
 * ------------------------------------------------------------------- */
int32_t csa2_quantize_fp8_rows(const void *x, int32_t x_dtype, int64_t rows, int32_t dim,
                               const int64_t *dst_row, uint8_t *codes, float *scale,
                               void *stream);

/* ---------------------------------------------------------------------
 * csa2_dequant_fp4 - exact decode of FP4 rows to fp32 (a probe of the same
 * device decode the indexer and attention kernels use).
 * codes/scales device planes, out device [rows][dim] fp32.
 * Errors: NULL_ARG, BAD_SHAPE (dim % 32 != 0), HIP.
 * ------------------------------------------------------------------- */
int32_t csa2_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int32_t dim,
                         float *out, void *stream);

/* ---------------------------------------------------------------------
 * csa2_index_full - the Full layer's indexer (P1 CSA2 section; P4 section
 * 二 and mode table; P5 figure caption "Hierarchical Sparse Indexer").
 *
 * For every query: score each visible indexer entry j,
 *     s_j = sum_h w_h * max(0, q_h . DQ4(k_j)),
 * (bf16 q, fp32 w, exact products, fp32 accumulation).
 * pool_blocks > 0 (decoder): rank the 8-position blocks (aligned at 0) by
 *   their max score, keep min(P, #blocks) blocks by (max desc, block asc) as
 *   the candidate pool (written ascending, -1 padded, count in pool_count),
 *   re-score the pool's visible positions and keep the Top-K by (score
 *   desc, position asc).
 * pool_blocks == 0 (encoder / prefill): Top-K over all visible positions;
 *   pool_out and pool_count are not written and may be NULL.
 * topk_out device [m][top_k] int32, ascending positions, -1 padded.
 * topk_score device [m][top_k] fp32 or NULL: the scores of topk_out (NaN
 *   in padded slots).
 * idx        the indexer-key cache; idx->dim = d_I in {64, 128, 256}.
 * q_idx      device [m][idx_heads][d_I] bf16 (uint16 bit patterns).
 * w_idx      device [m][idx_heads] fp32.
 * Limits: 1 <= idx_heads <= 16; 1 <= top_k <= 2048; pool_blocks <= 4096.
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, WORKSPACE, HIP.
 * ------------------------------------------------------------------- */
int32_t csa2_index_workspace_size(const csa2_fp4_cache *idx, int32_t m, int32_t pool_blocks,
                                  int32_t top_k, size_t *bytes);
int32_t csa2_index_full(const csa2_fp4_cache *idx, const csa2_queries *qs,
                        const uint16_t *q_idx, const float *w_idx, int32_t idx_heads,
                        int32_t pool_blocks, int32_t top_k, int32_t *pool_out,
                        int32_t *pool_count, int32_t *topk_out, float *topk_score,
                        void *workspace, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------
 * csa2_reindex - a Reindex layer (P1 CSA2 section; P4 mode table; P5
 * section "CSA2注意力"): reuse the Full layer's indexer keys, score only the
 * positions of the Full layer's candidate pool with this layer's own
 * (q_idx, w_idx), keep the Top-K by (score desc, position asc).
 * pool_in device [m][pool_blocks] block ids as written by csa2_index_full
 * (ascending, -1 padded); pool_count device [m].  Other arguments and
 * outputs as csa2_index_full.  Workspace: csa2_index_workspace_size.
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, WORKSPACE, HIP.
 * ------------------------------------------------------------------- */
int32_t csa2_reindex(const csa2_fp4_cache *idx, const csa2_queries *qs, const uint16_t *q_idx,
                     const float *w_idx, int32_t idx_heads, const int32_t *pool_in,
                     const int32_t *pool_count, int32_t pool_blocks, int32_t top_k,
                     int32_t *topk_out, float *topk_score, void *workspace, size_t ws_bytes,
                     void *stream);

/* ---------------------------------------------------------------------
 * csa2_sparse_swa_attn - per-layer core attention over the selected main-KV
 * entries concatenated with the layer's own FP8 window rows (P5 figure
 * caption of the attention diagram: Selection / Top-K / Concatenation; P1
 * CSA2 section: every layer keeps its own query and window KV).
 *
 * For query i and head h, over keys K = [DQ4(kv row of j) for valid j in
 * topk[i]] ++ [DQ8(window row)] (keys double as values, MQA over the shared
 * latent; no RoPE is applied - entries are stored post-RoPE, P5 section
 * "缓存精度与持久化分层"):
 *     z = softmax_scale * q_h . k ;  o_h = softmax(z) . K ;  lse_h = log sum exp z
 * q    device [m][heads][dim], fp32 or bf16 (q_dtype); kv->dim == swa->dim == dim.
 *      Arithmetic: keys are exact (FP4/FP8 values are bf16 and f16
 *      numbers); q.k products are exact and accumulate in fp32; the
 *      probabilities entering P V are rounded once to f16 (relative
 *      2^-11).  Query range: with few queries (m * ceil(heads/64) < 256,
 *      the decode schedule) bf16 queries are used as they are, any bf16
 *      value; with many queries the kernels convert bf16 to f16, so |q|
 *      must stay <= 65504 and values below 2^-14 become f16 subnormals
 *      (absolute error <= 2^-25).  fp32 queries are split into hi + lo f16
 *      parts (same range).
 * out  device [m][heads][dim] fp32.  lse device [m][heads] fp32 or NULL.
 * Limits: dim in {64, 128, 256, 512}; 1 <= heads <= 256; top_k <= 2048;
 *         window <= 1024.
 * Workspace: csa2_attn_workspace_size bytes (256-byte aligned), owned by
 *   the caller; no initial contents needed.  With few queries (m * ceil(
 *   heads/64) < 256) it holds the decode schedule's intermediates: f16
 *   probabilities per (query, head, key slot) and per-32-slot statistics;
 *   otherwise 256 bytes suffice.  Calls that run at the same time must not
 *   share a workspace.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, UNSUPPORTED, WORKSPACE, HIP.
 * ------------------------------------------------------------------- */
int32_t csa2_attn_workspace_size(int32_t m, int32_t heads, int32_t dim, int32_t top_k,
                                 int32_t window, size_t *bytes);
int32_t csa2_sparse_swa_attn(const csa2_fp4_cache *kv, const csa2_queries *qs, const void *q,
                             int32_t q_dtype, int32_t heads, const int32_t *topk,
                             int32_t top_k, const csa2_swa *swa, float softmax_scale,
                             float *out, float *lse, void *workspace, size_t ws_bytes,
                             void *stream);

/* ---------------------------------------------------------------------
 * csa2_group_step - one CSA2 layer group in the pages' static layout (P1
 * CSA2 section; P4 section 二): a Full or Reindex layer followed by Reuse
 * layers that copy its Top-K list and skip the indexer; every layer
 * attends with its own query and window rows.  Decoder: 5 groups of 4 at
 * ratio 1 (Full+3 Reuse, then Reindex+3 Reuse); encoder: 3 groups of 6 at
 * ratio 2 (Full+5 Reuse, flat Top-K: pool_blocks == 0).
 *
 * Enqueues, in order: (FULL, new_rows > 0) csa2_quantize_fp4 of the new
 * entries with their indexer keys; csa2_index_full (FULL) or csa2_reindex
 * (REINDEX); then csa2_sparse_swa_attn for layer 0 .. n_layers-1, all on the
 * group's single Top-K list.  All pointers inside are as documented on those
 * calls; the per-layer arrays are host arrays of n_layers entries.
 * Errors: those of the calls it makes, plus NULL_ARG / BAD_SHAPE for the
 * descriptor itself.
 * ------------------------------------------------------------------- */
typedef struct csa2_group_desc {
  int32_t first_mode;          /* CSA2_MODE_FULL or CSA2_MODE_REINDEX */
  int32_t n_layers;            /* 1 + number of Reuse layers */
  /* write path (FULL only; new_rows == 0 skips it) */
  const void *new_kv;          /* device [new_rows][kv.dim] */
  int32_t new_kv_dtype;
  int64_t new_rows;
  const int64_t *new_dst_row;  /* device [new_rows] cache rows */
  const float *w_ik;           /* device [kv.dim][idx.dim] */
  /* caches of the group's Full layer */
  csa2_fp4_cache kv;           /* main latent KV */
  csa2_fp4_cache idx;          /* indexer keys */
  csa2_queries qs;
  /* indexer of the first layer */
  const uint16_t *q_idx;
  const float *w_idx;
  int32_t idx_heads;
  int32_t pool_blocks;
  int32_t top_k;
  int32_t *pool;               /* device [m][pool_blocks]: FULL writes, REINDEX reads */
  int32_t *pool_count;         /* device [m] */
  int32_t *topk;               /* device [m][top_k]: the group's list */
  float *topk_score;           /* device [m][top_k] or NULL */
  /* per-layer attention (host arrays of n_layers) */
  const void *const *q;
  int32_t q_dtype;
  int32_t heads;
  const csa2_swa *swa;
  float *const *out;
  float *const *lse;           /* NULL, or an array whose entries may be NULL */
  float softmax_scale;
} csa2_group_desc;

/* Workspace of csa2_group_step: csa2_group_workspace_size bytes, 256-byte
 * aligned, no initial contents needed; not shared by calls that run at the
 * same time.  The group's layers run their attention together (batches of
 * up to 24 layers share one decoded copy of each Top-K key chunk), which
 * gives the same results as csa2_sparse_swa_attn layer by layer. */
int32_t csa2_group_workspace_size(const csa2_group_desc *g, size_t *bytes);
int32_t csa2_group_step(const csa2_group_desc *g, void *workspace, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------
 * csa2_group_steps - n_groups group steps in one call (P1 CSA2 section /
 * P4 section 二: a stack of layer groups, e.g. the decoder's 5 groups of 4
 * layers), with the same results as csa2_group_step on each group in order.
 *
 * Every group's write path and first-layer indexer are enqueued in group
 * order; a FULL group with a pool and the REINDEX groups after it that read
 * that pool (same indexer cache, queries, pool_blocks, top_k and idx_heads;
 * up to 8 groups) re-score and select their Top-K lists together (one launch
 * pair).  The attention of all their layers follows in batches of up to 24
 * layers across groups (one logits and one P V launch per batch; a layer
 * reads its own group's Top-K list).  Consecutive groups share a batch when
 * they have the same main cache, queries, query format, heads, top_k and
 * softmax scale.  The attention of earlier groups is enqueued before a FULL
 * group whose write path writes into a main cache they read.
 * groups    host array [n_groups], 1 <= n_groups <= 32, each as documented
 *           for csa2_group_step (a REINDEX group may read the pool a FULL
 *           group of the same call writes).
 * workspace csa2_group_steps_workspace_size bytes, 256-byte aligned, no
 *           initial contents needed; not shared by concurrent calls.
 * Errors: those of csa2_group_step for any group (nothing is enqueued
 * then); BAD_SHAPE for n_groups outside 1..32.
 * ------------------------------------------------------------------- */
int32_t csa2_group_steps_workspace_size(const csa2_group_desc *groups, int32_t n_groups, size_t *bytes);
int32_t csa2_group_steps(const csa2_group_desc *groups, int32_t n_groups, void *workspace, size_t ws_bytes,
                         void *stream);

/* ---------------------------------------------------------------------
 * csa2_group_step_static - csa2_group_step without a caller workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *
 * Runs exactly csa2_group_step(g, scratch, CSA2_STATIC_SCRATCH_BYTES,
 * stream) on a scratch array the library owns: one copy of
 * CSA2_STATIC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine) and needs no initial scratch contents, so
 * calls of any shape follow one another with nothing to clear.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and must be ordered
 * by the caller, e.g. on one stream.
 * Errors: those of csa2_group_step; CSA2_ERR_WORKSPACE when the group's
 * csa2_group_workspace_size exceeds CSA2_STATIC_SCRATCH_BYTES (large prefill
 * chunks do; decode batches of a few dozen sequences at 1M entries fit);
 * CSA2_ERR_HIP if the scratch address cannot be obtained.
 * ------------------------------------------------------------------- */
#define CSA2_STATIC_SCRATCH_BYTES (64u << 20)
int32_t csa2_group_step_static(const csa2_group_desc *g, void *stream);

/* ---------------------------------------------------------------------
 * csa2_profile_scan / csa2_profile_scan_read - timing of the Full layer's
 * first scan (the step whose cost grows with the context, P4 section 二):
 * the decoder's scan over every visible entry, or the multi-query scoring
 * kernel of the flat (prefill) indexer.
 * While enabled, every first-scan kernel launched by csa2_index_full /
 * csa2_group_step gets two HIP events that its own dispatch stamps with its
 * start and end times (an extended launch on its stream), so the elapsed time
 * is the kernel's alone.  Launches made while disabled are plain launches
 * (safe under stream capture).  enable != 0 clears earlier records and
 * starts recording; 0 stops.
 * _read waits for the recorded events and returns the summed kernel time in
 * milliseconds and the number of launches, then clears the records.  For
 * measurement only.  Not thread-safe: each hook keeps one process-wide
 * record, so enable, the timed launches and _read belong on one host
 * thread, with no other thread launching the timed kernels meanwhile.
 * Errors: NULL_ARG (read with a NULL output), HIP.
 * ------------------------------------------------------------------- */
int32_t csa2_profile_scan(int32_t enable);
int32_t csa2_profile_scan_read(double *total_ms, int64_t *launches);

/* csa2_profile_attn / csa2_profile_attn_read - the same timing for every
 * attention kernel launched by csa2_sparse_swa_attn / csa2_group_step (the
 * decode schedule launches a logits and a P V kernel per batch of up to 24
 * layers, the many-query schedules one kernel per layer).  Same contract
 * and errors as csa2_profile_scan. */
int32_t csa2_profile_attn(int32_t enable);
int32_t csa2_profile_attn_read(double *total_ms, int64_t *launches);

/* csa2_profile_write / csa2_profile_write_read - the same timing for every
 * FP4 quantise-on-write kernel launched by csa2_quantize_fp4 /
 * csa2_group_step (one launch per call or Full group with new rows; the FP8
 * window write is not included) and every key-derivation launch of
 * csa2_compress_fp4.  Same contract and errors as
 * csa2_profile_scan. */
int32_t csa2_profile_write(int32_t enable);
int32_t csa2_profile_write_read(double *total_ms, int64_t *launches);

/* csa2_profile_compress / csa2_profile_compress_read - the same timing for
 * every compressor kernel launched by csa2_compress_fp4 (one per call; its
 * key-derivation launch counts under csa2_profile_write).  Same contract and
 * errors as csa2_profile_scan. */
int32_t csa2_profile_compress(int32_t enable);
int32_t csa2_profile_compress_read(double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
