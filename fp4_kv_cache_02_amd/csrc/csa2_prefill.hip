// CSA2 flat Top-K indexer for encoder prefill chunks (P4 section 二: encoder
// groups select without a candidate pool).
#include "csa2_internal.hpp"

namespace csa2 {

size_t flat_ws_bytes(int64_t max_len, int m, int top_k) {
  (void)max_len; (void)m; (void)top_k;
  return 256;
}

int launch_index_flat(const csa2_fp4_cache &idx, const csa2_queries &qs, const uint16_t *q_idx,
                      const float *w_idx, int heads, int top_k, int32_t *topk_out, float *topk_score, void *ws,
                      hipStream_t stream) {
  (void)idx; (void)qs; (void)q_idx; (void)w_idx; (void)heads; (void)top_k; (void)topk_out; (void)topk_score;
  (void)ws; (void)stream;
  return CSA2_ERR_UNSUPPORTED;
}

}  // namespace csa2
