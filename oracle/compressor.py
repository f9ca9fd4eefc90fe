"""Oracle: the CSA2 compressor (ratio r) fused with quantise-on-write.

Test infrastructure only (see ``oracle/__init__``).

What the pages fix (P4 section 二 "CSA2：沿层轴压缩缓存"; P5 section
"CSA2注意力"; P1 CSA2 section): a CSA2 layer's global entries come from a
compressor at ratio r (2 in the 18 encoder layers, 1 in the 20 decoder
layers); CSA2's compressor, unlike CSA's, has no overlap between adjacent
compressed entries and no absolute position embedding; the indexer key is
projected from the main-KV entry rather than compressed separately from the
hidden states.  The pages give neither the compressor's form nor its
weights.  Reading taken (the plainest one those facts support):

* entry j of a sequence is a linear map of the concatenation of its own r
  token rows, c_j = W_c^T [x_{rj}; x_{rj+1}; ...; x_{rj+r-1}]: every token
  row feeds exactly one entry (no overlap) and no position term is added;
* token rows and W_c are bf16 values (W_c synthetic, [dim, r * d_in], row c
  holding output channel c's weights); the sum is accumulated in fp64 and
  rounded once to fp32 (every product of two bf16 values is exact in fp64,
  so the fp32 result does not depend on the summation order except within
  ~2^-50 of an fp32 rounding boundary); a zero sum is +0;
* c_j is then written like any other main-KV row: FP4-encoded
  (``codec.fp4_encode``) with its indexer key Q4(fp32(W_ik^T DQ4(c_j)))
  (``codec.indexer_key``).

Parity pins (tests/test_oracle_compressor.py): selection weights [I 0] and
[0 I] return the even and the odd token rows; [I/2 I/2] returns the exact
pair average rounded to fp32; a permutation at ratio 1 permutes channels;
entry j depends only on its own r token rows; exact-rational brute force of
the whole fused write (compressor, FP4 codes, indexer key) on small inputs.
"""
from __future__ import annotations

import numpy as np

from .codec import fp4_encode, indexer_key


def compress_entries(tokens: np.ndarray, w_c: np.ndarray, ratio: int) -> np.ndarray:
    """Compressed entries fp32(W_c^T [x_{rj}; ...; x_{rj+r-1}]), [n, dim].

    tokens [n * ratio, d_in] (values of the bf16 rows), w_c [dim, ratio * d_in]
    (values of the bf16 weights).  Entry j reads token rows r j .. r j + r - 1
    only; their concatenation is row j of tokens viewed as [n, r * d_in].
    """
    x = np.asarray(tokens, dtype=np.float64)
    w = np.asarray(w_c, dtype=np.float64)
    n_tok, d_in = x.shape
    assert ratio >= 1 and n_tok % ratio == 0
    n = n_tok // ratio
    assert w.shape[1] == ratio * d_in
    concat = x.reshape(n, ratio * d_in)
    return ((concat @ w.T) + 0.0).astype(np.float32)


def compress_write(tokens: np.ndarray, w_c: np.ndarray, ratio: int, w_ik: np.ndarray):
    """The fused write: (codes, scales, ik_codes, ik_scales) of the compressed entries."""
    c = compress_entries(tokens, w_c, ratio)
    codes, scales = fp4_encode(c)
    ik_codes, ik_scales = indexer_key(codes, scales, w_ik)
    return codes, scales, ik_codes, ik_scales
