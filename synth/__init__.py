"""Seeded synthetic inputs for the CSA2 hot path.

This module is shared by the HIP path's tests/benchmark and by the CPU
oracle.  It holds *no* arithmetic of the method: it only draws raw values
(Gaussian latent rows, projection weights, queries, window rows, sequence
lengths) and describes the five workload shapes.  Quantisation, indexer-key
derivation, scoring, selection and attention live in the oracle and, as an
independent implementation, in the HIP library.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence(
[ROOT_SEED, cfg, tag, layer, seq, chunk]))``.  Long row ranges are split in
chunks of ``CHUNK_ROWS`` rows, each with its own seed, so any sub-range can
be regenerated on its own (the oracle checks sampled rows of 1M-entry caches
without drawing the whole cache) and chunks can be drawn on several threads.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field
from typing import List

import numpy as np

ROOT_SEED = 20261203
CHUNK_ROWS = 1 << 16

# tensor tags of the seed sequence
TAG_MAIN_KV = 1   # pre-quantisation latent rows of the main KV cache
TAG_W_IK = 2      # indexer-key projection weight
TAG_Q_IDX = 3     # indexer queries
TAG_W_IDX = 4     # indexer head weights
TAG_Q = 5         # main attention queries
TAG_SWA = 6       # pre-quantisation sliding-window rows
TAG_LEN = 7       # ragged sequence lengths
TAG_IDX_KEY = 8   # pre-quantisation indexer-key rows when the indexer is exercised on its own
TAG_IDX_LIST = 9  # synthetic Top-K lists when attention is exercised on its own
TAG_FP4_BYTES = 10  # raw FP4 cache bytes (codes and scale bytes drawn directly)
TAG_TOKENS = 11   # pre-compression token rows fed to the compressor
TAG_W_C = 12      # compressor weight


def rng(cfg: int, tag: int, layer: int = 0, seq: int = 0, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([ROOT_SEED, cfg, tag, layer, seq, chunk]))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------------------
# raw draws
# ---------------------------------------------------------------------------

def gaussian_rows(cfg: int, tag: int, layer: int, seq: int, row0: int, nrows: int,
                  dim: int, out: np.ndarray | None = None) -> np.ndarray:
    """Rows ``row0 .. row0+nrows`` of an N(0,1) fp32 matrix [*, dim].

    Row r belongs to chunk ``r // CHUNK_ROWS``; a chunk is always drawn whole
    from its own generator, so the values of a row do not depend on which
    range is requested.
    """
    if out is None:
        out = np.empty((nrows, dim), dtype=np.float32)
    assert out.shape == (nrows, dim) and out.dtype == np.float32
    if nrows == 0:
        return out
    c0 = row0 // CHUNK_ROWS
    c1 = (row0 + nrows - 1) // CHUNK_ROWS

    def fill(c: int) -> None:
        lo = max(row0, c * CHUNK_ROWS)
        hi = min(row0 + nrows, (c + 1) * CHUNK_ROWS)
        g = rng(cfg, tag, layer, seq, c)
        if lo == c * CHUNK_ROWS and hi == (c + 1) * CHUNK_ROWS:
            g.standard_normal(out=out[lo - row0:hi - row0].reshape(-1), dtype=np.float32)
        else:
            full = np.empty(((c + 1) * CHUNK_ROWS - c * CHUNK_ROWS, dim), dtype=np.float32)
            # only the rows up to `hi` are needed; later rows of the chunk come
            # later in the stream, so drawing a prefix gives identical values
            need = hi - c * CHUNK_ROWS
            g.standard_normal(out=full[:need].reshape(-1), dtype=np.float32)
            out[lo - row0:hi - row0] = full[lo - c * CHUNK_ROWS:need]

    chunks = list(range(c0, c1 + 1))
    if len(chunks) == 1:
        fill(chunks[0])
    else:
        with _cf.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, chunks))
    return out


def main_kv_rows(cfg: int, seq: int, row0: int, nrows: int, dim: int) -> np.ndarray:
    """Pre-quantisation latent rows (positions row0..) of sequence ``seq``."""
    return gaussian_rows(cfg, TAG_MAIN_KV, 0, seq, row0, nrows, dim)


def w_ik(cfg: int, dim: int, d_idx: int) -> np.ndarray:
    """Indexer-key projection weight [dim, d_idx], N(0, 1/dim), fp32."""
    w = rng(cfg, TAG_W_IK).standard_normal((dim, d_idx), dtype=np.float32)
    return (w * np.float32(1.0 / math.sqrt(dim))).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def q_idx(cfg: int, layer: int, m: int, heads: int, d_idx: int) -> np.ndarray:
    """Indexer queries [m, heads, d_idx] as bf16 bit patterns (uint16)."""
    x = rng(cfg, TAG_Q_IDX, layer).standard_normal((m, heads, d_idx), dtype=np.float32)
    return f32_to_bf16_bits(x).reshape(m, heads, d_idx)


def w_idx(cfg: int, layer: int, m: int, heads: int) -> np.ndarray:
    """Indexer head weights [m, heads], N(0, 1/heads), fp32."""
    x = rng(cfg, TAG_W_IDX, layer).standard_normal((m, heads), dtype=np.float32)
    return (x * np.float32(1.0 / math.sqrt(heads))).astype(np.float32)


def q_main(cfg: int, layer: int, m: int, heads: int, dim: int, dtype: str) -> np.ndarray:
    """Main attention queries [m, heads, dim]: fp32 array, or bf16 bits (uint16)."""
    x = rng(cfg, TAG_Q, layer).standard_normal((m, heads, dim), dtype=np.float32)
    if dtype == "f32":
        return x
    assert dtype == "bf16"
    return f32_to_bf16_bits(x).reshape(m, heads, dim)


def swa_rows(cfg: int, layer: int, seq: int, nrows: int, dim: int, row0: int = 0) -> np.ndarray:
    """Pre-quantisation sliding-window rows of one layer and sequence."""
    return gaussian_rows(cfg, TAG_SWA, layer, seq, row0, nrows, dim)


def fp4_bytes(cfg: int, layer: int, nrows: int, dim: int):
    """Raw bytes of an FP4 cache [nrows, dim]: code bytes uniform over 0..255
    (two 4-bit codes each) and scale bytes uniform over 0x20..0x3F (positive
    E4M3 codes of the values 1/8 .. 15/8), drawn directly so that large caches
    need no quantisation pass.  Returns (codes uint8 [nrows, dim/2], scales
    uint8 [nrows, dim/16])."""
    g = rng(cfg, TAG_FP4_BYTES, layer)
    codes = g.integers(0, 256, size=(nrows, dim // 2), dtype=np.uint8)
    scales = g.integers(0x20, 0x40, size=(nrows, dim // 16), dtype=np.uint8)
    return codes, scales


def token_rows(cfg: int, layer: int, seq: int, row0: int, nrows: int, d_in: int) -> np.ndarray:
    """Pre-compression token rows row0.. of one sequence as bf16 bit patterns
    (uint16 [nrows, d_in]), N(0,1) before rounding."""
    x = gaussian_rows(cfg, TAG_TOKENS, layer, seq, row0, nrows, d_in)
    return f32_to_bf16_bits(x).reshape(nrows, d_in)


def w_c(cfg: int, layer: int, dim: int, ratio: int, d_in: int) -> np.ndarray:
    """Compressor weight as bf16 bit patterns, uint16 [dim, ratio * d_in]: row c
    holds output channel c's weights over the ratio concatenated token rows,
    N(0, 1/(ratio * d_in)) before rounding."""
    k = ratio * d_in
    x = rng(cfg, TAG_W_C, layer).standard_normal((dim, k), dtype=np.float32)
    x = (x * np.float32(1.0 / math.sqrt(k))).astype(np.float32)
    return f32_to_bf16_bits(x).reshape(dim, k)


def ragged_lengths(cfg: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Sequence lengths floor(exp(U(ln lo, ln hi))), int64."""
    u = rng(cfg, TAG_LEN).random(n)
    return np.floor(np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo)))).astype(np.int64)


# ---------------------------------------------------------------------------
# workload shapes
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    """Shape of one synthetic workload of the CSA2 hot path."""
    cfg: int
    name: str
    phase: str                 # "decode" or "prefill"
    seq_lens: List[int]        # cache entries per sequence
    dim: int                   # latent channels D
    heads: int                 # main query heads H
    q_dtype: str               # "f32" or "bf16"
    idx_heads: int             # indexer heads H_I
    idx_dim: int               # indexer dims d_I
    pool_blocks: int           # P (0 = flat top-k)
    top_k: int                 # K
    window: int                # SWA window W
    ratio: int                 # compression ratio r
    groups: List[List[str]]    # per group: modes of its layers, e.g. ["full","reuse",...]
    n_queries: int = 0         # prefill: query tokens in the chunk
    first_query_token: int = 0 # prefill: token index of the chunk's first query
    extra: dict = field(default_factory=dict)

    @property
    def n_layers(self) -> int:
        return sum(len(g) for g in self.groups)


DECODER_GROUPS = [["full", "reuse", "reuse", "reuse"]] + [["reindex", "reuse", "reuse", "reuse"]] * 4
ENCODER_GROUPS = [["full"] + ["reuse"] * 5] * 3


def workload(cfg: int) -> Workload:
    if cfg == 0:
        return Workload(0, "tiny-4k-d128", "decode", [4096], 128, 8, "f32", 4, 64, 64, 64, 128, 1,
                        [["full", "reuse", "reuse", "reuse"]])
    if cfg == 1:
        return Workload(1, "decoder-64k", "decode", [65536], 512, 64, "bf16", 8, 128, 2048, 512, 128, 1,
                        DECODER_GROUPS)
    if cfg == 2:
        # last 4,096-token chunk of a 131,072-token prompt at ratio 2
        return Workload(2, "encoder-prefill-128k", "prefill", [65536], 512, 64, "bf16", 8, 128, 0, 512, 128, 2,
                        ENCODER_GROUPS, n_queries=4096, first_query_token=131072 - 4096)
    if cfg == 3:
        lens = ragged_lengths(3, 32, 32768, 262144).tolist()
        return Workload(3, "batched-decode-32x[32k,256k]", "decode", lens, 512, 64, "bf16", 8, 128, 2048, 512,
                        128, 1, DECODER_GROUPS)
    if cfg == 4:
        return Workload(4, "long-decode-4x1m", "decode", [1 << 20] * 4, 512, 64, "bf16", 8, 128, 2048, 512, 128,
                        1, DECODER_GROUPS)
    if cfg == 5:
        # one decode token through the whole 40-layer encoder-decoder: the
        # encoder's 2 window-only layers and 3 groups at ratio 2 over the
        # tokens' 524,288 compressed entries, then the 20-layer decoder
        return Workload(5, "ced-decode-4x1m", "decode", [1 << 20] * 4, 512, 64, "bf16", 8, 128, 2048, 512, 128,
                        1, DECODER_GROUPS,
                        extra={"encoder_groups": ENCODER_GROUPS, "encoder_ratio": 2, "encoder_pool_blocks": 512,
                               "swa_only_layers": 2})
    if cfg == 6:
        # several decode tokens per sequence (drafted positions verified together)
        return Workload(6, "multi-token-decode-4x1m-t4", "decode", [1 << 20] * 4, 512, 64, "bf16", 8, 128, 2048,
                        512, 128, 1, DECODER_GROUPS, extra={"tokens_per_seq": 4})
    if cfg == 7:
        # the decoder's window state rebuilt by replaying the last 128 tokens of a 1M-token prompt
        return Workload(7, "replay-128-1m", "decode", [1 << 20], 512, 64, "bf16", 8, 128, 2048, 512, 128, 1,
                        DECODER_GROUPS, extra={"tokens_per_seq": 128})
    raise ValueError(cfg)
