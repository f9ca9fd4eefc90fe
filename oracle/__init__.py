"""CPU oracle of the CSA2 hot path (test infrastructure).

Plain, slow, fp64 NumPy code that states what each step of the hot path
computes.  It is test infrastructure only: the tests, the smoke check and the
CPU-baseline leg of the benchmark may import it; the library and its Python
binding never do, and the oracle imports nothing from them.

Citations name the source pages by these keys (title, address):

* P1 - "DeepSeek-V4.1-Flash 发布：100 万上下文 + FP4 KV Cache + 跨层注意力复用"
  (feinterview.poetries.top, Chinese translation of a MarkTechPost item)
* P2 - "DeepSeek V4.1 Flash 发布，百万上下文开始算缓存这笔账"
  (cnblogs.com/OpenCSG)
* P3 - "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
  (arxivdaily.com abstract page)
* P4 - DeepSeek V4.1-Flash CED / CSA2 paper notes (yomxxx.com, 2026-09-14)
* P5 - "V4.1 Flash 内测登场：40 天改架构、调用价不变" (tucaod.com)

Where the pages are silent the oracle takes one reading and says so in the
docstring; every reading is listed in the design doc.

Parity status per function (what pins it) is in each module header.
"""
from . import codec, compressor, indexer, attention, group  # noqa: F401
