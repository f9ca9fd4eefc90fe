"""C ABI checks that need no GPU: exports, struct layout, host-side validation."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import fp4_kv_cache_02_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

NULL_ARG, BAD_SHAPE, BAD_DTYPE, MISALIGNED, WORKSPACE, UNSUPPORTED = -1, -2, -3, -4, -5, -6
FAKE = 0x10000          # a 256-aligned non-null address; validation never dereferences it


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|const char \*)\s*(csa2_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = csa2.lib()
    names = declared_functions()
    assert len(names) == 24
    assert sorted(names) == sorted(csa2.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", csa2.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (csa2_\w+)$", out, re.M))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_abi_version_and_status_strings():
    assert csa2.csa2_abi_version() == 2
    assert csa2.status_string(0) == "ok"
    assert csa2.status_string(WORKSPACE).startswith("workspace")
    assert csa2.status_string(12345) == "unknown status"


def test_struct_layout_matches_header():
    src = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "csa2.h"
    int main(void) {
      printf("%zu %zu %zu %zu\n", sizeof(csa2_fp4_cache), sizeof(csa2_queries), sizeof(csa2_swa),
             sizeof(csa2_group_desc));
      printf("%zu %zu %zu %zu %zu\n", offsetof(csa2_group_desc, kv), offsetof(csa2_group_desc, q_idx),
             offsetof(csa2_group_desc, q), offsetof(csa2_group_desc, softmax_scale),
             offsetof(csa2_group_desc, new_rows));
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.c")
        exe = os.path.join(d, "probe")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    sizes = [int(v) for v in lines[0].split()]
    offs = [int(v) for v in lines[1].split()]
    assert sizes == [ctypes.sizeof(csa2.Fp4Cache), ctypes.sizeof(csa2.Queries), ctypes.sizeof(csa2.Swa),
                     ctypes.sizeof(csa2.GroupDesc)]
    G = csa2.GroupDesc
    assert offs == [G.kv.offset, G.q_idx.offset, G.q.offset, G.softmax_scale.offset, G.new_rows.offset]


def _lib():
    return csa2.lib()


def test_quantize_validation():
    L = _lib()
    assert L.csa2_quantize_fp4(FAKE, 0, 10, 100, None, FAKE, FAKE, None, 0, None, None, None) == BAD_SHAPE
    assert L.csa2_quantize_fp4(FAKE, 0, -1, 128, None, FAKE, FAKE, None, 0, None, None, None) == BAD_SHAPE
    assert L.csa2_quantize_fp4(FAKE, 7, 10, 128, None, FAKE, FAKE, None, 0, None, None, None) == BAD_DTYPE
    assert L.csa2_quantize_fp4(None, 0, 10, 128, None, FAKE, FAKE, None, 0, None, None, None) == NULL_ARG
    assert L.csa2_quantize_fp4(FAKE, 0, 10, 128, None, FAKE + 4, FAKE, None, 0, None, None, None) == MISALIGNED
    assert L.csa2_quantize_fp4(FAKE, 0, 10, 128, None, FAKE, FAKE, FAKE, 48, FAKE, FAKE, None) == UNSUPPORTED
    assert L.csa2_quantize_fp4(FAKE, 0, 10, 128, None, FAKE, FAKE, FAKE, 64, None, FAKE, None) == NULL_ARG
    assert L.csa2_quantize_fp4(FAKE, 0, 0, 128, None, None, None, None, 0, None, None, None) == 0   # empty = no-op
    assert L.csa2_quantize_fp8_rows(FAKE, 0, 4, 100, None, FAKE, FAKE, None) == BAD_SHAPE
    assert L.csa2_quantize_fp8_rows(FAKE, 0, 4, 128, None, None, FAKE, None) == NULL_ARG
    assert L.csa2_dequant_fp4(FAKE, FAKE, 4, 48, FAKE, None) == BAD_SHAPE


def _cache(dim=128, max_len=4096, ratio=1, codes=FAKE):
    return csa2.Fp4Cache(codes, FAKE, FAKE, FAKE, 1, dim, max_len, ratio)


def test_compress_validation():
    L = csa2.lib()
    ok = dict(tokens=FAKE, entries=10, ratio=2, d_in=512, w_c=FAKE, dim=512, dst=None, codes=FAKE, scales=FAKE,
              w_ik=FAKE, di=128, ikc=FAKE, iks=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return L.csa2_compress_fp4(a["tokens"], a["entries"], a["ratio"], a["d_in"], a["w_c"], a["dim"], a["dst"],
                                   a["codes"], a["scales"], a["w_ik"], a["di"], a["ikc"], a["iks"], None)

    assert call(entries=-1) == BAD_SHAPE
    assert call(ratio=0) == BAD_SHAPE
    assert call(ratio=17) == BAD_SHAPE
    assert call(d_in=48) == BAD_SHAPE
    assert call(d_in=8192, ratio=4) == BAD_SHAPE          # ratio * d_in > 16384
    assert call(dim=100) == BAD_SHAPE
    assert call(dim=1024) == UNSUPPORTED
    assert call(tokens=None) == NULL_ARG
    assert call(w_c=None) == NULL_ARG
    assert call(ikc=None) == NULL_ARG
    assert call(tokens=FAKE + 8) == MISALIGNED
    assert call(w_c=FAKE + 2) == MISALIGNED
    assert call(codes=FAKE + 4) == MISALIGNED
    assert call(di=48) == UNSUPPORTED
    assert call(di=256, dim=128) == UNSUPPORTED           # key wider than the entry
    assert call(entries=0, tokens=None, w_c=None) == 0    # empty = no-op


def test_index_validation():
    L = _lib()
    qs = csa2.Queries(FAKE, FAKE, 2)
    ws = ctypes.c_size_t(0)
    c = _cache()
    assert L.csa2_index_workspace_size(ctypes.byref(c), 2, 2048, 512, ctypes.byref(ws)) == 0 and ws.value > 0
    base = ws.value
    assert L.csa2_index_workspace_size(ctypes.byref(c), 4, 2048, 512, ctypes.byref(ws)) == 0 and ws.value > base

    def call(cache=c, q=qs, heads=8, pool=64, k=64, wsb=base, wsp=FAKE, pool_out=FAKE):
        return L.csa2_index_full(ctypes.byref(cache), ctypes.byref(q), FAKE, FAKE, heads, pool, k, pool_out, FAKE,
                                 FAKE, None, wsp, wsb, None)
    assert call(cache=_cache(dim=100)) == BAD_SHAPE
    assert call(cache=_cache(dim=96)) == UNSUPPORTED
    assert call(cache=_cache(ratio=0)) == BAD_SHAPE
    assert call(cache=_cache(codes=FAKE + 8)) == MISALIGNED
    assert call(heads=0) == BAD_SHAPE
    assert call(heads=17) == UNSUPPORTED
    assert call(k=0) == BAD_SHAPE
    assert call(k=4096) == UNSUPPORTED
    assert call(pool=-1) == BAD_SHAPE
    assert call(pool=8192) == UNSUPPORTED
    assert call(pool_out=None) == NULL_ARG
    assert call(wsp=None) == WORKSPACE
    assert call(wsb=16) == WORKSPACE
    assert call(wsp=FAKE + 64) == MISALIGNED
    assert call(q=csa2.Queries(None, FAKE, 2)) == NULL_ARG
    # flat (pool 0) indexer: more than 65,536 blocks per sequence is refused
    # before anything is enqueued, whatever the workspace
    big = _cache(max_len=65536 * 8 + 1)
    assert call(cache=big, pool=0) == UNSUPPORTED
    assert call(cache=big, pool=0, wsp=None) == UNSUPPORTED
    assert call(q=csa2.Queries(None, None, 0)) == 0          # no queries: nothing to do
    assert L.csa2_reindex(ctypes.byref(c), ctypes.byref(qs), FAKE, FAKE, 8, FAKE, FAKE, 0, 64, FAKE, None, FAKE,
                          base, None) == BAD_SHAPE
    assert L.csa2_reindex(ctypes.byref(c), ctypes.byref(qs), FAKE, FAKE, 8, None, FAKE, 64, 64, FAKE, None, FAKE,
                          base, None) == NULL_ARG


def test_attention_validation():
    L = _lib()
    qs = csa2.Queries(FAKE, FAKE, 1)
    kv = _cache(dim=512)
    sw = csa2.Swa(FAKE, FAKE, FAKE, FAKE, 512, 128)
    n = ctypes.c_size_t(0)
    assert L.csa2_attn_workspace_size(1, 64, 512, 512, 128, ctypes.byref(n)) == 0 and n.value >= 256
    need = n.value

    def call(kv=kv, sw=sw, dtype=1, heads=64, k=512, wsp=FAKE, wsb=need):
        return L.csa2_sparse_swa_attn(ctypes.byref(kv), ctypes.byref(qs), FAKE, dtype, heads, FAKE, k,
                                      ctypes.byref(sw), 0.04, FAKE, None, wsp, wsb, None)
    assert call(dtype=5) == BAD_DTYPE
    assert call(dtype=0) == UNSUPPORTED                      # fp32 queries at dim 512
    assert call(kv=_cache(dim=320), sw=csa2.Swa(FAKE, FAKE, FAKE, FAKE, 320, 128)) == UNSUPPORTED
    assert call(sw=csa2.Swa(FAKE, FAKE, FAKE, FAKE, 256, 128)) == BAD_SHAPE
    assert call(sw=csa2.Swa(None, FAKE, FAKE, FAKE, 512, 128)) == NULL_ARG
    assert call(sw=csa2.Swa(FAKE, FAKE, FAKE, FAKE, 512, 4096)) == UNSUPPORTED
    assert call(heads=0) == BAD_SHAPE
    assert call(k=0, sw=csa2.Swa(None, None, None, None, 512, 0)) == BAD_SHAPE
    if need > 256:
        assert call(wsp=None) == WORKSPACE


def test_group_validation():
    L = _lib()
    g = csa2.GroupDesc()
    assert L.csa2_group_step(ctypes.byref(g), FAKE, 1 << 20, None) == BAD_SHAPE   # n_layers = 0
    g.n_layers = 4
    g.first_mode = 3
    assert L.csa2_group_step(ctypes.byref(g), FAKE, 1 << 20, None) == BAD_SHAPE
    g.first_mode = csa2.CSA2_MODE_FULL
    assert L.csa2_group_step(ctypes.byref(g), FAKE, 1 << 20, None) == NULL_ARG      # per-layer arrays missing
    arr = (csa2.GroupDesc * 2)(g, g)
    n = ctypes.c_size_t(0)
    assert L.csa2_group_steps(None, 1, FAKE, 1 << 20, None) == NULL_ARG
    assert L.csa2_group_steps(arr, 0, FAKE, 1 << 20, None) == BAD_SHAPE
    assert L.csa2_group_steps(arr, 33, FAKE, 1 << 20, None) == BAD_SHAPE
    assert L.csa2_group_steps(arr, 2, FAKE, 1 << 20, None) == NULL_ARG           # a group's checks apply
    assert L.csa2_group_steps_workspace_size(arr, 0, ctypes.byref(n)) == BAD_SHAPE


def _group_desc(n_layers=2, pool_blocks=64, idx_len=4096):
    """A Full group descriptor whose pointers are never dereferenced (every
    call below is refused by the host checks)."""
    keep = []
    g = csa2.GroupDesc()
    g.first_mode, g.n_layers = csa2.CSA2_MODE_FULL, n_layers
    g.kv = _cache(dim=512)
    g.idx = _cache(dim=128, max_len=idx_len)
    g.qs = csa2.Queries(FAKE, FAKE, 1)
    g.q_idx, g.w_idx, g.idx_heads, g.pool_blocks, g.top_k = FAKE, FAKE, 8, pool_blocks, 64
    g.pool, g.pool_count, g.topk = FAKE, FAKE, FAKE
    q = (ctypes.c_void_p * n_layers)(*([FAKE] * n_layers))
    out = (ctypes.c_void_p * n_layers)(*([FAKE] * n_layers))
    sw = (csa2.Swa * n_layers)(*([csa2.Swa(FAKE, FAKE, FAKE, FAKE, 512, 128)] * n_layers))
    keep += [q, out, sw]
    g.q = ctypes.cast(q, ctypes.POINTER(ctypes.c_void_p))
    g.out = ctypes.cast(out, ctypes.POINTER(ctypes.c_void_p))
    g.swa = ctypes.cast(sw, ctypes.POINTER(csa2.Swa))
    g.q_dtype, g.heads, g.softmax_scale = csa2.CSA2_BF16, 64, 0.04
    return g, keep


def test_group_validation_runs_before_any_enqueue():
    L = _lib()
    g, keep = _group_desc()
    n = ctypes.c_size_t(0)
    assert L.csa2_group_workspace_size(ctypes.byref(g), ctypes.byref(n)) == 0
    # a workspace that is large enough but not 256-byte aligned
    assert L.csa2_group_step(ctypes.byref(g), FAKE + 64, n.value, None) == MISALIGNED
    # a flat Full group over a cache with more blocks than the flat indexer
    # keeps: refused up front (its write path must not run)
    g2, keep2 = _group_desc(pool_blocks=0, idx_len=65536 * 8 + 1)
    g2.new_rows, g2.new_kv, g2.new_dst_row, g2.w_ik, g2.new_kv_dtype = 16, FAKE, FAKE, FAKE, csa2.CSA2_BF16
    assert L.csa2_group_workspace_size(ctypes.byref(g2), ctypes.byref(n)) == 0
    assert L.csa2_group_step(ctypes.byref(g2), FAKE, n.value, None) == UNSUPPORTED
    # in a multi-group call every group is checked before the first is enqueued
    arr = (csa2.GroupDesc * 2)(g, g2)
    assert L.csa2_group_steps_workspace_size(arr, 2, ctypes.byref(n)) == 0
    assert L.csa2_group_steps(arr, 2, FAKE, n.value, None) == UNSUPPORTED


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(csa2, "_lib", None)
    monkeypatch.setattr(csa2, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        csa2.lib()


def test_descriptors_keep_their_tensors_alive():
    # a descriptor stores raw addresses: the tensors behind them must outlive it
    import weakref
    import torch
    refs = []

    def tmp(dtype):
        x = torch.zeros(3, dtype=dtype)
        refs.append(weakref.ref(x))
        return x
    c = csa2.fp4_cache(tmp(torch.uint8), tmp(torch.uint8), tmp(torch.int64), tmp(torch.int32), 128, 10, 1)
    q = csa2.queries(tmp(torch.int32), tmp(torch.int32))
    w = csa2.swa(tmp(torch.uint8), tmp(torch.float32), tmp(torch.int32), tmp(torch.int32), 128, 16)
    assert all(r() is not None for r in refs)
    g = csa2.Group(csa2.CSA2_MODE_FULL, c, c, q, tmp(torch.int16).view(1, 3), tmp(torch.float32), 4, 8,
                   tmp(torch.int32), tmp(torch.int32), tmp(torch.int32), None, [tmp(torch.float32)], 0, 8, [w],
                   [tmp(torch.float32)], None, 0.1)
    del c, q, w
    assert all(r() is not None for r in refs)
    del g
