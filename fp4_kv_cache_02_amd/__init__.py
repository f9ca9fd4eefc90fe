"""Python binding of the CSA2 hot-path library (libcsa2.so, gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in include/csa2.h.  Tensors are torch tensors on the GPU; the
binding passes their data pointers and the current HIP stream.  There is no
CPU fallback: if the library is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint16, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")

CSA2_OK = 0
CSA2_F32, CSA2_BF16 = 0, 1
CSA2_MODE_FULL, CSA2_MODE_REINDEX = 0, 1
CSA2_STATIC_SCRATCH_BYTES = 64 << 20   # include/csa2.h

EXPORTS = [
    "csa2_abi_version", "csa2_status_string", "csa2_quantize_fp4", "csa2_quantize_fp8_rows",
    "csa2_dequant_fp4", "csa2_index_workspace_size", "csa2_index_full", "csa2_reindex",
    "csa2_attn_workspace_size", "csa2_sparse_swa_attn", "csa2_group_workspace_size", "csa2_group_step",
    "csa2_profile_scan", "csa2_profile_scan_read", "csa2_profile_attn", "csa2_profile_attn_read",
    "csa2_profile_write", "csa2_profile_write_read", "csa2_group_step_static", "csa2_compress_fp4",
    "csa2_profile_compress", "csa2_profile_compress_read", "csa2_group_steps_workspace_size", "csa2_group_steps",
]


class Csa2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class Fp4Cache(ctypes.Structure):
    _fields_ = [("codes", c_void_p), ("scales", c_void_p), ("seq_start", c_void_p), ("seq_len", c_void_p),
                ("n_seq", c_int32), ("dim", c_int32), ("max_len", c_int32), ("ratio", c_int32)]


class Queries(ctypes.Structure):
    _fields_ = [("seq", c_void_p), ("pos", c_void_p), ("m", c_int32), ("run", c_int32)]


class Swa(ctypes.Structure):
    _fields_ = [("codes", c_void_p), ("scale", c_void_p), ("start", c_void_p), ("count", c_void_p),
                ("dim", c_int32), ("window", c_int32)]


class GroupDesc(ctypes.Structure):
    _fields_ = [
        ("first_mode", c_int32), ("n_layers", c_int32),
        ("new_kv", c_void_p), ("new_kv_dtype", c_int32), ("new_rows", c_int64), ("new_dst_row", c_void_p),
        ("w_ik", c_void_p),
        ("kv", Fp4Cache), ("idx", Fp4Cache), ("qs", Queries),
        ("q_idx", c_void_p), ("w_idx", c_void_p), ("idx_heads", c_int32), ("pool_blocks", c_int32),
        ("top_k", c_int32),
        ("pool", c_void_p), ("pool_count", c_void_p), ("topk", c_void_p), ("topk_score", c_void_p),
        ("q", POINTER(c_void_p)), ("q_dtype", c_int32), ("heads", c_int32), ("swa", POINTER(Swa)),
        ("out", POINTER(c_void_p)), ("lse", POINTER(c_void_p)), ("softmax_scale", c_float),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"CSA2 HIP library not built: {LIB_PATH} is missing "
                               "(run `python -m fp4_kv_cache_02_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = c_void_p, c_int32, c_int64, c_size_t
        sig = {
            "csa2_abi_version": (i32, []),
            "csa2_status_string": (ctypes.c_char_p, [i32]),
            "csa2_quantize_fp4": (i32, [vp, i32, i64, i32, vp, vp, vp, vp, i32, vp, vp, vp]),
            "csa2_quantize_fp8_rows": (i32, [vp, i32, i64, i32, vp, vp, vp, vp]),
            "csa2_dequant_fp4": (i32, [vp, vp, i64, i32, vp, vp]),
            "csa2_index_workspace_size": (i32, [POINTER(Fp4Cache), i32, i32, i32, POINTER(c_size_t)]),
            "csa2_index_full": (i32, [POINTER(Fp4Cache), POINTER(Queries), vp, vp, i32, i32, i32, vp, vp, vp, vp,
                                      vp, sz, vp]),
            "csa2_reindex": (i32, [POINTER(Fp4Cache), POINTER(Queries), vp, vp, i32, vp, vp, i32, i32, vp, vp, vp,
                                   sz, vp]),
            "csa2_attn_workspace_size": (i32, [i32, i32, i32, i32, i32, POINTER(c_size_t)]),
            "csa2_sparse_swa_attn": (i32, [POINTER(Fp4Cache), POINTER(Queries), vp, i32, i32, vp, i32,
                                           POINTER(Swa), c_float, vp, vp, vp, sz, vp]),
            "csa2_group_workspace_size": (i32, [POINTER(GroupDesc), POINTER(c_size_t)]),
            "csa2_group_step": (i32, [POINTER(GroupDesc), vp, sz, vp]),
            "csa2_profile_scan": (i32, [i32]),
            "csa2_profile_scan_read": (i32, [POINTER(ctypes.c_double), POINTER(c_int64)]),
            "csa2_profile_attn": (i32, [i32]),
            "csa2_profile_attn_read": (i32, [POINTER(ctypes.c_double), POINTER(c_int64)]),
            "csa2_profile_write": (i32, [i32]),
            "csa2_profile_write_read": (i32, [POINTER(ctypes.c_double), POINTER(c_int64)]),
            "csa2_group_step_static": (i32, [POINTER(GroupDesc), vp]),
            "csa2_compress_fp4": (i32, [vp, i64, i32, i32, vp, i32, vp, vp, vp, vp, i32, vp, vp, vp]),
            "csa2_profile_compress": (i32, [i32]),
            "csa2_profile_compress_read": (i32, [POINTER(ctypes.c_double), POINTER(c_int64)]),
            "csa2_group_steps_workspace_size": (i32, [POINTER(GroupDesc), i32, POINTER(c_size_t)]),
            "csa2_group_steps": (i32, [POINTER(GroupDesc), i32, vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().csa2_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != CSA2_OK:
        raise Csa2Error(status, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return CSA2_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return CSA2_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

# The descriptors below hold raw device addresses; each keeps a reference to
# the tensors it points at (attribute `_keep`) so they outlive the descriptor.

def fp4_cache(codes, scales, seq_start, seq_len, dim: int, max_len: int, ratio: int = 1) -> Fp4Cache:
    """Describe an FP4 cache (codes [rows, dim/2] u8, scales [rows, dim/16] u8, seq_start int64, seq_len int32)."""
    c = Fp4Cache(_ptr(codes), _ptr(scales), _ptr(seq_start), _ptr(seq_len), int(seq_len.numel()), int(dim),
                 int(max_len), int(ratio))
    c._keep = (codes, scales, seq_start, seq_len)
    return c


def queries(seq, pos, run: int = 1) -> Queries:
    """Queries (device int32 tensors); `run` = queries per run of one sequence (a schedule hint)."""
    q = Queries(_ptr(seq), _ptr(pos), int(seq.numel()), int(run))
    q._keep = (seq, pos)
    return q


def swa(codes, scale, start, count, dim: int, window: int) -> Swa:
    w = Swa(_ptr(codes), _ptr(scale), _ptr(start), _ptr(count), int(dim), int(window))
    w._keep = (codes, scale, start, count)
    return w


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def csa2_abi_version() -> int:
    return lib().csa2_abi_version()


def csa2_quantize_fp4(x, codes, scales, dst_row=None, w_ik=None, ik_codes=None, ik_scales=None, stream=None):
    rows, dim = int(x.shape[0]), int(x.shape[1])
    idx_dim = int(w_ik.shape[1]) if w_ik is not None else 0
    _check(lib().csa2_quantize_fp4(_ptr(x), _dtype_code(x), rows, dim, _ptr(dst_row), _ptr(codes), _ptr(scales),
                                   _ptr(w_ik), idx_dim, _ptr(ik_codes), _ptr(ik_scales), _stream(stream)),
           "csa2_quantize_fp4")


def csa2_compress_fp4(tokens, ratio, w_c, codes, scales, dst_row=None, w_ik=None, ik_codes=None, ik_scales=None,
                      stream=None):
    """tokens: bf16 bits (int16/uint16 tensor) [entries * ratio, d_in]; w_c: bf16 bits [dim, ratio * d_in]."""
    n_tok, d_in = int(tokens.shape[0]), int(tokens.shape[1])
    if ratio < 1 or n_tok % ratio:
        raise ValueError("token rows must be a whole number of entries")
    dim = int(w_c.shape[0])
    idx_dim = int(w_ik.shape[1]) if w_ik is not None else 0
    _check(lib().csa2_compress_fp4(_ptr(tokens), n_tok // ratio, int(ratio), d_in, _ptr(w_c), dim, _ptr(dst_row),
                                   _ptr(codes), _ptr(scales), _ptr(w_ik), idx_dim, _ptr(ik_codes), _ptr(ik_scales),
                                   _stream(stream)), "csa2_compress_fp4")


def csa2_quantize_fp8_rows(x, codes, scale, dst_row=None, stream=None):
    rows, dim = int(x.shape[0]), int(x.shape[1])
    _check(lib().csa2_quantize_fp8_rows(_ptr(x), _dtype_code(x), rows, dim, _ptr(dst_row), _ptr(codes),
                                        _ptr(scale), _stream(stream)), "csa2_quantize_fp8_rows")


def csa2_dequant_fp4(codes, scales, out, stream=None):
    rows, dim = int(out.shape[0]), int(out.shape[1])
    _check(lib().csa2_dequant_fp4(_ptr(codes), _ptr(scales), rows, dim, _ptr(out), _stream(stream)),
           "csa2_dequant_fp4")


def csa2_index_workspace_size(cache: Fp4Cache, m: int, pool_blocks: int, top_k: int) -> int:
    n = c_size_t(0)
    _check(lib().csa2_index_workspace_size(ctypes.byref(cache), int(m), int(pool_blocks), int(top_k),
                                           ctypes.byref(n)), "csa2_index_workspace_size")
    return int(n.value)


def csa2_index_full(cache: Fp4Cache, qs: Queries, q_idx, w_idx, pool_blocks: int, top_k: int, pool_out,
                    pool_count, topk_out, topk_score, workspace, stream=None):
    heads = int(q_idx.shape[1])
    _check(lib().csa2_index_full(ctypes.byref(cache), ctypes.byref(qs), _ptr(q_idx), _ptr(w_idx), heads,
                                 int(pool_blocks), int(top_k), _ptr(pool_out), _ptr(pool_count), _ptr(topk_out),
                                 _ptr(topk_score), _ptr(workspace), int(workspace.numel()) if workspace is not None
                                 else 0, _stream(stream)), "csa2_index_full")


def csa2_reindex(cache: Fp4Cache, qs: Queries, q_idx, w_idx, pool_in, pool_count, top_k: int, topk_out,
                 topk_score, workspace, stream=None):
    heads = int(q_idx.shape[1])
    pool_blocks = int(pool_in.shape[1])
    _check(lib().csa2_reindex(ctypes.byref(cache), ctypes.byref(qs), _ptr(q_idx), _ptr(w_idx), heads,
                              _ptr(pool_in), _ptr(pool_count), pool_blocks, int(top_k), _ptr(topk_out),
                              _ptr(topk_score), _ptr(workspace), int(workspace.numel()) if workspace is not None
                              else 0, _stream(stream)), "csa2_reindex")


def csa2_attn_workspace_size(m: int, heads: int, dim: int, top_k: int, window: int) -> int:
    n = c_size_t(0)
    _check(lib().csa2_attn_workspace_size(int(m), int(heads), int(dim), int(top_k), int(window), ctypes.byref(n)),
           "csa2_attn_workspace_size")
    return int(n.value)


def csa2_sparse_swa_attn(kv: Fp4Cache, qs: Queries, q, topk, top_k: int, window: Swa, softmax_scale: float, out,
                         lse=None, workspace=None, stream=None):
    heads = int(q.shape[1])
    _check(lib().csa2_sparse_swa_attn(ctypes.byref(kv), ctypes.byref(qs), _ptr(q), _dtype_code(q), heads,
                                      _ptr(topk), int(top_k), ctypes.byref(window), float(softmax_scale), _ptr(out),
                                      _ptr(lse), _ptr(workspace),
                                      int(workspace.numel()) if workspace is not None else 0, _stream(stream)),
           "csa2_sparse_swa_attn")


class Group:
    """Keeps a GroupDesc and the host arrays it points to alive."""

    def __init__(self, first_mode, kv: Fp4Cache, idx: Fp4Cache, qs: Queries, q_idx, w_idx, pool_blocks, top_k,
                 pool, pool_count, topk, topk_score, q_list, q_dtype, heads, swa_list, out_list, lse_list,
                 softmax_scale, new_kv=None, new_dst_row=None, w_ik=None):
        n = len(q_list)
        # keep every tensor and descriptor the raw addresses below refer to
        self._keep = (kv, idx, qs, q_idx, w_idx, pool, pool_count, topk, topk_score, list(q_list), list(swa_list),
                      list(out_list), list(lse_list) if lse_list is not None else None, new_kv, new_dst_row, w_ik)
        self._q = (c_void_p * n)(*[_ptr(t) for t in q_list])
        self._swa = (Swa * n)(*swa_list)
        self._out = (c_void_p * n)(*[_ptr(t) for t in out_list])
        self._lse = (c_void_p * n)(*[_ptr(t) for t in lse_list]) if lse_list is not None else None
        d = GroupDesc()
        d.first_mode = first_mode
        d.n_layers = n
        if new_kv is not None:
            d.new_kv = _ptr(new_kv)
            d.new_kv_dtype = _dtype_code(new_kv)
            d.new_rows = int(new_kv.shape[0])
            d.new_dst_row = _ptr(new_dst_row)
            d.w_ik = _ptr(w_ik)
        d.kv, d.idx, d.qs = kv, idx, qs
        d.q_idx, d.w_idx = _ptr(q_idx), _ptr(w_idx)
        d.idx_heads = int(q_idx.shape[1])
        d.pool_blocks, d.top_k = int(pool_blocks), int(top_k)
        d.pool, d.pool_count = _ptr(pool), _ptr(pool_count)
        d.topk, d.topk_score = _ptr(topk), _ptr(topk_score)
        d.q = ctypes.cast(self._q, POINTER(c_void_p))
        d.q_dtype = q_dtype
        d.heads = int(heads)
        d.swa = ctypes.cast(self._swa, POINTER(Swa))
        d.out = ctypes.cast(self._out, POINTER(c_void_p))
        d.lse = ctypes.cast(self._lse, POINTER(c_void_p)) if self._lse is not None else None
        d.softmax_scale = float(softmax_scale)
        self.desc = d


def csa2_group_workspace_size(group: Group) -> int:
    n = c_size_t(0)
    _check(lib().csa2_group_workspace_size(ctypes.byref(group.desc), ctypes.byref(n)), "csa2_group_workspace_size")
    return int(n.value)


def csa2_group_step(group: Group, workspace, stream=None):
    _check(lib().csa2_group_step(ctypes.byref(group.desc), _ptr(workspace),
                                 int(workspace.numel()) if workspace is not None else 0, _stream(stream)),
           "csa2_group_step")


def _desc_array(groups):
    return (GroupDesc * len(groups))(*[g.desc for g in groups])


def csa2_group_steps_workspace_size(groups) -> int:
    n = c_size_t(0)
    _check(lib().csa2_group_steps_workspace_size(_desc_array(groups), len(groups), ctypes.byref(n)),
           "csa2_group_steps_workspace_size")
    return int(n.value)


def csa2_group_steps(groups, workspace, stream=None):
    """Several group steps in one call: every group's write and index, then
    the attention of all their layers batched across groups."""
    _check(lib().csa2_group_steps(_desc_array(groups), len(groups), _ptr(workspace),
                                  int(workspace.numel()) if workspace is not None else 0, _stream(stream)),
           "csa2_group_steps")


def csa2_group_step_static(group: Group, stream=None):
    """csa2_group_step on the library's own scratch array (no workspace argument)."""
    _check(lib().csa2_group_step_static(ctypes.byref(group.desc), _stream(stream)), "csa2_group_step_static")


def csa2_profile_scan(enable: bool) -> None:
    _check(lib().csa2_profile_scan(1 if enable else 0), "csa2_profile_scan")


def csa2_profile_scan_read() -> tuple[float, int]:
    """(summed first-scan kernel milliseconds, launches) since profiling was enabled."""
    ms, n = ctypes.c_double(0.0), c_int64(0)
    _check(lib().csa2_profile_scan_read(ctypes.byref(ms), ctypes.byref(n)), "csa2_profile_scan_read")
    return float(ms.value), int(n.value)


def csa2_profile_attn(enable: bool) -> None:
    _check(lib().csa2_profile_attn(1 if enable else 0), "csa2_profile_attn")


def csa2_profile_attn_read() -> tuple[float, int]:
    """(summed attention kernel milliseconds, launches) since attention timing was enabled."""
    ms, n = ctypes.c_double(0.0), c_int64(0)
    _check(lib().csa2_profile_attn_read(ctypes.byref(ms), ctypes.byref(n)), "csa2_profile_attn_read")
    return float(ms.value), int(n.value)


def csa2_profile_write(enable: bool) -> None:
    _check(lib().csa2_profile_write(1 if enable else 0), "csa2_profile_write")


def csa2_profile_write_read() -> tuple[float, int]:
    """(summed quantise-on-write kernel milliseconds, launches) since write timing was enabled."""
    ms, n = ctypes.c_double(0.0), c_int64(0)
    _check(lib().csa2_profile_write_read(ctypes.byref(ms), ctypes.byref(n)), "csa2_profile_write_read")
    return float(ms.value), int(n.value)


def csa2_profile_compress(enable: bool) -> None:
    _check(lib().csa2_profile_compress(1 if enable else 0), "csa2_profile_compress")


def csa2_profile_compress_read() -> tuple[float, int]:
    """(summed compressor kernel milliseconds, launches) since compressor timing was enabled."""
    ms, n = ctypes.c_double(0.0), c_int64(0)
    _check(lib().csa2_profile_compress_read(ctypes.byref(ms), ctypes.byref(n)), "csa2_profile_compress_read")
    return float(ms.value), int(n.value)
