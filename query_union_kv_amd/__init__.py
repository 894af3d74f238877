"""Python binding of libpw.so: query-union sparse-attention prefill on MI355X.

The functions below carry the C-ABI entry points' names and only marshal
arguments: they check tensor devices, dtypes, shapes and contiguity, pass raw
device pointers and the current HIP stream, and raise ``PWError`` on a non-OK
status.  Every step of the path runs in the library's HIP kernels; PyTorch
provides device memory and streams.  There is no fallback: if the library is
missing or no GPU is present the calls fail.

``SparsePrefill`` chains the four calls for one workload shape and owns the
intermediate buffers (bitsets, groups, union tables).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "PWError", "lib", "pw_version", "pw_words", "pw_num_groups", "pw_union_capacity",
    "pw_append_kv", "pw_page_bitsets", "pw_group", "pw_union_tables", "pw_prepare", "pw_sparse_prefill",
    "pw_schedule_items",
    "SparsePrefill",
    "PW_KV_BF16", "PW_KV_FP8_E4M3", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpw.so")
# the same library built with -DPW_DEBUG: device-side invariant counters (pw_debug_violations)
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpw_debug.so")
PW_KV_BF16 = 0
PW_KV_FP8_E4M3 = 1
_STATUS = {0: "PW_OK", -1: "PW_ERR_ARG", -2: "PW_ERR_UNSUPPORTED", -3: "PW_ERR_CAPACITY",
           -4: "PW_ERR_HIP"}


class PWError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libpw.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        sig = {
            "pw_version": (ctypes.c_char_p, []),
            "pw_debug_violations": (I64, []),
            "pw_last_error": (ctypes.c_char_p, []),
            "pw_words": (I, [I]),
            "pw_num_groups": (I, [I, I, I]),
            "pw_union_capacity": (I64, [I, I, I, I]),
            "pw_append_kv": (I, [P, P, I, I, I, I64, I, P, P, I, P, P, I, I, I64, I64, P]),
            "pw_page_bitsets": (I, [P, I, I, I, I, P, P, P]),
            "pw_group": (I, [P, I, I, I, I, I, P, P, P]),
            "pw_union_tables": (I, [P, I, I, I, P, P, I, I, I, P, P, P, I64, P]),
            "pw_arrange_groups": (I, [P, I, I, I, I, I, I, P, P, P, P, I64, P]),
            "pw_prepare": (I, [P, I, I, I, I, I, I, P, P, P, P, P, P, P, I64, P, P]),
            "pw_prepare_halves": (I, [P, I, I, I, I, I, I, P, P, P, P, P, P, P, I64, P, P]),
            "pw_sparse_prefill": (I, [P, I, I, I, I, P, P, I, P, P, I, I, I64, I64, P, I, F,
                                      P, P, I, I, I, P, P, P, I64, P, P, P, P]),
            "pw_schedule_items": (I, [P, I, P, P]),
            "pw_shared_table_prefill": (I, [P, I, I, I, I, P, P, I, P, P, I, I, I64, I64, P, I, F,
                                            I, P, P, I64, I, P, P, P, P, P]),
            "pw_shared_table_prefill_noalloc": (I, [P, I, I, I, I, P, P, I, P, P, I, I, I64, I64, P, I,
                                                    F, I, P, P, I64, I, P, P, P]),
            "pw_noalloc_scratch_bytes": (ctypes.c_size_t, []),
            "pw_page_items_capacity": (I64, [I, I, I, I, I]),
            "pw_page_workspace_bytes": (ctypes.c_size_t, [I, I, I]),
            "pw_page_tables": (I, [P, I, I, I, I, I, P, ctypes.c_size_t, P, P, P, P, P, P, I64, P]),
            "pw_page_union_prefill": (I, [P, I, I, I, I, P, P, I, P, P, I, I, I64, I64, P, I, F,
                                          P, I, I, P, P, P, P, P, P, I64, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise PWError(status, lib().pw_last_error().decode())


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def pw_version() -> str:
    return lib().pw_version().decode()


def pw_debug_violations() -> int:
    """Invariant violations counted by a debug build since the last call (then cleared);
    -2 from a release build."""
    return lib().pw_debug_violations()


def use_library(path: str) -> None:
    """Makes the binding call the library at `path` from now on (e.g. DEBUG_LIB_PATH)."""
    global _lib, LIB_PATH
    LIB_PATH = path
    _lib = None
    lib()


def pw_words(n_pages: int) -> int:
    return lib().pw_words(n_pages)


def pw_num_groups(nq: int, window: int, max_group: int) -> int:
    return lib().pw_num_groups(nq, window, max_group)


def pw_union_capacity(n_tables: int, group_width: int, k_max: int, n_pages: int) -> int:
    return lib().pw_union_capacity(n_tables, group_width, k_max, n_pages)


def _token_rows(t: torch.Tensor, name: str):
    """A bf16 [n_tok, hkv, d] view whose tokens may be strided (e.g. a slice of a fused
    QKV output): returns (pointer, stride between tokens in elements)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.bfloat16 or t.dim() != 3:
        raise ValueError(f"{name} must be bf16 [n_tok, hkv, d]")
    if t.numel() == 0:
        return t.data_ptr(), t.shape[1] * t.shape[2]
    if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name}: heads and elements of a token must be contiguous")
    return t.data_ptr(), (t.stride(0) if t.shape[0] > 1 else t.shape[1] * t.shape[2])


def pw_append_kv(k_new: torch.Tensor, v_new: torch.Tensor, first_token: int,
                 k_cache: torch.Tensor, v_cache: torch.Tensor,
                 k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                 stream=None) -> None:
    """Writes a chunk's bf16 keys/values [n_tok, hkv, d] at positions first_token.. into
    the paged caches [hkv, n_pages, page_size, d] (bf16, or uint8 e4m3fn codes with fp32
    scales [hkv, n_pages], which are updated)."""
    n_tok, hkv, d = k_new.shape
    if tuple(v_new.shape) != (n_tok, hkv, d):
        raise ValueError("k_new and v_new shapes differ")
    kp, ks_tok = _token_rows(k_new, "k_new")
    vp, vs_tok = _token_rows(v_new, "v_new")
    if ks_tok != vs_tok:
        raise ValueError("k_new and v_new must share one token stride")
    if k_cache.dim() != 4 or tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.shape[0] != hkv \
            or k_cache.shape[3] != d:
        raise ValueError("caches must be [hkv, n_pages, page_size, d]")
    fp8 = k_cache.dtype == torch.uint8
    dt = torch.uint8 if fp8 else torch.bfloat16
    _, n_pages, ps, _ = k_cache.shape
    if fp8 and (k_scale is None or v_scale is None or tuple(k_scale.shape) != (hkv, n_pages)
                or tuple(v_scale.shape) != (hkv, n_pages)):
        raise ValueError("fp8 caches need k_scale and v_scale [hkv, n_pages]")
    _check(lib().pw_append_kv(kp, vp, n_tok, hkv, d, ks_tok, first_token,
                              _ptr(k_cache, dt, "k_cache"), _ptr(v_cache, dt, "v_cache"),
                              PW_KV_FP8_E4M3 if fp8 else PW_KV_BF16,
                              _ptr(k_scale, torch.float32, "k_scale") if fp8 else None,
                              _ptr(v_scale, torch.float32, "v_scale") if fp8 else None,
                              ps, n_pages, n_pages * ps * d, ps * d, _stream(stream)))


def pw_page_bitsets(topk: torch.Tensor, n_pages: int, bits: torch.Tensor,
                    bad_id_count: Optional[torch.Tensor] = None, stream=None) -> None:
    """topk int32 [n_rows, hkv, k] -> bits int64 (uint64 words) [hkv, n_rows, words]."""
    n_rows, hkv, k = topk.shape
    if tuple(bits.shape) != (hkv, n_rows, pw_words(n_pages)):
        raise ValueError(f"bits shape {tuple(bits.shape)} != {(hkv, n_rows, pw_words(n_pages))}")
    _check(lib().pw_page_bitsets(_ptr(topk, torch.int32, "topk"), n_rows, hkv, k, n_pages,
                                 _ptr(bits, torch.int64, "bits"),
                                 _ptr(bad_id_count, torch.int32, "bad_id_count"), _stream(stream)))


def pw_group(bits: torch.Tensor, n_pages: int, window: int, max_group: int,
             group_qids: torch.Tensor, group_size: torch.Tensor, stream=None) -> None:
    """bits [hkv, nq, words] -> group_qids int32 [hkv, G, max_group], group_size int32 [hkv, G]."""
    hkv, nq, _ = bits.shape
    n_groups = pw_num_groups(nq, window, max_group)
    if tuple(group_qids.shape) != (hkv, n_groups, max_group) or tuple(group_size.shape) != (hkv, n_groups):
        raise ValueError("group_qids/group_size shapes do not match pw_num_groups")
    _check(lib().pw_group(_ptr(bits, torch.int64, "bits"), nq, hkv, n_pages, window, max_group,
                          _ptr(group_qids, torch.int32, "group_qids"),
                          _ptr(group_size, torch.int32, "group_size"), _stream(stream)))


def pw_arrange_groups(bits: torch.Tensor, n_pages: int, hq: int, group_qids: torch.Tensor,
                      group_size: torch.Tensor, union_off: torch.Tensor,
                      union_qmask: Optional[torch.Tensor] = None, stream=None) -> None:
    """Reorders each group's members for 4-member row tiles (hq/hkv = 4, groups of 5..8) and
    permutes its member-mask bits to match; a no-op for other shapes."""
    hkv, nq, _ = bits.shape
    _, n_groups, max_group = group_qids.shape
    _check(lib().pw_arrange_groups(_ptr(bits, torch.int64, "bits"), nq, hkv, n_pages, hq, n_groups,
                                   max_group, _ptr(group_qids, torch.int32, "group_qids"),
                                   _ptr(group_size, torch.int32, "group_size"),
                                   _ptr(union_off, torch.int32, "union_off"),
                                   _ptr(union_qmask, torch.uint8, "union_qmask"),
                                   union_qmask.numel() if union_qmask is not None else 0, _stream(stream)))


def pw_union_tables(bits: torch.Tensor, n_pages: int, group_rows: Optional[torch.Tensor],
                    group_size: Optional[torch.Tensor], k_max: int, union_off: torch.Tensor,
                    union_pages: torch.Tensor, union_qmask: Optional[torch.Tensor] = None,
                    stream=None, *, n_groups: Optional[int] = None, width: Optional[int] = None) -> None:
    """bits [hkv, n_rows, words], group_rows int32 [hkv, n_groups, width] -> CSR union tables.
    group_rows None: consecutive groups of ``width`` rows (``n_groups`` of them per KV head)."""
    hkv, n_rows, _ = bits.shape
    if group_rows is not None:
        _, n_groups, width = group_rows.shape
    elif n_groups is None or width is None:
        raise ValueError("consecutive groups (group_rows=None) need n_groups and width")
    if union_off.numel() != hkv * n_groups + 1:
        raise ValueError("union_off must have hkv*n_groups+1 entries")
    if union_qmask is not None and union_qmask.numel() < union_pages.numel():
        raise ValueError("union_qmask smaller than union_pages")
    _check(lib().pw_union_tables(_ptr(bits, torch.int64, "bits"), n_rows, hkv, n_pages,
                                 _ptr(group_rows, torch.int32, "group_rows"),
                                 _ptr(group_size, torch.int32, "group_size"), n_groups, width, k_max,
                                 _ptr(union_off, torch.int32, "union_off"),
                                 _ptr(union_pages, torch.int32, "union_pages"),
                                 _ptr(union_qmask, torch.uint8, "union_qmask"),
                                 union_pages.numel(), _stream(stream)))


def pw_prepare(topk: torch.Tensor, n_pages: int, window: int, max_group: int,
               bits: torch.Tensor, group_qids: torch.Tensor, group_size: torch.Tensor,
               union_off: torch.Tensor, union_pages: torch.Tensor, union_qmask: torch.Tensor,
               bad_id_count: Optional[torch.Tensor] = None, stream=None,
               item_order: Optional[torch.Tensor] = None, halves: bool = False) -> None:
    """Fused pw_page_bitsets + pw_group + pw_union_tables (same outputs); with item_order,
    also the work order of pw_schedule_items.  halves=True calls pw_prepare_halves: the
    tables are those of each group's two halves (2 * hkv * n_groups tables)."""
    nq, hkv, k = topk.shape
    n_groups = pw_num_groups(nq, window, max_group)
    n_tables = hkv * n_groups * (2 if halves else 1)
    if item_order is not None and item_order.numel() != n_tables:
        raise ValueError("item_order must hold one entry per union table")
    if tuple(bits.shape) != (hkv, nq, pw_words(n_pages)):
        raise ValueError("bits shape")
    if tuple(group_qids.shape) != (hkv, n_groups, max_group) or tuple(group_size.shape) != (hkv, n_groups):
        raise ValueError("group_qids/group_size shapes do not match pw_num_groups")
    if union_off.numel() != n_tables + 1 or union_qmask.numel() < union_pages.numel():
        raise ValueError("union table buffer sizes")
    fn = lib().pw_prepare_halves if halves else lib().pw_prepare
    _check(fn(_ptr(topk, torch.int32, "topk"), nq, hkv, k, n_pages, window, max_group,
                            _ptr(bits, torch.int64, "bits"),
                            _ptr(bad_id_count, torch.int32, "bad_id_count"),
                            _ptr(group_qids, torch.int32, "group_qids"),
                            _ptr(group_size, torch.int32, "group_size"),
                            _ptr(union_off, torch.int32, "union_off"),
                            _ptr(union_pages, torch.int32, "union_pages"),
                            _ptr(union_qmask, torch.uint8, "union_qmask"),
                            union_pages.numel(), _ptr(item_order, torch.int32, "item_order"),
                            _stream(stream)))


def pw_sparse_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      q_pos: torch.Tensor, kv_len: int, union_off: torch.Tensor,
                      union_pages: torch.Tensor, out: torch.Tensor, *,
                      hkv: int, n_groups: int, max_group: int,
                      group_qids: Optional[torch.Tensor] = None,
                      group_size: Optional[torch.Tensor] = None,
                      union_qmask: Optional[torch.Tensor] = None,
                      k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                      shared_table: bool = False, sm_scale: Optional[float] = None,
                      lse: Optional[torch.Tensor] = None, item_order: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """q bf16 [nq, hq, d]; k_cache/v_cache [hkv, n_pages, page_size, d] (bf16 or uint8 fp8 codes);
    item_order: int32 [hkv * n_groups] work order from pw_schedule_items, or None."""
    nq, hq, d = q.shape
    if k_cache.shape != v_cache.shape or k_cache.dim() != 4 or k_cache.shape[0] != hkv:
        raise ValueError("k_cache/v_cache must be [hkv, n_pages, page_size, d]")
    _, n_pages, page_size, dk = k_cache.shape
    if dk != d:
        raise ValueError("head dim mismatch")
    if k_cache.dtype == torch.bfloat16:
        kv_dtype = PW_KV_BF16
    elif k_cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        kv_dtype = PW_KV_FP8_E4M3
    else:
        raise ValueError(f"unsupported cache dtype {k_cache.dtype}")
    if out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must be bf16 shaped like q")
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    _check(lib().pw_sparse_prefill(
        _ptr(q, torch.bfloat16, "q"), nq, hq, hkv, d, _ptr(k_cache, name="k_cache"),
        _ptr(v_cache, name="v_cache"), kv_dtype, _ptr(k_scale, torch.float32, "k_scale"),
        _ptr(v_scale, torch.float32, "v_scale"), page_size, n_pages, n_pages * page_size * d,
        page_size * d, _ptr(q_pos, torch.int32, "q_pos"), kv_len, sm,
        _ptr(group_qids, torch.int32, "group_qids"), _ptr(group_size, torch.int32, "group_size"),
        n_groups, max_group, 1 if shared_table else 0, _ptr(union_off, torch.int32, "union_off"),
        _ptr(union_pages, torch.int32, "union_pages"), _ptr(union_qmask, torch.uint8, "union_qmask"),
        union_pages.numel(), _ptr(item_order, torch.int32, "item_order"),
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"), _stream(stream)))


def pw_schedule_items(union_off: torch.Tensor, item_order: torch.Tensor, stream=None) -> None:
    """Work order for pw_sparse_prefill: each of the 8 consecutive position ranges lists its
    items by union size, largest first (ties: lower item index)."""
    n = union_off.numel() - 1
    if item_order.numel() != n:
        raise ValueError("item_order must hold one entry per table")
    _check(lib().pw_schedule_items(_ptr(union_off, torch.int32, "union_off"), n,
                                   _ptr(item_order, torch.int32, "item_order"), _stream(stream)))


def _cache_dtype(k_cache: torch.Tensor) -> int:
    if k_cache.dtype == torch.bfloat16:
        return PW_KV_BF16
    if k_cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PW_KV_FP8_E4M3
    raise ValueError(f"unsupported cache dtype {k_cache.dtype}")


def pw_shared_table_prefill(q, k_cache, v_cache, q_pos, kv_len: int, union_off, union_pages, out, *,
                            hkv: int, max_group: int, n_split: int, partial_o=None, partial_lse=None,
                            k_scale=None, v_scale=None, sm_scale: Optional[float] = None, lse=None,
                            stream=None) -> None:
    """Attention of consecutive query groups over one shared table per KV head, each table
    cut into n_split slices whose partial rows are merged by lse."""
    nq, hq, d = q.shape
    _, n_pages, page_size, _ = k_cache.shape
    if n_split > 1 and (partial_o is None or partial_lse is None or partial_o.numel() < nq * hq * n_split * d
                        or partial_lse.numel() < nq * hq * n_split):
        raise ValueError("partial buffers too small for n_split")
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    _check(lib().pw_shared_table_prefill(
        _ptr(q, torch.bfloat16, "q"), nq, hq, hkv, d, _ptr(k_cache, name="k_cache"),
        _ptr(v_cache, name="v_cache"), _cache_dtype(k_cache), _ptr(k_scale, torch.float32, "k_scale"),
        _ptr(v_scale, torch.float32, "v_scale"), page_size, n_pages, n_pages * page_size * d,
        page_size * d, _ptr(q_pos, torch.int32, "q_pos"), kv_len, sm, max_group,
        _ptr(union_off, torch.int32, "union_off"), _ptr(union_pages, torch.int32, "union_pages"),
        union_pages.numel(), n_split, _ptr(partial_o, torch.bfloat16, "partial_o"),
        _ptr(partial_lse, torch.float32, "partial_lse"), _ptr(out, torch.bfloat16, "out"),
        _ptr(lse, torch.float32, "lse"), _stream(stream)))


def pw_shared_table_prefill_noalloc(q, k_cache, v_cache, q_pos, kv_len: int, union_off, union_pages,
                                    out, *, hkv: int, max_group: int, n_split: int, k_scale=None,
                                    v_scale=None, sm_scale: Optional[float] = None, lse=None,
                                    stream=None) -> None:
    """pw_shared_table_prefill with the slice partials in the library's own device array
    (pw_noalloc_scratch_bytes() per device): no device memory is allocated for the call.
    Calls that overlap in time on one GPU share that array and race."""
    nq, hq, d = q.shape
    _, n_pages, page_size, _ = k_cache.shape
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    _check(lib().pw_shared_table_prefill_noalloc(
        _ptr(q, torch.bfloat16, "q"), nq, hq, hkv, d, _ptr(k_cache, name="k_cache"),
        _ptr(v_cache, name="v_cache"), _cache_dtype(k_cache), _ptr(k_scale, torch.float32, "k_scale"),
        _ptr(v_scale, torch.float32, "v_scale"), page_size, n_pages, n_pages * page_size * d,
        page_size * d, _ptr(q_pos, torch.int32, "q_pos"), kv_len, sm, max_group,
        _ptr(union_off, torch.int32, "union_off"), _ptr(union_pages, torch.int32, "union_pages"),
        union_pages.numel(), n_split, _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"),
        _stream(stream)))


def pw_noalloc_scratch_bytes() -> int:
    return lib().pw_noalloc_scratch_bytes()


def pw_page_items_capacity(nq: int, hkv: int, k_max: int, n_pages: int, chunk: int) -> int:
    return lib().pw_page_items_capacity(nq, hkv, k_max, n_pages, chunk)


def pw_page_workspace_bytes(nq: int, hkv: int, n_pages: int) -> int:
    return lib().pw_page_workspace_bytes(nq, hkv, n_pages)


def pw_page_tables(bits: torch.Tensor, n_pages: int, k_max: int, chunk: int, workspace: torch.Tensor,
                   item_off: torch.Tensor, item_kvh: torch.Tensor, item_page: torch.Tensor,
                   item_qids: torch.Tensor, item_size: torch.Tensor, item_slot: torch.Tensor,
                   stream=None) -> None:
    """Page-major work items of the direct KV-page union from bits [hkv, nq, words]."""
    hkv, nq, _ = bits.shape
    cap = item_kvh.numel()
    if item_off.numel() != hkv * n_pages + 1:
        raise ValueError("item_off size")
    if item_page.numel() != cap or item_size.numel() != cap or item_qids.numel() != cap * chunk \
            or item_slot.numel() != cap * chunk:
        raise ValueError("item array sizes")
    _check(lib().pw_page_tables(_ptr(bits, torch.int64, "bits"), nq, hkv, n_pages, k_max, chunk,
                                _ptr(workspace, name="workspace"),
                                workspace.numel() * workspace.element_size(),
                                _ptr(item_off, torch.int32, "item_off"),
                                _ptr(item_kvh, torch.int32, "item_kvh"),
                                _ptr(item_page, torch.int32, "item_page"),
                                _ptr(item_qids, torch.int32, "item_qids"),
                                _ptr(item_size, torch.int32, "item_size"),
                                _ptr(item_slot, torch.int32, "item_slot"), cap, _stream(stream)))


def pw_page_union_prefill(q, k_cache, v_cache, q_pos, kv_len: int, bits, k_max: int, chunk: int,
                          item_off, item_kvh, item_page, item_qids, item_size, item_slot,
                          partial_o, partial_lse, out, k_scale=None, v_scale=None,
                          sm_scale: Optional[float] = None, lse=None, stream=None) -> None:
    """Attention through page-major items into partials, then their lse merge into out/lse."""
    nq, hq, d = q.shape
    hkv, n_pages, page_size, _ = k_cache.shape
    G = hq // hkv
    if partial_o.numel() < nq * hkv * k_max * G * d or partial_lse.numel() < nq * hkv * k_max * G:
        raise ValueError("partial buffers too small")
    if out.shape != q.shape or out.dtype != torch.bfloat16:
        raise ValueError("out must be bf16 shaped like q")
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    _check(lib().pw_page_union_prefill(
        _ptr(q, torch.bfloat16, "q"), nq, hq, hkv, d, _ptr(k_cache, name="k_cache"),
        _ptr(v_cache, name="v_cache"), _cache_dtype(k_cache), _ptr(k_scale, torch.float32, "k_scale"),
        _ptr(v_scale, torch.float32, "v_scale"), page_size, n_pages, n_pages * page_size * d,
        page_size * d, _ptr(q_pos, torch.int32, "q_pos"), kv_len, sm, _ptr(bits, torch.int64, "bits"),
        k_max, chunk, _ptr(item_off, torch.int32, "item_off"), _ptr(item_kvh, torch.int32, "item_kvh"),
        _ptr(item_page, torch.int32, "item_page"), _ptr(item_qids, torch.int32, "item_qids"),
        _ptr(item_size, torch.int32, "item_size"), _ptr(item_slot, torch.int32, "item_slot"),
        item_kvh.numel(), _ptr(partial_o, torch.bfloat16, "partial_o"),
        _ptr(partial_lse, torch.float32, "partial_lse"), _ptr(out, torch.bfloat16, "out"),
        _ptr(lse, torch.float32, "lse"), _stream(stream)))


@dataclass
class PageUnionPrefill:
    """The direct KV-page union for TopK supports: page bitsets -> page-major work
    items (each (KV head, page) once, its selecting queries in chunks) -> attention
    into per-(query, page) partials -> their lse merge.  Owns the tables and the
    partial workspace (nq * hq * k * d bf16)."""
    nq: int
    hq: int
    hkv: int
    d: int
    n_pages: int
    page_size: int
    kv_len: int
    k: int                      # TopK width: bounds every support size
    chunk: int = 0              # queries per work item (0: 64 query-head rows per item)
    device: str = "cuda"

    def __post_init__(self):
        dev = self.device
        i32 = dict(dtype=torch.int32, device=dev)
        G = self.hq // self.hkv
        if self.chunk <= 0:
            self.chunk = max(1, min(64, 64 // G))
        self.bits = torch.empty((self.hkv, self.nq, pw_words(self.n_pages)), dtype=torch.int64, device=dev)
        self.bad_ids = torch.zeros(1, **i32)
        ws = pw_page_workspace_bytes(self.nq, self.hkv, self.n_pages)
        self.workspace = torch.empty(max(-(-ws // 8), 1), dtype=torch.int64, device=dev)
        cap = max(pw_page_items_capacity(self.nq, self.hkv, self.k, self.n_pages, self.chunk), 1)
        self.item_off = torch.empty(self.hkv * self.n_pages + 1, **i32)
        self.item_kvh = torch.empty(cap, **i32)
        self.item_page = torch.empty(cap, **i32)
        self.item_size = torch.empty(cap, **i32)
        self.item_qids = torch.empty((cap, self.chunk), **i32)
        self.item_slot = torch.empty((cap, self.chunk), **i32)
        rows = max(self.nq * self.hkv * self.k * G, 1)
        self.partial_o = torch.empty((rows, self.d), dtype=torch.bfloat16, device=dev)
        self.partial_lse = torch.empty(rows, dtype=torch.float32, device=dev)

    @property
    def n_items(self) -> int:
        return int(self.item_off[-1].item())

    def prepare(self, topk: torch.Tensor, stream=None) -> None:
        pw_page_bitsets(topk, self.n_pages, self.bits, self.bad_ids, stream)
        pw_page_tables(self.bits, self.n_pages, self.k, self.chunk, self.workspace, self.item_off,
                       self.item_kvh, self.item_page, self.item_qids, self.item_size, self.item_slot,
                       stream)

    def attend(self, q, k_cache, v_cache, q_pos, out, k_scale=None, v_scale=None, lse=None,
               sm_scale=None, stream=None) -> None:
        pw_page_union_prefill(q, k_cache, v_cache, q_pos, self.kv_len, self.bits, self.k, self.chunk,
                              self.item_off, self.item_kvh, self.item_page, self.item_qids,
                              self.item_size, self.item_slot, self.partial_o, self.partial_lse, out,
                              k_scale, v_scale, sm_scale, lse, stream)

    def __call__(self, topk, q, k_cache, v_cache, q_pos, out, k_scale=None, v_scale=None, lse=None,
                 stream=None) -> None:
        self.prepare(topk, stream)
        self.attend(q, k_cache, v_cache, q_pos, out, k_scale, v_scale, lse, stream=stream)


@dataclass
class SparsePrefill:
    """The four calls of one complete sparse-prefill call, with their buffers.

    Per-query mode (``topk`` given): page bitsets -> affinity grouping (or
    original-order groups when ``grouping='original'``) -> union tables with
    member masks -> union attention.  With ``halves=True`` the groups are run as
    two halves, each over the union of its own members' pages (a page both halves
    selected is read twice): every row sees the same pages in the same order, so
    the outputs are bit-identical, and wide groups (8 members x 8 query heads)
    avoid the two-wave form, whose waves wait on each other's tiles.  The default
    (``halves=None``) runs groups of more than 32 query-head rows as halves.
    Block-union mode (``mask_rows`` given, CompactAttention's per-KV-group
    block table): bitsets of the mask rows -> one union over every row of a
    KV head -> attention of consecutive query groups over that shared table;
    there ``max_group`` may exceed 8 (up to 256 query-head rows per work item)
    so that each staged tile serves many rows.
    """
    nq: int
    hq: int
    hkv: int
    d: int
    n_pages: int
    page_size: int
    kv_len: int
    k: int                      # ids per row of topk / mask_rows
    window: int = 64
    max_group: int = 8
    mode: str = "topk"          # "topk" or "block_union"
    grouping: str = "affinity"  # "affinity" or "original" (topk mode)
    n_rows: int = 0             # block_union: mask rows per KV head
    fused: bool = True          # topk/affinity mode: one pw_prepare call for the three steps
    arrange: bool = False       # topk mode: members arranged for row tiles (pw_arrange_groups)
    n_split: int = 0            # block_union mode: table slices per KV head (0: enough to
                                # give every SIMD two waves; 1: no partials)
    schedule: bool = True       # topk mode: start the largest unions first (the work order of
                                # pw_schedule_items; listed by pw_prepare when fused)
    halves: Optional[bool] = None   # topk mode: run each group as two halves of max_group / 2
                                # members, each over the union of its own members' pages
                                # (None: when a group has more than 32 query-head rows)
    device: str = "cuda"

    def __post_init__(self):
        dev = self.device
        w = pw_words(self.n_pages)
        i32 = dict(dtype=torch.int32, device=dev)
        if self.halves is None:
            self.halves = (self.mode == "topk" and self.grouping == "affinity" and not self.arrange
                           and self.max_group % 2 == 0 and self.max_group * (self.hq // self.hkv) > 32)
        if self.halves and (self.mode != "topk" or self.max_group % 2):
            raise ValueError("halves needs topk mode and an even max_group")
        if self.halves and self.arrange:
            raise ValueError("halves and arrange are not combined")
        if self.mode == "topk":
            self.n_rows = self.nq
            self.n_groups = pw_num_groups(self.nq, self.window, self.max_group)
            self.width = self.max_group // 2 if self.halves else self.max_group
            n_tables = self.hkv * self.n_groups * (2 if self.halves else 1)
        elif self.mode == "block_union":
            self.n_groups = -(-self.nq // self.max_group)
            self.width = self.n_rows
            n_tables = self.hkv
        else:
            raise ValueError(self.mode)
        self.bits = torch.empty((self.hkv, self.n_rows, w), dtype=torch.int64, device=dev)
        self.bad_ids = torch.zeros(1, **i32)
        cap = pw_union_capacity(n_tables, self.width, self.k, self.n_pages)
        self.union_off = torch.empty(n_tables + 1, **i32)
        self.union_pages = torch.empty(max(cap, 1), **i32)
        if self.mode == "topk":
            self.group_qids = torch.empty((self.hkv, self.n_groups, self.max_group), **i32)
            self.group_size = torch.empty((self.hkv, self.n_groups), **i32)
            self.union_qmask = torch.empty(max(cap, 1), dtype=torch.uint8, device=dev)
            self.item_order = torch.empty(n_tables, **i32) if self.schedule else None
            if self.halves:
                # half h of group j is the row [h * mg/2, (h + 1) * mg/2) of its member list (a
                # view); absent members stay -1, so every half reports mg/2 members
                self.half_qids = self.group_qids.view(self.hkv, 2 * self.n_groups, self.width)
                self.half_size = torch.full((self.hkv, 2 * self.n_groups), self.width, **i32)
            if self.grouping == "original":
                # consecutive groups: the library lists their unions and runs them from
                # their ranks alone (group_rows / group_qids NULL), no member lists
                if self.halves or self.arrange:
                    raise ValueError("original-order groups take neither halves nor arrange")
                if -(-self.nq // self.max_group) != self.n_groups:
                    raise ValueError("original-order groups need window % max_group == 0")
                self.group_qids = self.group_size = None
        else:
            self.group_rows = torch.arange(self.n_rows, **i32).view(1, 1, -1).repeat(self.hkv, 1, 1)
            self.group_qids = self.group_size = self.union_qmask = self.item_order = None
            if self.n_split <= 0:
                G = self.hq // self.hkv
                waves = self.hkv * self.n_groups * max(1, -(-self.max_group * G // 32))
                self.n_split = max(1, min(8, -(-2048 // waves)))
            self.partial_o = self.partial_lse = None
            if self.n_split > 1:
                rows = self.nq * self.hq * self.n_split
                self.partial_o = torch.empty((rows, self.d), dtype=torch.bfloat16, device=dev)
                self.partial_lse = torch.empty(rows, dtype=torch.float32, device=dev)

    def prepare(self, ids: torch.Tensor, stream=None) -> None:
        """Bitsets, grouping and union tables from topk [nq, hkv, k] or mask rows [n_rows, hkv, k]."""
        if self.halves and self.grouping == "affinity" and self.fused:
            # bitsets, groups and the halves' tables (and their work order) in the fused launches
            pw_prepare(ids, self.n_pages, self.window, self.max_group, self.bits, self.group_qids,
                       self.group_size, self.union_off, self.union_pages, self.union_qmask,
                       self.bad_ids, stream, item_order=self.item_order, halves=True)
            return
        if self.halves:
            pw_page_bitsets(ids, self.n_pages, self.bits, self.bad_ids, stream)
            if self.grouping == "affinity":
                pw_group(self.bits, self.n_pages, self.window, self.max_group, self.group_qids,
                         self.group_size, stream)
            pw_union_tables(self.bits, self.n_pages, self.half_qids, None, self.k, self.union_off,
                            self.union_pages, self.union_qmask, stream)
            if self.item_order is not None:
                pw_schedule_items(self.union_off, self.item_order, stream)
            return
        if self.mode == "topk" and self.grouping == "affinity" and self.fused:
            # (the work order comes with the tables; arranging members keeps union sizes)
            pw_prepare(ids, self.n_pages, self.window, self.max_group, self.bits, self.group_qids,
                       self.group_size, self.union_off, self.union_pages, self.union_qmask,
                       self.bad_ids, stream, item_order=self.item_order)
            if self.arrange:
                pw_arrange_groups(self.bits, self.n_pages, self.hq, self.group_qids, self.group_size,
                                  self.union_off, self.union_qmask, stream)
            return
        pw_page_bitsets(ids, self.n_pages, self.bits, self.bad_ids, stream)
        if self.mode == "topk":
            if self.grouping == "affinity":
                pw_group(self.bits, self.n_pages, self.window, self.max_group, self.group_qids,
                         self.group_size, stream)
            pw_union_tables(self.bits, self.n_pages, self.group_qids, self.group_size, self.k,
                            self.union_off, self.union_pages, self.union_qmask, stream,
                            n_groups=self.n_groups, width=self.max_group)
            if self.arrange:
                pw_arrange_groups(self.bits, self.n_pages, self.hq, self.group_qids, self.group_size,
                                  self.union_off, self.union_qmask, stream)
            if self.item_order is not None:
                pw_schedule_items(self.union_off, self.item_order, stream)
        else:
            pw_union_tables(self.bits, self.n_pages, self.group_rows, None, self.k,
                            self.union_off, self.union_pages, None, stream)

    def attend(self, q, k_cache, v_cache, q_pos, out, k_scale=None, v_scale=None, lse=None,
               sm_scale=None, stream=None, kv_len: Optional[int] = None) -> None:
        kv_len = self.kv_len if kv_len is None else kv_len
        if self.mode == "block_union" and self.n_split > 1:
            pw_shared_table_prefill(q, k_cache, v_cache, q_pos, kv_len, self.union_off, self.union_pages,
                                    out, hkv=self.hkv, max_group=self.max_group, n_split=self.n_split,
                                    partial_o=self.partial_o, partial_lse=self.partial_lse,
                                    k_scale=k_scale, v_scale=v_scale, sm_scale=sm_scale, lse=lse,
                                    stream=stream)
            return
        if self.halves:
            pw_sparse_prefill(q, k_cache, v_cache, q_pos, kv_len, self.union_off, self.union_pages,
                              out, hkv=self.hkv, n_groups=2 * self.n_groups, max_group=self.width,
                              group_qids=self.half_qids, group_size=self.half_size,
                              union_qmask=self.union_qmask, k_scale=k_scale, v_scale=v_scale,
                              sm_scale=sm_scale, lse=lse, item_order=self.item_order, stream=stream)
            return
        pw_sparse_prefill(q, k_cache, v_cache, q_pos, kv_len, self.union_off, self.union_pages,
                          out, hkv=self.hkv, n_groups=self.n_groups, max_group=self.max_group,
                          group_qids=self.group_qids, group_size=self.group_size,
                          union_qmask=self.union_qmask, k_scale=k_scale, v_scale=v_scale,
                          shared_table=self.mode == "block_union", sm_scale=sm_scale, lse=lse,
                          item_order=self.item_order, stream=stream)

    def __call__(self, ids, q, k_cache, v_cache, q_pos, out, k_scale=None, v_scale=None, lse=None,
                 stream=None) -> None:
        self.prepare(ids, stream)
        self.attend(q, k_cache, v_cache, q_pos, out, k_scale, v_scale, lse, stream=stream)


class ChunkedPrefill:
    """Chunked sparse prefill of one sequence through the query-union path.

    For chunk c (queries at positions first_c .. first_c + n_c - 1, the cache then
    holding first_c + n_c tokens): append the chunk's keys and values into the paged
    cache, build its bitsets, groups and union tables from its TopK pages, and attend.
    Preparation needs only the chunk's TopK IDs, so with ``overlap=True`` chunk c+1's
    preparation runs on a second stream while chunk c attends (PageWeaver Fig. 6: the
    online cost decides the net gain; QUILT hides preparation by pipelining it).  The
    tables are double-buffered: preparing chunk c+2 waits until chunk c's attention is
    done with its buffers.  Appends stay on the main stream after the previous chunk's
    attention, since a chunk may share its first page with the previous one.
    Both streams have the default priority.
    """

    def __init__(self, hq: int, hkv: int, d: int, n_pages: int, page_size: int, max_chunk: int,
                 k: int, window: int = 64, max_group: int = 8, device="cuda"):
        self.page_size = page_size
        self.plans = [SparsePrefill(nq=max_chunk, hq=hq, hkv=hkv, d=d, n_pages=n_pages,
                                    page_size=page_size, kv_len=n_pages * page_size, k=k,
                                    window=window, max_group=max_group, device=device)
                      for _ in range(2)]
        self.max_chunk = max_chunk
        self.side = torch.cuda.Stream(device=device)

    def _plan_for(self, i: int, n: int) -> "SparsePrefill":
        p = self.plans[i % 2]
        if n == p.nq:
            return p
        # a shorter (last) chunk: a plan of its own size on the same buffers' device
        return SparsePrefill(nq=n, hq=p.hq, hkv=p.hkv, d=p.d, n_pages=p.n_pages, page_size=p.page_size,
                             kv_len=p.kv_len, k=p.k, window=p.window, max_group=p.max_group,
                             device=p.device)

    def run(self, chunks, k_cache, v_cache, k_scale=None, v_scale=None, overlap: bool = True,
            stream=None) -> None:
        """chunks: sequence of dicts with q [n, hq, d] bf16, k_new / v_new [n, hkv, d] bf16,
        topk [n, hkv, k] int32, q_pos [n] int32, out [n, hq, d] bf16, optional lse
        [n, hq] fp32, and first_token (the chunk's first position)."""
        main = torch.cuda.current_stream() if stream is None else stream
        side = self.side if overlap else main
        plans = [self._plan_for(i, c["q"].shape[0]) for i, c in enumerate(chunks)]
        prepared = [torch.cuda.Event() for _ in chunks]
        attended = [torch.cuda.Event() for _ in chunks]

        def prepare(i):
            if overlap:
                if i == 0:
                    side.wait_stream(main)              # inputs written earlier on the main stream
                elif i >= 2:
                    side.wait_event(attended[i - 2])   # chunk i-2 is done with these buffers
            plans[i].prepare(chunks[i]["topk"], side)
            prepared[i].record(side)

        if chunks:
            prepare(0)
        for i, c in enumerate(chunks):
            n = c["q"].shape[0]
            pw_append_kv(c["k_new"], c["v_new"], c["first_token"], k_cache, v_cache, k_scale, v_scale,
                         stream=main)
            if i + 1 < len(chunks) and overlap:
                prepare(i + 1)
            main.wait_event(prepared[i])
            plans[i].attend(c["q"], k_cache, v_cache, c["q_pos"], c["out"], k_scale, v_scale,
                            c.get("lse"), stream=main, kv_len=c["first_token"] + n)
            attended[i].record(main)
            if i + 1 < len(chunks) and not overlap:
                prepare(i + 1)
        if overlap:
            main.wait_stream(side)   # later work (and buffer reuse) follows every preparation


def sparse_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, topk: torch.Tensor,
                   q_pos: torch.Tensor, *, kv_len: int, k_scale: Optional[torch.Tensor] = None,
                   v_scale: Optional[torch.Tensor] = None, window: int = 64, max_group: int = 8,
                   sm_scale: Optional[float] = None, with_lse: bool = False,
                   halves: Optional[bool] = None,
                   stream=None):
    """One complete query-union call on the current stream: bitsets, affinity grouping and
    union tables from topk [nq, hkv, K], then attention.  q bf16 [nq, hq, d]; caches
    [hkv, n_pages, page_size, d] (bf16, or uint8 e4m3fn codes with fp32 scales
    [hkv, n_pages]).  ``halves`` runs every group as two halves over their own unions
    (the same outputs; see SparsePrefill; None: for groups of more than 32 rows).  Returns (out, aux): out bf16 [nq, hq, d]; aux
    holds the plan with its bitsets, groups and union tables, and lse [nq, hq] when
    with_lse."""
    nq, hq, d = q.shape
    hkv, n_pages, page_size, _ = k_cache.shape
    plan = SparsePrefill(nq=nq, hq=hq, hkv=hkv, d=d, n_pages=n_pages, page_size=page_size, kv_len=kv_len,
                         k=topk.shape[2], window=window, max_group=max_group, halves=halves,
                         device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty((nq, hq), dtype=torch.float32, device=q.device) if with_lse else None
    plan.prepare(topk, stream)
    plan.attend(q, k_cache, v_cache, q_pos, out, k_scale, v_scale, lse, sm_scale, stream)
    aux = {"plan": plan, "bits": plan.bits, "group_qids": plan.group_qids, "group_size": plan.group_size,
           "union_off": plan.union_off, "union_pages": plan.union_pages, "union_qmask": plan.union_qmask,
           "bad_ids": plan.bad_ids}
    if with_lse:
        aux["lse"] = lse
    return out, aux
