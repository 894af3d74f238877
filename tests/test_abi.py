"""The C-ABI library: it loads, exports every entry point include/pw.h declares, and
rejects bad arguments on the host before any device work (no GPU needed)."""
import ctypes
import os
import re

import pytest
import torch

import query_union_kv_amd as pw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pw.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pw_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"pw_page_bitsets", "pw_group", "pw_union_tables", "pw_sparse_prefill"} <= set(names)
    L = ctypes.CDLL(pw.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_host_helpers():
    assert pw.pw_version()
    assert pw.pw_words(1) == 1 and pw.pw_words(64) == 1 and pw.pw_words(65) == 2
    assert pw.pw_num_groups(256, 64, 8) == 32
    assert pw.pw_num_groups(70, 64, 8) == 9
    assert pw.pw_num_groups(75, 64, 8) == 10
    assert pw.pw_num_groups(0, 64, 8) == 0
    assert pw.pw_num_groups(10, 0, 8) == -1
    assert pw.pw_union_capacity(4096, 8, 16, 1024) == 4096 * 128
    assert pw.pw_union_capacity(8, 32, 205, 1024) == 8 * 1024


L = pw.lib()
NULL = None


def _err(status):
    return status, L.pw_last_error().decode()


@pytest.mark.parametrize("args,code", [
    ((NULL, 4, 1, 0, 16, NULL, NULL, NULL), -1),       # k = 0
    ((NULL, 4, 0, 4, 16, NULL, NULL, NULL), -1),       # hkv = 0
    ((NULL, 4, 1, 4, 0, NULL, NULL, NULL), -1),        # n_pages = 0
    ((NULL, 4, 1, 5000, 16, NULL, NULL, NULL), -2),    # k too large
    ((NULL, 4, 1, 4, 70000, NULL, NULL, NULL), -2),    # too many pages
    ((NULL, 4, 1, 4, 16, NULL, NULL, NULL), -1),       # null pointers
])
def test_bitsets_validation(args, code):
    st, msg = _err(L.pw_page_bitsets(*args))
    assert st == code and msg.startswith("pw_page_bitsets")


def test_bitsets_empty_is_ok():
    assert L.pw_page_bitsets(NULL, 0, 1, 4, 16, NULL, NULL, NULL) == 0


@pytest.mark.parametrize("args,code", [
    ((NULL, 64, 1, 16, 64, 9, NULL, NULL, NULL), -2),   # max_group 9
    ((NULL, 64, 1, 16, 60, 8, NULL, NULL, NULL), -1),   # window % max_group
    ((NULL, 64, 1, 16, 2048, 8, NULL, NULL, NULL), -2), # window > 1024
    ((NULL, 64, 1, 5000, 64, 8, NULL, NULL, NULL), -2), # n_pages > 4096
    ((NULL, 64, 1, 16, 64, 8, NULL, NULL, NULL), -1),   # null pointers
    ((NULL, -1, 1, 16, 64, 8, NULL, NULL, NULL), -1),   # nq < 0
])
def test_group_validation(args, code):
    st, msg = _err(L.pw_group(*args))
    assert st == code and msg.startswith("pw_group")


@pytest.mark.parametrize("args,code", [
    # bits, n_rows, hkv, n_pages, rows, size, n_groups, width, k_max, off, pages, qmask, cap, stream
    ((NULL, 8, 1, 16, NULL, NULL, 1, 0, 4, NULL, NULL, NULL, 64, NULL), -2),    # width 0
    ((NULL, 8, 1, 16, NULL, NULL, 1, 65, 4, NULL, NULL, NULL, 64, NULL), -2),   # width 65
    ((NULL, 8, 1, 16, NULL, NULL, 1, 16, 4, NULL, NULL, 1, 64, NULL), -2),      # qmask needs width <= 8
    ((NULL, 8, 1, 16, NULL, NULL, 2, 8, 4, NULL, NULL, NULL, 31, NULL), -3),    # capacity < 2*16
    ((NULL, 8, 1, 16, NULL, NULL, 2, 8, 4, NULL, NULL, NULL, 32, NULL), -1),    # null union_off
])
def test_union_validation(args, code):
    st, msg = _err(L.pw_union_tables(*args))
    assert st == code and msg.startswith("pw_union_tables")


def _attn(**kw):
    a = dict(q=NULL, nq=8, hq=4, hkv=1, d=128, k=NULL, v=NULL, kv_dtype=0, ks=NULL, vs=NULL, ps=64,
             n_pages=4, sh=4 * 64 * 128, sp=64 * 128, q_pos=NULL, kv_len=256, sm=0.088,
             gq=NULL, gs=NULL, n_groups=1, mg=8, shared=0, off=NULL, pages=NULL, qmask=NULL,
             cap=4, order=NULL, out=NULL, lse=NULL, stream=NULL)
    a.update(kw)
    return _err(L.pw_sparse_prefill(*a.values()))


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), -2), (dict(ps=32), -2), (dict(hq=6, hkv=4), -1),
    (dict(mg=9, gq=16, gs=16), -2),                # explicit groups hold <= 8 members
    (dict(hq=16, mg=8, gq=16, gs=16), -2),         # G * max_group = 128 > 64 with groups
    (dict(mg=300), -2),                            # consecutive wide groups: <= 256 members
    (dict(hq=64, mg=8), -2),                       # 512 rows per work item > 256 (bf16, d=128)
    (dict(hq=64, mg=4, kv_dtype=1, ks=16, vs=16), -2),  # fp8 d=128 wide items: <= 128 rows
    (dict(kv_dtype=2), -2), (dict(shared=2), -1), (dict(sp=100), -1),
    (dict(n_groups=0, nq=9), -1),                  # consecutive groups must cover nq
    (dict(sm=0.0), -1), (dict(nq=-1), -1),
    (dict(n_pages=1 << 24), -2),                   # page IDs are packed into 24 bits
    (dict(), -1),                                  # null required pointers
])
def test_attention_validation(kw, code):
    st, msg = _attn(**kw)
    assert st == code and msg.startswith("pw_sparse_prefill"), msg


def test_attention_nothing_to_do_is_ok():
    assert _attn(nq=0)[0] == 0


def test_work_order_needs_per_group_tables():
    fake = 1 << 12      # aligned non-null stand-ins: rejected on the host before any launch
    st, msg = _attn(q=fake, k=fake, v=fake, q_pos=fake, off=fake, pages=fake, out=fake, shared=1,
                    order=fake)
    assert st == -1 and "item_order" in msg, msg


@pytest.mark.parametrize("n,off,order,code", [(-1, NULL, NULL, -1), (4, NULL, 4096, -1),
                                              (4, 4096, NULL, -1), (0, NULL, NULL, 0)])
def test_schedule_validation(n, off, order, code):
    st, msg = _err(L.pw_schedule_items(off, n, order, NULL))
    assert st == code and (code == 0 or msg.startswith("pw_schedule_items")), msg
    assert _attn(n_groups=0, nq=0)[0] == 0


def test_binding_rejects_host_tensors():
    topk = torch.zeros((4, 1, 2), dtype=torch.int32)
    bits = torch.zeros((1, 4, 1), dtype=torch.int64)
    with pytest.raises(ValueError):
        pw.pw_page_bitsets(topk, 16, bits)


@pytest.mark.parametrize("args,code", [
    # topk, nq, hkv, k, n_pages, window, mg, bits, bad, qids, size, off, pages, qmask, cap, order,
    # stream
    ((NULL, 64, 1, 4, 16, 64, 9, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 512, NULL, NULL), -2),  # mg 9
    ((NULL, 64, 1, 4, 16, 60, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 512, NULL, NULL), -1),  # W % mg
    ((NULL, 64, 1, 4, 5000, 64, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 512, NULL, NULL), -2),  # pages
    ((NULL, 64, 1, 4, 16, 64, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 127, NULL, NULL), -3),  # capacity
    ((NULL, 64, 1, 4, 16, 64, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 128, NULL, NULL), -1),  # nulls
])
def test_prepare_validation(args, code):
    st, msg = _err(L.pw_prepare(*args))
    assert st == code and msg.startswith("pw_prepare"), msg


@pytest.mark.parametrize("args,code", [
    # as pw_prepare; the halves' 16 tables of width 4 need 16 * min(16, 4 * 4) = 256 entries
    ((NULL, 64, 1, 4, 16, 64, 7, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 512, NULL, NULL), -1),  # odd mg
    ((NULL, 64, 1, 4, 16, 64, 10, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 512, NULL, NULL), -2),  # mg 10
    ((NULL, 64, 1, 4, 16, 64, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 255, NULL, NULL), -3),  # capacity
    ((NULL, 64, 1, 4, 16, 64, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 256, NULL, NULL), -1),  # nulls
])
def test_prepare_halves_validation(args, code):
    st, msg = _err(L.pw_prepare_halves(*args))
    assert st == code and msg.startswith("pw_prepare_halves"), msg


def _append(**kw):
    a = dict(k_new=NULL, v_new=NULL, n_tok=10, hkv=2, d=128, stride_tok=256, first=0, kc=NULL,
             vc=NULL, kv_dtype=0, ks=NULL, vs=NULL, ps=64, n_pages=4, sh=4 * 64 * 128,
             sp=64 * 128, stream=NULL)
    a.update(kw)
    return _err(L.pw_append_kv(*a.values()))


@pytest.mark.parametrize("kw,code", [
    (dict(d=100), -2), (dict(d=0), -2), (dict(hkv=0), -1), (dict(n_tok=-1), -1),
    (dict(first=-1), -1), (dict(kv_dtype=3), -2),
    (dict(stride_tok=128), -1),                    # < hkv*d
    (dict(stride_tok=260), -1),                    # not a multiple of 8 elements
    (dict(sp=100), -1),                            # stride_page < page_size*d
    (dict(first=250, n_tok=10), -3),               # tokens 250..259 past 4 pages of 64
    (dict(), -1),                                  # null pointers
    (dict(kv_dtype=1, k_new=16, v_new=16, kc=16, vc=16), -1),   # fp8 without scales
])
def test_append_validation(kw, code):
    st, msg = _append(**kw)
    assert st == code and msg.startswith("pw_append_kv"), msg


def test_append_nothing_to_do_is_ok():
    assert _append(n_tok=0)[0] == 0


def test_page_workspace_bytes():
    assert pw.pw_page_workspace_bytes(4096, 8, 1024) == 8 * 1024 * 64 * 8 + 8 * 4096 * 16 * 4
    assert pw.pw_page_workspace_bytes(0, 1, 1) == 0 and pw.pw_page_workspace_bytes(-1, 1, 1) == 0


def test_page_items_capacity():
    assert pw.pw_page_items_capacity(4096, 8, 16, 1024, 8) == (4096 * 8 * 16 + 8192 * 7 + 7) // 8
    assert pw.pw_page_items_capacity(10, 1, 4, 2, 8) == (10 * 2 + 2 * 7 + 7) // 8   # k_max capped at n_pages
    assert pw.pw_page_items_capacity(3, 1, 4, 100, 8) == 12                          # items <= edges
    assert pw.pw_page_items_capacity(-1, 1, 4, 2, 8) == -1


@pytest.mark.parametrize("args,code", [
    # bits, nq, hkv, n_pages, k_max, chunk, ws, ws_bytes, off, kvh, page, qids, size, slot, cap, stream
    ((NULL, 64, 1, 16, 4, 0, NULL, 1 << 20, NULL, NULL, NULL, NULL, NULL, NULL, 1000, NULL), -2),  # chunk 0
    ((NULL, 64, 1, 16, 4, 65, NULL, 1 << 20, NULL, NULL, NULL, NULL, NULL, NULL, 1000, NULL), -2), # chunk 65
    ((NULL, 64, 1, 70000, 4, 8, NULL, 1 << 30, NULL, NULL, NULL, NULL, NULL, NULL, 10 ** 6, NULL), -2),
    ((NULL, 64, 1, 16, 0, 8, NULL, 1 << 20, NULL, NULL, NULL, NULL, NULL, NULL, 1000, NULL), -1),  # k_max 0
    ((NULL, 64, 1, 16, 4, 8, NULL, 1 << 20, NULL, NULL, NULL, NULL, NULL, NULL, 33, NULL), -3),    # capacity
    ((NULL, 64, 1, 16, 4, 8, NULL, 100, NULL, NULL, NULL, NULL, NULL, NULL, 1000, NULL), -3),      # workspace
    ((NULL, 64, 1, 16, 4, 8, NULL, 1 << 20, NULL, NULL, NULL, NULL, NULL, NULL, 1000, NULL), -1),  # nulls
])
def test_page_tables_validation(args, code):
    st, msg = _err(L.pw_page_tables(*args))
    assert st == code and msg.startswith("pw_page_tables"), msg


def _page_attn(**kw):
    a = dict(q=NULL, nq=8, hq=4, hkv=1, d=128, k=NULL, v=NULL, kv_dtype=0, ks=NULL, vs=NULL, ps=64,
             n_pages=4, sh=4 * 64 * 128, sp=64 * 128, q_pos=NULL, kv_len=256, sm=0.088, bits=NULL,
             k_max=4, chunk=8, off=NULL, kvh=NULL, page=NULL, qids=NULL, size=NULL, slot=NULL,
             cap=16, po=NULL, pl=NULL, out=NULL, lse=NULL, stream=NULL)
    a.update(kw)
    return _err(L.pw_page_union_prefill(*a.values()))


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), -2), (dict(ps=32), -2), (dict(hq=6, hkv=4), -1), (dict(kv_dtype=2), -2),
    (dict(chunk=65), -2), (dict(chunk=0), -2), (dict(hq=64, chunk=8), -2),  # 64 * 8 rows > 256
    (dict(k_max=0), -1), (dict(k_max=5000), -2),                           # k_max * G > 16384
    (dict(sp=100), -1), (dict(sm=0.0), -1), (dict(), -1),
])
def test_page_union_validation(kw, code):
    st, msg = _page_attn(**kw)
    assert st == code and msg.startswith("pw_page_union_prefill"), msg


def test_page_union_nothing_to_do_is_ok():
    assert _page_attn(nq=0)[0] == 0


def _shared(**kw):
    a = dict(q=NULL, nq=8, hq=4, hkv=1, d=128, k=NULL, v=NULL, kv_dtype=0, ks=NULL, vs=NULL, ps=64,
             n_pages=4, sh=4 * 64 * 128, sp=64 * 128, q_pos=NULL, kv_len=256, sm=0.088, mg=8,
             off=NULL, pages=NULL, cap=4, n_split=2, po=NULL, pl=NULL, out=NULL, lse=NULL, stream=NULL)
    a.update(kw)
    return _err(L.pw_shared_table_prefill(*a.values()))


@pytest.mark.parametrize("kw,code", [
    (dict(n_split=0), -2), (dict(n_split=65), -2), (dict(mg=0), -1),
    (dict(), -1),                                   # no partial buffers for n_split > 1
    (dict(po=16, pl=16, d=96), -2),                 # the attention's own checks
    (dict(po=16, pl=16, hq=64, mg=8), -2),          # 512 rows per work item
])
def test_shared_table_validation(kw, code):
    st, msg = _shared(**kw)
    assert st == code and msg.startswith(("pw_shared_table_prefill", "pw_sparse_prefill")), msg


def test_shared_table_nothing_to_do_is_ok():
    assert _shared(nq=0, po=16, pl=16)[0] == 0


@pytest.mark.parametrize("args,code", [
    # bits, nq, hkv, n_pages, hq, n_groups, mg, qids, size, off, qmask, cap, stream
    ((NULL, 64, 2, 16, 8, 8, 9, NULL, NULL, NULL, NULL, 0, NULL), -2),     # max_group 9
    ((NULL, 64, 2, 16, 7, 8, 8, NULL, NULL, NULL, NULL, 0, NULL), -1),     # hq % hkv
    ((NULL, 64, 2, 70000, 8, 8, 8, NULL, NULL, NULL, NULL, 0, NULL), -2),  # n_pages
    ((NULL, 64, 2, 16, 8, 8, 8, NULL, NULL, NULL, NULL, 0, NULL), -1),     # null pointers (G = 4)
])
def test_arrange_validation(args, code):
    st, msg = _err(L.pw_arrange_groups(*args))
    assert st == code and msg.startswith("pw_arrange_groups"), msg


def test_arrange_is_a_noop_where_tiles_leave_no_choice():
    assert L.pw_arrange_groups(NULL, 64, 2, 16, 16, 8, 8, NULL, NULL, NULL, NULL, 0, NULL) == 0  # G = 8
    assert L.pw_arrange_groups(NULL, 64, 2, 16, 8, 16, 4, NULL, NULL, NULL, NULL, 0, NULL) == 0  # 4 members


def test_sparse_prefill_rejects_bad_half_groups():
    """halves=True needs per-query mode, an even group size and no member arrangement
    (checked before any device memory is touched)."""
    kw = dict(nq=64, hq=8, hkv=2, d=128, n_pages=16, page_size=64, kv_len=1024, k=4, device="cpu")
    with pytest.raises(ValueError):
        pw.SparsePrefill(max_group=7, halves=True, **kw)
    with pytest.raises(ValueError):
        pw.SparsePrefill(max_group=8, halves=True, arrange=True, **kw)
    with pytest.raises(ValueError):
        pw.SparsePrefill(max_group=8, halves=True, mode="block_union", n_rows=8, **kw)


def test_debug_build_loads_and_exports_every_symbol():
    """libpw_debug.so (-DPW_DEBUG) is built beside libpw.so and exports the same entry
    points; the release build reports no debug counters (-2, no device call)."""
    assert os.path.exists(pw.DEBUG_LIB_PATH)
    D = ctypes.CDLL(pw.DEBUG_LIB_PATH)
    for n in _declared():
        assert hasattr(D, n), n
    L.pw_debug_violations.restype = ctypes.c_int64
    assert L.pw_debug_violations() == -2
