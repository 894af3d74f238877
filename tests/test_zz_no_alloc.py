"""GPU: pw_shared_table_prefill_noalloc (the slice partials in the library's own device
array) against pw_shared_table_prefill with caller-allocated partials, through the C ABI:
two calls in a row, the second with a smaller input, and the size limit."""
import ctypes
import math

import numpy as np
import pytest
import torch

import query_union_kv_amd as pw
from gpu_util import device_inputs
from oracle import prep
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu


def _noalloc(q, k, v, q_pos, kv_len, off, pages, out, lse, hkv, max_group, n_split, k_scale=None,
             v_scale=None):
    nq, hq, d = q.shape
    _, n_pages, ps, _ = k.shape
    fp8 = k.dtype == torch.uint8
    L = pw.lib()
    st = L.pw_shared_table_prefill_noalloc(
        q.data_ptr(), nq, hq, hkv, d, k.data_ptr(), v.data_ptr(), 1 if fp8 else 0,
        k_scale.data_ptr() if fp8 else None, v_scale.data_ptr() if fp8 else None, ps, n_pages,
        n_pages * ps * d, ps * d, q_pos.data_ptr(), kv_len, 1.0 / math.sqrt(d), max_group,
        off.data_ptr(), pages.data_ptr(), pages.numel(), n_split, out.data_ptr(),
        lse.data_ptr() if lse is not None else None, torch.cuda.current_stream().cuda_stream)
    return st, L.pw_last_error().decode()


def _case(cfg, n_split, max_group):
    w = make_workload(cfg)
    d = device_inputs(w)
    tables = prep.block_tables(w.mask_rows if w.mask_rows is not None else w.topk, cfg.n_pages)
    off = np.zeros(cfg.hkv + 1, dtype=np.int32)
    off[1:] = np.cumsum([len(t) for t in tables])
    off_t = torch.from_numpy(off).cuda()
    pages_t = torch.from_numpy(np.concatenate([np.asarray(t, dtype=np.int32) for t in tables])).cuda()
    rows = cfg.nq * cfg.hq * n_split
    part_o = torch.empty((rows, cfg.d), dtype=torch.bfloat16, device="cuda")
    part_lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    ref = torch.full_like(d["q"], float("nan"))
    ref_lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pw.pw_shared_table_prefill(d["q"], d["k"], d["v"], d["q_pos"], cfg.kv_len, off_t, pages_t, ref,
                               hkv=cfg.hkv, max_group=max_group, n_split=n_split, partial_o=part_o,
                               partial_lse=part_lse, k_scale=d["k_scale"], v_scale=d["v_scale"],
                               lse=ref_lse)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    st, msg = _noalloc(d["q"], d["k"], d["v"], d["q_pos"], cfg.kv_len, off_t, pages_t, out, lse,
                       cfg.hkv, max_group, n_split, d["k_scale"], d["v_scale"])
    torch.cuda.synchronize()
    assert st == 0, msg
    return out, lse, ref, ref_lse


def test_noalloc_equals_allocating_entry_point_twice():
    """The 128K block-union chunk at its full size (1024 queries, 32 heads, 2 slices: 17 MB of
    partials), then a smaller fp8 call: both equal the allocating entry point bit for bit."""
    print("[no-alloc] block-union 1024 queries, n_split=2", flush=True)
    out, lse, ref, ref_lse = _case(CONFIGS["c4_block_union"], n_split=2, max_group=4)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    print("[no-alloc] smaller fp8 call, n_split=3", flush=True)
    small = CONFIGS["c3_long_fp8"].scaled(nq=200, kv_len=8192, seed=9)
    out, lse, ref, ref_lse = _case(small, n_split=3, max_group=8)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))


def test_noalloc_rejects_partials_beyond_its_array():
    L = pw.lib()
    L.pw_noalloc_scratch_bytes.restype = ctypes.c_size_t
    cap = L.pw_noalloc_scratch_bytes()
    assert cap == 32 << 20
    nq, hq, d, n_split = 4096, 64, 128, 2          # 524288 partial rows: 130 MiB
    q = torch.zeros((nq, hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((8, 16, 64, d), dtype=torch.bfloat16, device="cuda")
    q_pos = torch.zeros(nq, dtype=torch.int32, device="cuda")
    off = torch.zeros(9, dtype=torch.int32, device="cuda")
    pages = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    st, msg = _noalloc(q, k, k, q_pos, 1024, off, pages, out, None, 8, 8, n_split)
    assert st == -3 and "scratch" in msg
