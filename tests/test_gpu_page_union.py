"""GPU parity of the direct KV-page union (pw_page_tables + pw_page_union_prefill):
page-major work items bit for bit against the oracle's, and attention outputs
against the definition (route A) at the same tolerances as the query-union path."""
import numpy as np
import pytest
import torch

import query_union_kv_amd as pw
from gpu_util import check_close, check_lse, device_inputs, oracle_attention
from helpers import add_padding_and_duplicates
from oracle import prep
from workloads import CONFIGS, make_workload
from workloads.configs import Config

pytestmark = pytest.mark.gpu


def run_page(w, chunk=8):
    c = w.cfg
    d = device_inputs(w)
    plan = pw.PageUnionPrefill(nq=c.nq, hq=c.hq, hkv=c.hkv, d=c.d, n_pages=c.n_pages, page_size=c.ps,
                               kv_len=c.kv_len, k=w.topk.shape[2], chunk=chunk)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    plan(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], out, d["k_scale"], d["v_scale"], lse)
    torch.cuda.synchronize()
    n = plan.n_items
    res = {"out": out.float().cpu().numpy(), "lse": lse.cpu().numpy(), "n_items": n,
           "item_off": plan.item_off.cpu().numpy(), "item_kvh": plan.item_kvh[:n].cpu().numpy(),
           "item_page": plan.item_page[:n].cpu().numpy(), "item_qids": plan.item_qids[:n].cpu().numpy(),
           "item_size": plan.item_size[:n].cpu().numpy(), "item_slot": plan.item_slot[:n].cpu().numpy()}
    assert n <= plan.item_kvh.numel()
    return res


def oracle_items(w, chunk=8):
    c = w.cfg
    bits = prep.page_bitsets(w.topk, c.n_pages)
    items = prep.page_items(bits, c.n_pages, chunk, w.topk.shape[2])
    kvh, pages, qids, slots, size = prep.page_items_to_arrays(items, chunk)
    counts = np.zeros(c.hkv * c.n_pages, dtype=np.int64)
    np.add.at(counts, kvh.astype(np.int64) * c.n_pages + pages, 1)
    off = np.zeros(c.hkv * c.n_pages + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    return {"item_off": off, "item_kvh": kvh, "item_page": pages, "item_qids": qids,
            "item_size": size, "item_slot": slots, "S": prep.supports(w.topk, c.n_pages)}


def compare_items(res, ref):
    assert res["n_items"] == len(ref["item_kvh"]), "item count differs"
    for k in ("item_off", "item_kvh", "item_page", "item_qids", "item_size", "item_slot"):
        assert np.array_equal(res[k], ref[k]), f"{k} differs"


TOPK_WORKLOADS = [n for n, c in CONFIGS.items() if c.support != "block_union"]


@pytest.mark.parametrize("name", TOPK_WORKLOADS)
def test_workload_parity(name):
    cfg = CONFIGS[name]
    print(f"[page-union] {name}", flush=True)
    w = make_workload(cfg)
    res = run_page(w)
    ref = oracle_items(w)
    compare_items(res, ref)
    O, L = oracle_attention(w, ref["S"])                # every row
    mx, mean, nrms = check_close(res["out"], O, cfg.kv_dtype, name)
    check_lse(res["lse"], L, name)
    print(f"[page-union] {name}: items={res['n_items']} rows={cfg.nq * cfg.hq} max_abs={mx:.3e} "
          f"mean_abs={mean:.3e}", flush=True)


def _small(**kw):
    base = dict(name="small", hq=4, hkv=1, d=128, ps=64, kv_len=1024, nq=65, kv_dtype="bf16",
                support="uniform", k=4, forced=False, seed=41)
    base.update(kw)
    return Config(**base)


SMALL = [
    (dict(nq=1), 8), (dict(nq=9), 8), (dict(nq=65), 3), (dict(nq=130, k=16, kv_len=4096), 1),
    (dict(hq=8, hkv=1, k=8, kv_len=2048), 8), (dict(hq=16, hkv=2, k=5), 4), (dict(hq=1, hkv=1), 8),
    (dict(d=64), 8), (dict(ps=128, kv_len=2048), 8), (dict(kv_dtype="fp8", k=8, kv_len=2048), 8),
    (dict(kv_dtype="fp8", d=64, hq=8, hkv=2), 5), (dict(kv_len=1000, nq=77), 8),
    (dict(k=64, kv_len=8192, nq=70, hq=8, hkv=1), 8),
    (dict(support="community", k=6, n_comm=4, comm_size=6, forced=True, kv_len=2048, nq=200), 8),
    (dict(nq=200, k=8, kv_len=2048), 16), (dict(nq=300, hq=8, hkv=1, k=8, kv_len=2048), 32),
    (dict(kv_dtype="fp8", hq=8, hkv=2, k=8, kv_len=2048, nq=150), 32),
    (dict(nq=5000, hq=2, hkv=2, k=3, kv_len=8192), 64),                 # columns over 64 words
]


@pytest.mark.parametrize("kw,chunk", SMALL, ids=[",".join(f"{k}={v}" for k, v in s.items()) + f",chunk={c}"
                                                 for s, c in SMALL])
def test_small_shapes(kw, chunk):
    cfg = _small(**kw)
    print(f"[page-union] small {kw} chunk={chunk}", flush=True)
    w = make_workload(cfg)
    w.topk = add_padding_and_duplicates(w.topk, seed=cfg.seed)
    res = run_page(w, chunk)
    ref = oracle_items(w, chunk)
    compare_items(res, ref)
    O, L = oracle_attention(w, ref["S"])
    check_close(res["out"], O, cfg.kv_dtype, str(kw))
    check_lse(res["lse"], L, str(kw))


def test_headline_workload_wide_items():
    """The 64K fp8 Top16 workload with 16 queries (64 rows) per work item."""
    cfg = CONFIGS["c3_long_fp8"]
    w = make_workload(cfg)
    res = run_page(w, chunk=16)
    ref = oracle_items(w, chunk=16)
    compare_items(res, ref)
    O, L = oracle_attention(w, ref["S"])
    check_close(res["out"], O, cfg.kv_dtype, "c3 chunk 16")
    check_lse(res["lse"], L, "c3 chunk 16")


def test_future_pages_and_empty_supports():
    cfg = _small(nq=200, kv_len=1024, k=3, hq=8, hkv=2)
    w = make_workload(cfg)
    n_pages = cfg.n_pages
    w.topk[:5] = -1                                  # empty supports: O = 0, lse = -inf
    w.topk[5:10, :, 0] = n_pages - 1                 # a page wholly in these queries' future
    w.topk[10:15, :, :] = n_pages - 1                # only future pages
    res = run_page(w)
    ref = oracle_items(w)
    compare_items(res, ref)
    O, L = oracle_attention(w, ref["S"])
    check_close(res["out"], O, "bf16", "future/empty")
    check_lse(res["lse"], L, "future/empty")
    assert (res["out"][:5] == 0).all() and np.isneginf(res["lse"][:5]).all()


def test_repeated_calls_are_identical():
    w = make_workload(_small(nq=100, k=8, kv_len=2048, hq=8, hkv=2, kv_dtype="fp8"))
    a = run_page(w)
    b = run_page(w)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])


def test_kv_head_batches_give_identical_results(monkeypatch):
    """Running the KV heads in batches (attention then merge per batch) changes only the
    order of launches, so every bit of the output is the same."""
    w = make_workload(_small(nq=150, k=8, kv_len=2048, hq=16, hkv=4, kv_dtype="fp8"))
    monkeypatch.delenv("PW_PAGE_HEAD_BATCH", raising=False)
    a = run_page(w, chunk=8)
    for hb in ("1", "3"):
        monkeypatch.setenv("PW_PAGE_HEAD_BATCH", hb)
        b = run_page(w, chunk=8)
        assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"]), hb
