"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer outputs (bitsets, groups, union tables, member masks) must match bit for
bit; attention outputs must be within max-abs 2e-2 and mean-abs 2e-3 for bf16 KV
and max-abs 6e-2 for fp8 KV.  Every workload, the five full-size ones included,
compares every integer table and every attention row and lse against the
oracle.
"""
import os

import numpy as np
import pytest
import torch

import query_union_kv_amd as pw
from gpu_util import (check_close, check_lse, device_inputs, oracle_attention, oracle_tables,
                      run_gpu)
from oracle import prep
from helpers import add_padding_and_duplicates
from workloads import CONFIGS, make_workload
from workloads.configs import Config

pytestmark = pytest.mark.gpu


def _compare_tables(res, ref, has_groups=True):
    assert np.array_equal(res["bits"], ref["bits"]), "bitsets differ"
    if has_groups:
        assert np.array_equal(res["group_size"], ref["group_size"]), "group sizes differ"
        assert np.array_equal(res["group_qids"], ref["group_qids"]), "group ids differ"
    assert np.array_equal(res["union_off"], ref["union_off"]), "union offsets differ"
    assert np.array_equal(res["union_pages"], ref["union_pages"]), "union pages differ"
    if has_groups:
        assert np.array_equal(res["union_qmask"], ref["union_qmask"]), "member masks differ"


@pytest.mark.parametrize("name", list(CONFIGS))
def test_workload_parity(name):
    cfg = CONFIGS[name]
    print(f"[parity] {name}", flush=True)
    w = make_workload(cfg)
    res, _ = run_gpu(w)
    ref = oracle_tables(w)
    _compare_tables(res, ref, has_groups=w.topk is not None)
    assert res["bad_ids"] == 0
    O, L = oracle_attention(w, ref["S"])                # every row
    mx, mean, nrms = check_close(res["out"], O, cfg.kv_dtype, name)
    check_lse(res["lse"], L, name)
    print(f"[parity] {name}: rows={cfg.nq * cfg.hq} max_abs={mx:.3e} mean_abs={mean:.3e} nrms={nrms:.3f}%",
          flush=True)
    if w.topk is not None and cfg.g * cfg.max_group > 32:
        # the default plan runs these wide groups as two halves over their own unions: the
        # halves' tables are the oracle's unions of each half, and every output and lse bit
        # equals the whole-group run checked above
        hv, plan = run_gpu(w, halves=True)
        assert plan.halves
        half = [[h for m in grp for h in (m[:cfg.max_group // 2], m[cfg.max_group // 2:])]
                for grp in ref["groups"]]
        off, pages, qmask = prep.union_tables(prep.page_bitsets(w.topk, cfg.n_pages), half)
        assert np.array_equal(hv["union_off"], off)
        assert np.array_equal(hv["union_pages"], pages)
        assert np.array_equal(hv["union_qmask"], qmask)
        assert np.array_equal(hv["out"], res["out"]) and np.array_equal(hv["lse"], res["lse"])


def _small(**kw):
    base = dict(name="small", hq=4, hkv=1, d=128, ps=64, kv_len=1024, nq=65, kv_dtype="bf16",
                support="uniform", k=4, forced=False, window=64, max_group=8, seed=31)
    base.update(kw)
    return Config(**base)


SMALL = [
    dict(nq=1), dict(nq=7), dict(nq=8), dict(nq=9), dict(nq=63), dict(nq=64), dict(nq=65),
    dict(k=1), dict(k=16, kv_len=2048), dict(k=64, kv_len=8192, nq=130),
    dict(hq=1, hkv=1), dict(hq=8, hkv=1), dict(hq=16, hkv=2, max_group=4),
    dict(d=64), dict(ps=128, kv_len=2048), dict(kv_dtype="fp8"), dict(kv_dtype="fp8", d=64),
    dict(kv_dtype="fp8", hq=8, hkv=1, k=16, kv_len=4096), dict(kv_len=1000, nq=77),
    dict(window=16, max_group=4), dict(window=128, nq=300, k=8, kv_len=4096),
    dict(window=1024, nq=1100, k=6, kv_len=2048, hq=2, hkv=2), dict(max_group=1),
    dict(support="community", k=6, n_comm=4, comm_size=6, forced=True, kv_len=2048, nq=200),
    dict(hq=12, hkv=4, max_group=5, window=60, nq=100, k=5),
]


@pytest.mark.parametrize("kw", SMALL, ids=[",".join(f"{k}={v}" for k, v in s.items()) for s in SMALL])
def test_small_shapes(kw):
    cfg = _small(**kw)
    print(f"[parity] small {kw}", flush=True)
    w = make_workload(cfg)
    w.topk = add_padding_and_duplicates(w.topk, seed=cfg.seed)
    res, _ = run_gpu(w)
    ref = oracle_tables(w)
    _compare_tables(res, ref)
    O, L = oracle_attention(w, ref["S"])
    check_close(res["out"], O, cfg.kv_dtype, str(kw))
    check_lse(res["lse"], L, str(kw))


MAX_SHAPES = [
    # the preparation's page limit (4096 pages: the separate steps) with TopK 512 per query
    dict(hq=2, hkv=1, d=64, ps=64, kv_len=262144, nq=16, k=512, window=16, max_group=8, kv_dtype="fp8"),
    # the largest grouping window (1024 candidates: the general grouping kernel)
    dict(hq=1, hkv=1, d=64, ps=64, kv_len=70400, nq=1024, k=64, window=1024, max_group=8, kv_dtype="bf16"),
]


@pytest.mark.parametrize("kw", MAX_SHAPES, ids=["pages4096-k512", "window1024"])
def test_maximum_sizes(kw):
    """The limits of the preparation calls (4096 pages, TopK 512, a 1024-query window) through
    the whole path: tables bit-exact, every output row and lse within tolerance."""
    cfg = Config(name="max", support="uniform", forced=True, seed=77, **kw)
    print(f"[parity] maximum sizes {kw}", flush=True)
    w = make_workload(cfg)
    res, _ = run_gpu(w)
    ref = oracle_tables(w)
    _compare_tables(res, ref)
    assert res["bad_ids"] == 0
    O, L = oracle_attention(w, ref["S"])
    check_close(res["out"], O, cfg.kv_dtype, "maximum sizes")
    check_lse(res["lse"], L, "maximum sizes")


def test_future_pages_and_empty_supports():
    cfg = _small(nq=200, kv_len=1024, k=3, hq=8, hkv=2)   # queries on pages 12..15
    w = make_workload(cfg)
    n_pages = cfg.n_pages
    w.topk[:5] = -1                                  # empty supports: O = 0, lse = -inf
    w.topk[5:10, :, 0] = n_pages - 1                 # page 15 lies wholly in these queries' future
    w.topk[10:15, :, :] = n_pages - 1                # only future pages
    res, _ = run_gpu(w)
    ref = oracle_tables(w)
    _compare_tables(res, ref)
    O, L = oracle_attention(w, ref["S"])
    check_close(res["out"], O, "bf16", "future/empty")
    check_lse(res["lse"], L, "future/empty")
    assert (res["out"][:5] == 0).all()


def test_out_of_range_ids_are_counted_and_ignored():
    cfg = _small(nq=16, k=4, hq=4, hkv=2)
    w = make_workload(cfg)
    w.topk[3, 1, 2] = cfg.n_pages + 5
    w.topk[7, 0, 0] = 1 << 20
    res, _ = run_gpu(w)
    assert res["bad_ids"] == 2
    cleaned = w.topk.copy()
    cleaned[cleaned >= cfg.n_pages] = -1
    w.topk = cleaned
    ref = oracle_tables(w)
    _compare_tables(res, ref)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_grouping_invariance_on_gpu(kv_dtype):
    cfg = _small(nq=128, k=6, hq=8, hkv=2, kv_len=4096, kv_dtype=kv_dtype,
                 support="community", n_comm=6, comm_size=10, forced=True)
    w = make_workload(cfg)
    outs = {}
    for name, kw in {"affinity": {}, "original": dict(grouping="original"),
                     "singletons": dict(max_group=1, window=1)}.items():
        res, _ = run_gpu(w, **kw)
        outs[name] = res["out"]
    ref = oracle_attention(w, oracle_tables(w)["S"])[0]
    for name, o in outs.items():
        check_close(o, ref, kv_dtype, name)
    # masked pages are exact no-ops, so the grouping does not change a single bit
    assert np.array_equal(outs["affinity"], outs["original"])
    assert np.array_equal(outs["affinity"], outs["singletons"])


def test_run_to_run_determinism():
    w = make_workload(CONFIGS["c2_gqa_bf16"].scaled(nq=512, kv_len=4096 + 512))
    a, _ = run_gpu(w)
    b, _ = run_gpu(w)
    for k in ("out", "lse", "group_qids", "union_pages", "union_qmask"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k


FUSE_SHAPES = [
    dict(nq=200, k=6, kv_len=2048),                                  # fused path
    dict(nq=77, k=16, kv_len=4096, hq=8, hkv=2, window=32, max_group=4),
    dict(nq=130, k=3, kv_len=65536, ps=64),                          # 1024 pages: last fused size
    dict(nq=100, k=4, kv_len=70000),                                 # 1094 pages: three steps
    dict(nq=300, k=8, kv_len=4096, window=128),                      # window > 64: three steps
    dict(nq=9, k=64, kv_len=8192, max_group=1),
]


@pytest.mark.parametrize("kw", FUSE_SHAPES, ids=[",".join(f"{k}={v}" for k, v in s.items()) for s in FUSE_SHAPES])
def test_fused_prepare_equals_separate_steps(kw):
    """pw_prepare gives the same bitsets, groups and tables as the three separate calls,
    and both equal the oracle."""
    cfg = _small(**kw)
    print(f"[parity] fused {kw}", flush=True)
    w = make_workload(cfg)
    w.topk = add_padding_and_duplicates(w.topk, seed=cfg.seed + 1)
    a, _ = run_gpu(w, fused=True)
    b, _ = run_gpu(w, fused=False)
    for key in ("bits", "group_qids", "group_size", "union_off", "union_pages", "union_qmask",
                "item_order", "out"):
        assert np.array_equal(a[key], b[key]), key
    _compare_tables(a, oracle_tables(w))


HALF_SHAPES = [
    dict(hq=16, hkv=2, nq=130, k=16, kv_len=4096, kv_dtype="fp8"),           # G = 8: 64-row groups
    dict(hq=16, hkv=2, nq=77, k=8, kv_len=2048, kv_dtype="bf16"),            # ragged last window
    dict(hq=8, hkv=2, nq=200, k=16, kv_len=8192, kv_dtype="fp8", window=32),  # G = 4
]


@pytest.mark.parametrize("kw", HALF_SHAPES, ids=["g8-fp8", "g8-bf16-ragged", "g4-fp8"])
def test_half_groups_bit_identical(kw):
    """Running every group as two halves over their own unions gives the outputs and lse of
    the whole-group execution bit for bit, and both match the oracle."""
    from gpu_util import make_plan
    cfg = _small(**kw)
    print(f"[parity] half groups {kw}", flush=True)
    w = make_workload(cfg)
    w.topk = add_padding_and_duplicates(w.topk, seed=cfg.seed + 3)
    d = device_inputs(w)
    res = []
    for halves in (False, True):
        base = make_plan(w)
        plan = type(base)(**{**{f: getattr(base, f) for f in ("nq", "hq", "hkv", "d", "n_pages", "page_size",
                                                               "kv_len", "k", "window", "max_group", "mode",
                                                               "grouping", "n_rows", "fused")},
                             "halves": halves})
        out = torch.full_like(d["q"], float("nan"))
        lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        plan(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], out, d["k_scale"], d["v_scale"], lse)
        torch.cuda.synchronize()
        res.append((out.view(torch.int16).cpu(), lse.cpu(), plan))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    # the halves' tables are the unions of each half's members
    ref = oracle_tables(w)
    assert np.array_equal(res[1][2].group_qids.cpu().numpy(), ref["group_qids"])
    bits = prep.page_bitsets(w.topk, cfg.n_pages)
    halves_per_head = [[h for m in grp for h in (m[:cfg.max_group // 2], m[cfg.max_group // 2:])]
                       for grp in ref["groups"]]
    off, pages, qmask = prep.union_tables(bits, halves_per_head)
    plan = res[1][2]
    assert np.array_equal(plan.union_off.cpu().numpy(), off)
    assert np.array_equal(plan.union_pages[:len(pages)].cpu().numpy(), pages)
    assert np.array_equal(plan.union_qmask[:len(qmask)].cpu().numpy(), qmask)
    O, L = oracle_attention(w, ref["S"])
    check_close(res[1][0].view(torch.bfloat16).float().numpy(), O, cfg.kv_dtype, "halves")
    check_lse(res[1][1].numpy(), L, "halves")


HALF_PREP_SHAPES = [
    dict(hq=8, hkv=2, nq=200, k=16, kv_len=8192, kv_dtype="fp8", window=64, max_group=8),
    dict(hq=4, hkv=1, nq=77, k=8, kv_len=4096, window=16, max_group=4),       # ragged last window
    dict(hq=2, hkv=1, nq=130, k=6, kv_len=8192, window=60, max_group=6),      # odd half width 3
    dict(hq=2, hkv=2, nq=90, k=5, kv_len=4096, window=64, max_group=2),       # halves of one member
    dict(hq=4, hkv=1, nq=100, k=8, kv_len=70016, window=64, max_group=8),     # 1094 pages: separate steps
    dict(hq=4, hkv=1, nq=150, k=8, kv_len=8192, window=128, max_group=8),     # W = 128: separate steps
]


@pytest.mark.parametrize("schedule", [True, False], ids=["order", "no-order"])
@pytest.mark.parametrize("kw", HALF_PREP_SHAPES,
                         ids=["mg8", "mg4-ragged", "mg6", "mg2", "pages1094", "w128"])
def test_fused_half_tables_equal_separate_steps(kw, schedule):
    """pw_prepare_halves (bitsets, groups, the halves' union tables and their work order in
    the fused launches where the shape allows) writes the bytes of the separate calls -
    pw_page_bitsets, pw_group, pw_union_tables over the member lists viewed as halves,
    pw_schedule_items - and the tables are the oracle's unions of each half."""
    from gpu_util import make_plan
    cfg = _small(**kw)
    print(f"[parity] fused half tables {kw}", flush=True)
    w = make_workload(cfg)
    w.topk = add_padding_and_duplicates(w.topk, seed=cfg.seed + 5)
    d = device_inputs(w)
    plans = []
    for fused in (True, False):
        base = make_plan(w)
        plan = type(base)(**{**{f: getattr(base, f) for f in ("nq", "hq", "hkv", "d", "n_pages", "page_size",
                                                               "kv_len", "k", "window", "max_group", "mode",
                                                               "grouping", "n_rows")},
                             "fused": fused, "halves": True, "schedule": schedule})
        for t in (plan.union_off, plan.union_pages, plan.group_qids, plan.item_order):
            if t is not None:
                t.fill_(-7)
        plan.union_qmask.fill_(0xAB)
        plan.prepare(d["ids"])
        plans.append(plan)
    torch.cuda.synchronize()
    a, b = plans
    total = int(a.union_off[-1].item())
    assert torch.equal(a.bits, b.bits)
    assert torch.equal(a.group_qids, b.group_qids) and torch.equal(a.group_size, b.group_size)
    assert torch.equal(a.union_off, b.union_off)
    assert torch.equal(a.union_pages[:total], b.union_pages[:total])
    assert torch.equal(a.union_qmask[:total], b.union_qmask[:total])
    assert (a.item_order is None) == (not schedule)
    if schedule:
        assert torch.equal(a.item_order, b.item_order)
    ref = oracle_tables(w)
    bits = prep.page_bitsets(w.topk, cfg.n_pages)
    h = cfg.max_group // 2
    halves_per_head = [[x for m in grp for x in (m[:h], m[h:])] for grp in ref["groups"]]
    off, pages, qmask = prep.union_tables(bits, halves_per_head)
    assert np.array_equal(a.union_off.cpu().numpy(), off)
    assert np.array_equal(a.union_pages[:total].cpu().numpy(), pages)
    assert np.array_equal(a.union_qmask[:total].cpu().numpy(), qmask)


@pytest.mark.parametrize("n_split", [1, 2, 3, 7])
def test_block_union_table_slices(n_split):
    """Shared per-KV-group tables cut into n_split slices (partials merged by lse) give the
    attention of the whole table."""
    from gpu_util import make_plan, device_inputs
    cfg = CONFIGS["c4_block_union"].scaled(kv_len=16384, nq=256, seed=44)
    print(f"[parity] block-union slices n_split={n_split}", flush=True)
    w = make_workload(cfg)
    d = device_inputs(w)
    plan = make_plan(w)
    plan_split = type(plan)(**{**{f: getattr(plan, f) for f in ("nq", "hq", "hkv", "d", "n_pages", "page_size",
                                                              "kv_len", "k", "window", "max_group", "mode",
                                                              "grouping", "n_rows", "fused")},
                               "n_split": n_split})
    assert plan_split.n_split == n_split
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    plan_split(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], out, d["k_scale"], d["v_scale"], lse)
    torch.cuda.synchronize()
    ref = oracle_tables(w)
    O, L = oracle_attention(w, ref["S"])
    check_close(out.float().cpu().numpy(), O, cfg.kv_dtype, f"n_split={n_split}")
    check_lse(lse.cpu().numpy(), L, f"n_split={n_split}")


def test_one_call_convenience_matches_oracle():
    from gpu_util import device_inputs
    cfg = _small(nq=130, k=8, kv_len=2048, hq=8, hkv=2, kv_dtype="fp8")
    w = make_workload(cfg)
    d = device_inputs(w)
    out, aux = pw.sparse_prefill(d["q"], d["k"], d["v"], d["ids"], d["q_pos"], kv_len=cfg.kv_len,
                                 k_scale=d["k_scale"], v_scale=d["v_scale"], window=cfg.window,
                                 max_group=cfg.max_group, with_lse=True)
    torch.cuda.synchronize()
    ref = oracle_tables(w)
    assert np.array_equal(aux["group_qids"].cpu().numpy(), ref["group_qids"])
    O, L = oracle_attention(w, ref["S"])
    check_close(out.float().cpu().numpy(), O, cfg.kv_dtype, "sparse_prefill")
    check_lse(aux["lse"].cpu().numpy(), L, "sparse_prefill")


ARRANGE = [("c2_gqa_bf16", {}), ("c3_long_fp8", {}), ("c1_tiny", {}),
           ("small", dict(nq=200, k=6, kv_len=2048, hq=8, hkv=2)),
           ("small", dict(nq=77, k=5, kv_len=2048, hq=8, hkv=2, window=30, max_group=6)),
           ("small", dict(nq=150, k=8, kv_len=2048, hq=16, hkv=2))]      # G = 8: no-op


@pytest.mark.parametrize("name,kw", ARRANGE, ids=[f"{n}-{i}" for i, (n, _) in enumerate(ARRANGE)])
def test_tile_arrangement(name, kw):
    """pw_arrange_groups: groups and member masks bit for bit against the oracle's
    arrangement, and the attention output identical, bit for bit, to the unarranged run."""
    cfg = CONFIGS[name] if name != "small" else _small(**kw)
    print(f"[parity] tile arrangement {name} {kw}", flush=True)
    w = make_workload(cfg)
    res, _ = run_gpu(w, arrange=True)
    ref = oracle_tables(w, arrange=True)
    _compare_tables(res, ref)
    base, _ = run_gpu(w)
    assert np.array_equal(res["out"], base["out"]) and np.array_equal(res["lse"], base["lse"])


def _scale_rows_bf16(bits, factors):
    """bf16 bit patterns scaled elementwise by powers of two (exact: no overflow or
    subnormal results for the exponents used here)."""
    x = (bits.astype(np.uint32) << 16).view(np.float32) * factors.astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (16, 2)])
def test_fp8_query_dynamic_range(hq, hkv):
    """fp8 KV: query rows of very different magnitudes and rows whose elements span a wide
    range (zero rows, rows scaled by 2^-40 .. 2^2, elements scaled by up to 2^-20, one
    dominant element) against the definition."""
    cfg = _small(kv_dtype="fp8", hq=hq, hkv=hkv, nq=96, k=8, kv_len=2048, seed=77)
    w = make_workload(cfg)
    rng = np.random.default_rng(5)
    nq, d = cfg.nq, cfg.d
    f = np.ones((nq, hq, d), dtype=np.float64)
    row_exp = rng.choice([-40, -12, -3, 0, 1, 2], size=(nq, hq))
    f *= np.exp2(row_exp)[:, :, None]
    wide = rng.random((nq, hq)) < 0.3                       # elements spread over 2^-20 .. 1
    f[wide] *= np.exp2(-rng.integers(0, 21, size=(int(wide.sum()), d)))
    q = _scale_rows_bf16(w.q, f)
    q[rng.random((nq, hq)) < 0.05] = 0                      # zero rows
    spike = rng.random((nq, hq)) < 0.05                     # one dominant element
    q[spike] = _scale_rows_bf16(q[spike], np.full((int(spike.sum()), d), 2.0 ** -16))
    q[spike, 0] = 0x4100                                    # bf16 8.0
    w.q = q
    res, _ = run_gpu(w)
    ref = oracle_tables(w)
    _compare_tables(res, ref)
    O, L = oracle_attention(w, ref["S"])
    mx, mean, _ = check_close(res["out"], O, "fp8", f"dynamic range hq={hq}")
    check_lse(res["lse"], L, f"dynamic range hq={hq}")
    print(f"[parity] fp8 dynamic range hq={hq}: max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)


@pytest.mark.parametrize("n", [1, 7, 8, 9, 100, 513, 4096, 8192, 8200, 65536, 65537, 65600])
def test_work_order_matches_oracle(n):
    """pw_schedule_items against the oracle's work order on synthetic union sizes: ranges
    of <= 1024 items (one key per thread), longer ones (keys in LDS), at 65600 items
    ranges of 8200 > 8192 that keep item order, and at 65537 seven such ranges of 8193
    beside a last one of 8186 that is sorted."""
    rng = np.random.default_rng(n)
    sizes = rng.integers(0, 130, size=n).astype(np.int64)
    sizes[rng.random(n) < 0.2] = 64                       # many ties
    off = np.zeros(n + 1, dtype=np.int32)
    off[1:] = np.cumsum(sizes)
    order = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    pw.pw_schedule_items(torch.from_numpy(off).cuda(), order)
    assert np.array_equal(order.cpu().numpy(), np.array(prep.work_order(sizes.tolist()), dtype=np.int32))


@pytest.mark.parametrize("n", [100, 3000])
def test_work_order_large_unions(n):
    """Unions of 2^19 pages and more (past the one-key-per-thread form's size field) are
    still ordered by their exact sizes."""
    rng = np.random.default_rng(n + 1)
    sizes = rng.integers(0, 1 << 21, size=n).astype(np.int64) if n <= 100 else \
        np.where(rng.random(n) < 0.01, rng.integers(1 << 19, 1 << 20, size=n), rng.integers(0, 600, size=n))
    sizes[:3] = [(1 << 19) + 5, (1 << 19) - 1, (1 << 19) + 5]   # ties across the boundary
    off = np.zeros(n + 1, dtype=np.int64)
    off[1:] = np.cumsum(sizes)
    assert off[-1] < 2**31
    order = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    pw.pw_schedule_items(torch.from_numpy(off.astype(np.int32)).cuda(), order)
    assert np.array_equal(order.cpu().numpy(), np.array(prep.work_order(sizes.tolist()), dtype=np.int32))


@pytest.mark.parametrize("nq,max_group", [(9, 8), (700, 1), (9000, 1), (65537, 1), (66000, 1)])
def test_prepare_work_order(nq, max_group):
    """pw_prepare's work order (listed in the union listing's launch) equals pw_schedule_items
    on the same tables and the oracle's: ranges of <= 1024 tables, longer ones (keys in
    LDS), at 66000 tables ranges of 8250 > 8192 that keep item order, and at 65537 a last
    range of 8186 that is sorted beside seven of 8193 that are not."""
    rng = np.random.default_rng(nq)
    n_pages, k, window = 64, 3, 64
    print(f"[parity] prepare work order nq={nq} max_group={max_group}", flush=True)
    topk = torch.from_numpy(rng.integers(-1, n_pages, size=(nq, 1, k)).astype(np.int32)).cuda()
    G = pw.pw_num_groups(nq, window, max_group)
    cap = pw.pw_union_capacity(G, max_group, k, n_pages)
    i32 = dict(dtype=torch.int32, device="cuda")
    bits = torch.empty((1, nq, pw.pw_words(n_pages)), dtype=torch.int64, device="cuda")
    qids, size = torch.empty((1, G, max_group), **i32), torch.empty((1, G), **i32)
    off, pages = torch.empty(G + 1, **i32), torch.empty(cap, **i32)
    qmask = torch.empty(cap, dtype=torch.uint8, device="cuda")
    order = torch.full((G,), -7, **i32)
    pw.pw_prepare(topk, n_pages, window, max_group, bits, qids, size, off, pages, qmask,
                  item_order=order)
    order2 = torch.full((G,), -7, **i32)
    pw.pw_schedule_items(off, order2)
    torch.cuda.synchronize()
    sizes = np.diff(off.cpu().numpy().astype(np.int64))
    assert np.array_equal(order.cpu().numpy(), order2.cpu().numpy())
    assert np.array_equal(order.cpu().numpy(), np.array(prep.work_order(sizes.tolist()), dtype=np.int32))


@pytest.mark.parametrize("name", ["c2_gqa_bf16", "c3_long_fp8"])
def test_work_order_changes_no_output_bit(name):
    cfg = CONFIGS[name]
    w = make_workload(cfg)
    d = device_inputs(w)
    outs = []
    for schedule in (False, True):
        plan = pw.SparsePrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                                page_size=cfg.ps, kv_len=cfg.kv_len, k=w.topk.shape[2],
                                window=cfg.window, max_group=cfg.max_group, schedule=schedule)
        out = torch.full_like(d["q"], float("nan"))
        lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        plan(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], out, d["k_scale"], d["v_scale"], lse)
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu(), lse.cpu()))
        if schedule:
            sizes = np.diff(plan.union_off.cpu().numpy().astype(np.int64))
            assert np.array_equal(plan.item_order.cpu().numpy(), np.array(prep.work_order(sizes.tolist())))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
