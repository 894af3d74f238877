"""bench.py's table statistics on the CPU: the page visits, member x page slots and
selected edges it reports from the union tables equal the oracle's union_stats
(PageWeaver Fig. 2 / Fig. 6 counts), and the row-tile work count follows its rule."""
import os
import sys

import numpy as np

from oracle import prep
from workloads import CONFIGS, make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _tables(cfg, grouping):
    w = make_workload(cfg)
    bits = prep.page_bitsets(w.topk, cfg.n_pages)
    if grouping == "affinity":
        groups = [prep.group_affinity(b, cfg.window, cfg.max_group) for b in bits]
        qids, _ = prep.groups_to_arrays(groups, cfg.max_group)
    else:
        groups = [prep.group_original(cfg.nq, cfg.max_group) for _ in bits]
        qids = None
    off, pages, qmask = prep.union_tables(bits, groups)
    return w, bits, groups, qids, off, pages, qmask


def test_stats_of_the_headline_tables_match_the_oracle():
    cfg = CONFIGS["c3_long_fp8"]
    for grouping in ("affinity", "original"):
        w, bits, groups, qids, off, pages, qmask = _tables(cfg, grouping)
        n_tables = len(off) - 1
        members = bench.item_members(qids, n_tables, cfg.max_group, cfg.nq)
        got = bench.union_table_stats(off, qmask, members)
        ref = prep.union_stats(bits, groups)
        for k in ("visits", "slots", "selected", "masked"):
            assert got[k] == ref[k], (grouping, k)
        assert abs(got["masked_frac"] - ref["masked_frac"]) < 1e-15


def test_stats_of_the_fig2_construction():
    """PageWeaver Fig. 2: original-order pairs visit 16 pages with 16 masked slots, the
    affinity pairs 8 pages with none, and all 16 selected edges are kept."""
    topk = np.array([[[0, 1]], [[2, 3]]] * 4, dtype=np.int32)          # even IDs -> {0,1}, odd -> {2,3}
    bits = prep.page_bitsets(topk, 4)
    for grouping, visits, masked in (("original", 16, 16), ("affinity", 8, 0)):
        groups = ([prep.group_affinity(b, 8, 2) for b in bits] if grouping == "affinity"
                  else [prep.group_original(8, 2) for _ in bits])
        off, _, qmask = prep.union_tables(bits, groups)
        qids = prep.groups_to_arrays(groups, 2)[0] if grouping == "affinity" else None
        st = bench.union_table_stats(off, qmask, bench.item_members(qids, len(off) - 1, 2, 8))
        assert (st["visits"], st["masked"], st["selected"]) == (visits, masked, 16)


def test_row_tile_work_rule():
    """Two members of G = 8 rows each (one 16-row tile); pages 0 and 1 of 64 tokens (two
    32-token tiles each).  Member 0 selected page 0, nobody page 1 (mask 0): page 0 runs
    its tiles at or before the tile's last usable token, page 1 is skipped."""
    off = np.array([0, 2])
    pages = np.array([0, 1])
    qmask = np.array([0b01, 0b00], dtype=np.uint8)
    members = np.array([[0, 1]])
    q_pos = np.array([40, 10])                                          # last usable: 40 (tile 0..31, 32..63)
    r = bench.row_tile_work(off, pages, qmask, members, q_pos, G=8, ps=64, kv_len=1000)
    assert r == {"active_pairs": 2, "pairs": 4, "row_tiles": 1}
    q_pos = np.array([20, 10])                                          # only the first tile
    assert bench.row_tile_work(off, pages, qmask, members, q_pos, 8, 64, 1000)["active_pairs"] == 1
    # no member masks (a shared table): every tile of every page at or before the limit
    r = bench.row_tile_work(off, pages, None, members, np.array([90, 10]), 8, 64, 1000,
                            shared_table=True)
    assert r["active_pairs"] == 3                                       # the tile at token 96 > 90 is skipped


def test_roofline_levels_follow_the_committed_counters():
    """With the live kernel time equal to the profiled mean, every counter level reproduces the
    per-launch figures of the committed summary: bytes / mean duration / peak, and the busy
    fractions as measured; at twice the time every fraction halves."""
    ctr = bench.profiled_counters("c3_long_fp8")
    if ctr is None:   # the summary was taken with another attention source
        import pytest
        pytest.skip("profiles/k_attn_c3_long_fp8.md does not match the attention source")
    peaks = {"l2": {"lds_GBs": 29000.0}, "mall": {"lds_GBs": 7000.0}}
    t = ctr["mean_us"] * 1e-6
    Bu, qo = 6.0e9, 1.0e8
    lv = bench.roofline_levels(Bu, qo, t, ctr, peaks)
    hb = ctr["fetch_bytes"] + ctr["write_bytes"]
    assert abs(lv["hbm"]["frac"] - hb / t / 8e12) < 1e-12
    assert abs(lv["l2"]["frac"] - (Bu + qo) / t / 29000e9) < 1e-12
    assert abs(lv["valu"]["frac"] - ctr["valu_busy"]) < 1e-12
    assert abs(lv["simd"]["frac"] - (ctr["valu_busy"] + ctr["mfma_busy"])) < 1e-12
    t_mfma = (ctr["mops_bf16"] * 512 / 2.5e15) + (ctr["mops_f8"] * 512 / 5.0e15)
    assert abs(lv["mfma"]["frac"] - t_mfma / t) < 1e-12
    assert lv["logical"]["bound"] is False and lv["llc"]["bound"] is False
    lv2 = bench.roofline_levels(Bu, qo, 2 * t, ctr, peaks)
    for k in ("hbm", "l2", "valu", "simd", "mfma"):
        assert abs(lv2[k]["frac"] - lv[k]["frac"] / 2) < 1e-12, k
