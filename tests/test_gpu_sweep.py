"""Seeded random shapes through the whole union path, against the oracle.

Each case draws head counts (G = 1, 2, 4, 8 query heads per KV head), d, the KV type,
page size, context length, chunk size, TopK, grouping window and group size, optional
padding / duplicate / out-of-range IDs and the half-group execution, then checks the
groups, union tables (of the groups, or of their halves) and work order bit for bit and the
attention output and lse within the tolerances."""
import random

import numpy as np
import pytest
import torch

from gpu_util import check_close, check_lse, device_inputs, make_plan, oracle_attention, oracle_tables
from helpers import add_padding_and_duplicates
from oracle import prep
from workloads import make_workload
from workloads.configs import Config

N_CASES = 60
N_LONG = 20   # contexts up to 140K tokens (past 1024 pages: the unfused preparation), windows up to 256


def _case(i, long=False):
    rng = random.Random((5000 if long else 1000) + i)
    d = rng.choice([64, 128])
    kvd = rng.choice(["bf16", "fp8"])
    hkv = rng.choice([1, 2, 3])
    G = rng.choice([1, 2, 4, 8])
    mg = rng.choice([1, 2, 3, 4, 5, 6, 7, 8])
    while G * mg > 64:
        mg -= 1
    ps = rng.choice([64, 128])
    kv_len = rng.choice([70000, 140000] if long else [ps, 2 * ps + 5, 1000, 3000, 5000])
    nq = rng.randint(1, min(kv_len, 300))
    k = rng.randint(1, min(24, -(-kv_len // ps) + 2))
    window = mg * rng.randint(1, max(1, (256 if long else 64) // mg))
    halves = mg % 2 == 0 and rng.random() < 0.3
    cfg = Config(name=f"sweep{i}", hq=hkv * G, hkv=hkv, d=d, ps=ps, kv_len=kv_len, nq=nq, kv_dtype=kvd,
                 support="uniform", k=k, forced=rng.random() < 0.5, window=window, max_group=mg,
                 seed=rng.randint(1, 10**6))
    return cfg, halves, rng.random() < 0.5


@pytest.mark.gpu
@pytest.mark.parametrize("i,long", [(i, False) for i in range(N_CASES)] + [(i, True) for i in range(N_LONG)])
def test_random_shape(i, long):
    cfg, halves, pad = _case(i, long)
    print(f"[sweep] case {i}: {cfg} halves={halves} pad={pad}", flush=True)
    w = make_workload(cfg)
    if pad:
        w.topk = add_padding_and_duplicates(w.topk, seed=cfg.seed + 1)
    d = device_inputs(w)
    base = make_plan(w)
    fields = ("nq", "hq", "hkv", "d", "n_pages", "page_size", "kv_len", "k", "window", "max_group", "mode",
              "grouping", "n_rows", "fused")
    plan = type(base)(**{**{f: getattr(base, f) for f in fields}, "halves": halves})
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    plan(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], out, d["k_scale"], d["v_scale"], lse)
    torch.cuda.synchronize()
    ref = oracle_tables(w)
    assert np.array_equal(plan.group_qids.cpu().numpy(), ref["group_qids"])
    assert np.array_equal(plan.group_size.cpu().numpy(), ref["group_size"])
    if halves:   # the tables of each group's two member halves, in pick order
        h = cfg.max_group // 2
        halves_per_head = [[x for m in grp for x in (m[:h], m[h:])] for grp in ref["groups"]]
        r_off, r_pages, r_qmask = prep.union_tables(prep.page_bitsets(w.topk, cfg.n_pages), halves_per_head)
    else:
        r_off, r_pages, r_qmask = ref["union_off"], ref["union_pages"], ref["union_qmask"]
    n = int(plan.union_off[-1])
    assert np.array_equal(plan.union_off.cpu().numpy(), r_off)
    assert np.array_equal(plan.union_pages[:n].cpu().numpy(), r_pages)
    assert np.array_equal(plan.union_qmask[:n].cpu().numpy(), r_qmask)
    sizes = np.diff(np.asarray(r_off, dtype=np.int64))
    assert np.array_equal(plan.item_order.cpu().numpy(), np.array(prep.work_order(sizes.tolist())))
    O, L = oracle_attention(w, ref["S"])
    check_close(out.float().cpu().numpy(), O, cfg.kv_dtype, f"case {i}")
    check_lse(lse.cpu().numpy(), L, f"case {i}")
