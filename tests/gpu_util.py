"""Shared pieces of the GPU parity tests: moving a workload to the device, running
the HIP path through the C ABI, and the oracle's view of the same call."""
import math
import os

import numpy as np
import torch

import query_union_kv_amd as pw
from oracle import attention, prep

TOL = {"bf16": dict(max_abs=2e-2, mean_abs=2e-3), "fp8": dict(max_abs=6e-2, mean_abs=None)}


def device_inputs(w, dev="cuda"):
    c = w.cfg
    d = {}
    d["q"] = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if c.kv_dtype == "bf16":
        d["k"] = torch.from_numpy(w.k.view(np.int16)).view(torch.bfloat16).to(dev)
        d["v"] = torch.from_numpy(w.v.view(np.int16)).view(torch.bfloat16).to(dev)
        d["k_scale"] = d["v_scale"] = None
    else:
        d["k"] = torch.from_numpy(w.k).to(dev)
        d["v"] = torch.from_numpy(w.v).to(dev)
        d["k_scale"] = torch.from_numpy(w.k_scale).to(dev)
        d["v_scale"] = torch.from_numpy(w.v_scale).to(dev)
    d["q_pos"] = torch.from_numpy(np.ascontiguousarray(w.q_pos, dtype=np.int32)).to(dev)
    ids = w.topk if w.topk is not None else w.mask_rows
    d["ids"] = torch.from_numpy(np.ascontiguousarray(ids)).to(dev)
    return d


def make_plan(w, grouping="affinity", window=None, max_group=None, dev="cuda", fused=True, arrange=False,
              halves=False):
    c = w.cfg
    ids = w.topk if w.topk is not None else w.mask_rows
    mode = "topk" if w.topk is not None else "block_union"
    if mode == "block_union" and max_group is None:
        max_group = max(1, c.item_rows // c.g)
    return pw.SparsePrefill(nq=c.nq, hq=c.hq, hkv=c.hkv, d=c.d, n_pages=c.n_pages, page_size=c.ps,
                            kv_len=c.kv_len, k=ids.shape[2], window=window or c.window,
                            max_group=max_group or c.max_group, mode=mode, grouping=grouping,
                            n_rows=ids.shape[0] if mode == "block_union" else 0, fused=fused,
                            arrange=arrange, halves=halves if mode == "topk" else False, device=dev)


def run_gpu(w, grouping="affinity", window=None, max_group=None, with_lse=True, fused=True,
            arrange=False, halves=False):
    d = device_inputs(w)
    plan = make_plan(w, grouping, window, max_group, fused=fused, arrange=arrange, halves=halves)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    plan(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], out, d["k_scale"], d["v_scale"], lse)
    torch.cuda.synchronize()
    res = {"out": out.float().cpu().numpy(), "bits": plan.bits.cpu().numpy().view(np.uint64),
           "union_off": plan.union_off.cpu().numpy(), "bad_ids": int(plan.bad_ids.item())}
    total = int(res["union_off"][-1])
    res["union_pages"] = plan.union_pages[:total].cpu().numpy()
    if plan.union_qmask is not None:
        res["union_qmask"] = plan.union_qmask[:total].cpu().numpy()
    if plan.group_qids is not None:
        res["group_qids"] = plan.group_qids.cpu().numpy()
        res["group_size"] = plan.group_size.cpu().numpy()
    if getattr(plan, "item_order", None) is not None:
        res["item_order"] = plan.item_order.cpu().numpy()
    if with_lse:
        res["lse"] = lse.cpu().numpy()
    return res, plan


def oracle_tables(w, grouping="affinity", window=None, max_group=None, arrange=False):
    """Bitsets, groups and union tables exactly as the oracle defines them (optionally with
    the members of every group arranged for 4-member row tiles when hq/hkv = 4)."""
    c = w.cfg
    window = window or c.window
    max_group = max_group or c.max_group
    if w.topk is not None:
        bits = prep.page_bitsets(w.topk, c.n_pages)
        if grouping == "affinity":
            groups = [prep.group_affinity(b, window, max_group) for b in bits]
        else:
            groups = [prep.group_original(c.nq, max_group) for _ in bits]
        if arrange and c.g == 4:
            groups = [[prep.arrange_for_tiles(b, m, 4) for m in grp] for b, grp in zip(bits, groups)]
        qids, size = prep.groups_to_arrays(groups, max_group)
        off, pages, qmask = prep.union_tables(bits, groups)
        return {"bits": prep.bits_to_words(bits, c.n_pages), "group_qids": qids, "group_size": size,
                "union_off": off, "union_pages": pages, "union_qmask": qmask, "groups": groups,
                "S": prep.supports(w.topk, c.n_pages), "stats": prep.union_stats(bits, groups)}
    bits = prep.page_bitsets(w.mask_rows, c.n_pages)
    n_rows = w.mask_rows.shape[0]
    off, pages, _ = prep.union_tables(bits, [[list(range(n_rows))] for _ in bits], with_qmask=False)
    tables = prep.block_tables(w.mask_rows, c.n_pages)
    return {"bits": prep.bits_to_words(bits, c.n_pages), "union_off": off, "union_pages": pages,
            "tables": tables, "S": attention.shared_supports(tables, c.nq)}


def oracle_workers() -> int:
    """Threads for the oracle: the cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_attention(w, S, queries=None):
    """Route A (the definition) for every row, or for ``queries``; batched over queries
    and threaded over KV heads so that whole chunks take seconds."""
    c = w.cfg
    return attention.route_a_batched(w.q, w.k, w.v, w.k_scale, w.v_scale, c.kv_dtype, S, w.q_pos,
                                     c.kv_len, c.ps, 1.0 / math.sqrt(c.d), queries,
                                     workers=oracle_workers())


def check_close(got, ref, kv_dtype, what=""):
    err = np.abs(got.astype(np.float64) - ref)
    tol = TOL[kv_dtype]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err.max() <= tol["max_abs"], f"{what}: max_abs {err.max():.4g} > {tol['max_abs']}"
    if tol["mean_abs"] is not None:
        assert err.mean() <= tol["mean_abs"], f"{what}: mean_abs {err.mean():.4g} > {tol['mean_abs']}"
    return float(err.max()), float(err.mean()), attention.nrms(got, ref)


# lse is not given a tolerance by the task; this one follows from the arithmetic: the
# kernel's row sum adds the bf16-rounded probabilities that its PV products use (each within
# 2^-9 relative), so ln(l) may be off by ln(1 + 2^-9) = 1.95e-3, on top of the fp32 score
# error (and, for fp8 K, the split of each query row into two e4m3 parts)
LSE_TOL = 4e-3


def check_lse(got, ref, what=""):
    fin = np.isfinite(ref)
    assert (np.isneginf(got) == ~fin).all(), f"{what}: lse -inf pattern differs"
    assert np.abs(got[fin] - ref[fin]).max(initial=0) <= LSE_TOL, f"{what}: lse differs"
