"""GPU: the boundary's contracts beyond the workload parity.

* original-order groups listed and run by the library from their ranks alone;
* grouping invariance with random groups passed in as member lists;
* the dense case (every query selects every page) against a library attention;
* masked slots are exact no-ops for finite cache contents: junk in the slots past
  the cache end and in pages that only other members selected changes no bit of the
  rows that do not use them;
* more than 64 query heads per KV head through the two entry points that merge
  partial rows by lse.
"""
import math

import numpy as np
import pytest
import torch

import query_union_kv_amd as pw
from gpu_util import check_close, check_lse, device_inputs, oracle_attention, run_gpu
from oracle import attention, prep
from workloads import make_workload
from workloads.configs import Config

pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(name="contract", hq=8, hkv=2, d=128, ps=64, kv_len=4096, nq=150, kv_dtype="bf16",
                support="community", k=6, n_comm=6, comm_size=10, forced=True, window=64,
                max_group=8, seed=61)
    base.update(kw)
    return Config(**base)


def _attend(w, d, group_qids, group_size, n_groups, max_group, off, pages, qmask):
    c = w.cfg
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pw.pw_sparse_prefill(d["q"], d["k"], d["v"], d["q_pos"], c.kv_len, off, pages, out, hkv=c.hkv,
                         n_groups=n_groups, max_group=max_group, group_qids=group_qids,
                         group_size=group_size, union_qmask=qmask, k_scale=d["k_scale"],
                         v_scale=d["v_scale"], lse=lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_original_order_groups_listed_by_the_library(kv_dtype):
    """grouping='original': pw_union_tables with no member lists (consecutive groups) gives
    the oracle's tables of the original-order groups, and pw_sparse_prefill with no member
    lists runs them; the output equals the affinity run's bit for bit."""
    cfg = _small(kv_dtype=kv_dtype, nq=203)
    print(f"[contract] original-order groups {kv_dtype}", flush=True)
    w = make_workload(cfg)
    res, plan = run_gpu(w, grouping="original")
    assert plan.group_qids is None and plan.group_size is None
    bits = prep.page_bitsets(w.topk, cfg.n_pages)
    groups = [prep.group_original(cfg.nq, cfg.max_group) for _ in bits]
    off, pages, qmask = prep.union_tables(bits, groups)
    assert np.array_equal(res["union_off"], off)
    assert np.array_equal(res["union_pages"], pages)
    assert np.array_equal(res["union_qmask"], qmask)
    aff, _ = run_gpu(w)
    assert np.array_equal(res["out"], aff["out"]) and np.array_equal(res["lse"], aff["lse"])
    O, L = oracle_attention(w, prep.supports(w.topk, cfg.n_pages))
    check_close(res["out"], O, kv_dtype, "original")
    check_lse(res["lse"], L, "original")


@pytest.mark.parametrize("kv_dtype,max_group", [("bf16", 8), ("fp8", 5), ("bf16", 3)])
def test_random_grouping_invariance(kv_dtype, max_group):
    """Random groups (a seeded permutation cut into groups, the last one short) through
    pw_union_tables and pw_sparse_prefill: the same output bits as the affinity grouping,
    and within tolerance of the oracle."""
    cfg = _small(kv_dtype=kv_dtype, nq=131)
    print(f"[contract] random grouping {kv_dtype} max_group={max_group}", flush=True)
    w = make_workload(cfg)
    d = device_inputs(w)
    rng = np.random.default_rng(max_group)
    n_groups = -(-cfg.nq // max_group)
    qids = np.full((cfg.hkv, n_groups, max_group), -1, dtype=np.int32)
    size = np.zeros((cfg.hkv, n_groups), dtype=np.int32)
    groups = []
    for g in range(cfg.hkv):
        perm = rng.permutation(cfg.nq)
        gg = [list(perm[j:j + max_group]) for j in range(0, cfg.nq, max_group)]
        groups.append(gg)
        for j, m in enumerate(gg):
            qids[g, j, :len(m)] = m
            size[g, j] = len(m)
    i32 = dict(dtype=torch.int32, device="cuda")
    bits = torch.empty((cfg.hkv, cfg.nq, pw.pw_words(cfg.n_pages)), dtype=torch.int64, device="cuda")
    pw.pw_page_bitsets(d["ids"], cfg.n_pages, bits)
    cap = pw.pw_union_capacity(cfg.hkv * n_groups, max_group, cfg.k, cfg.n_pages)
    off, pages = torch.empty(cfg.hkv * n_groups + 1, **i32), torch.empty(cap, **i32)
    qmask = torch.empty(cap, dtype=torch.uint8, device="cuda")
    qids_t, size_t = torch.from_numpy(qids).cuda(), torch.from_numpy(size).cuda()
    pw.pw_union_tables(bits, cfg.n_pages, qids_t, size_t, cfg.k, off, pages, qmask)
    torch.cuda.synchronize()
    ref_off, ref_pages, ref_qmask = prep.union_tables(prep.page_bitsets(w.topk, cfg.n_pages), groups)
    n = int(ref_off[-1])
    assert np.array_equal(off.cpu().numpy(), ref_off)
    assert np.array_equal(pages[:n].cpu().numpy(), ref_pages)
    assert np.array_equal(qmask[:n].cpu().numpy(), ref_qmask)
    out, lse = _attend(w, d, qids_t, size_t, n_groups, max_group, off, pages, qmask)
    aff, _ = run_gpu(w)
    assert np.array_equal(out, aff["out"]) and np.array_equal(lse, aff["lse"])
    O, L = oracle_attention(w, prep.supports(w.topk, cfg.n_pages))
    check_close(out, O, kv_dtype, "random groups")
    check_lse(lse, L, "random groups")


@pytest.mark.parametrize("kv_dtype,d", [("bf16", 128), ("bf16", 64), ("fp8", 128)])
def test_dense_supports_against_library_attention(kv_dtype, d):
    """TopK = every page: the union path is dense causal attention, compared with torch's
    scaled_dot_product_attention in fp32 on the CPU over the decoded cache."""
    cfg = _small(kv_dtype=kv_dtype, d=d, kv_len=1000, nq=70, support="uniform", k=16, forced=False)
    print(f"[contract] dense vs SDPA {kv_dtype} d={d}", flush=True)
    w = make_workload(cfg)
    w.topk = np.broadcast_to(np.arange(cfg.n_pages, dtype=np.int32), (cfg.nq, cfg.hkv, cfg.n_pages)).copy()
    res, _ = run_gpu(w)
    from oracle import numerics
    G = cfg.hq // cfg.hkv
    q = torch.from_numpy(numerics.bf16_bits_to_f64(w.q)).float().permute(1, 0, 2)[None]
    k = numerics.decode_kv(w.k, w.k_scale, kv_dtype).reshape(cfg.hkv, -1, d)[:, :cfg.kv_len]
    v = numerics.decode_kv(w.v, w.v_scale, kv_dtype).reshape(cfg.hkv, -1, d)[:, :cfg.kv_len]
    k = torch.from_numpy(k).float().repeat_interleave(G, dim=0)[None].contiguous()
    v = torch.from_numpy(v).float().repeat_interleave(G, dim=0)[None].contiguous()
    mask = torch.arange(cfg.kv_len)[None, :] <= torch.from_numpy(w.q_pos.astype(np.int64))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=1.0 / math.sqrt(d))
    ref = ref[0].permute(1, 0, 2).double().numpy()
    check_close(res["out"], ref, kv_dtype, "dense vs SDPA")


def _junk_like(a, kv_dtype, rng):
    """Finite junk of large magnitude: bf16 +-1e4, or the largest e4m3fn codes +-448."""
    if kv_dtype == "bf16":
        return np.where(rng.random(a.shape) < 0.5, np.uint16(0x461C), np.uint16(0xC61C))   # +-9984
    return np.where(rng.random(a.shape) < 0.5, np.uint8(0x7E), np.uint8(0xFE)).astype(np.uint8)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_masked_slots_are_exact_noops(kv_dtype):
    """Finite junk in the slots past the cache end, and in pages that exactly one query of
    a KV head selected, leaves every row that does not use those slots bit for bit as it
    was (masked keys pass through the MFMAs with probability 0), and the rows match the
    oracle on the modified cache."""
    # uniform supports over 125 pages: a few pages are selected by one query only; the last
    # page holds 54 of its 64 slots
    cfg = _small(kv_dtype=kv_dtype, kv_len=7990, nq=96, k=6, support="uniform")
    print(f"[contract] masked slots are no-ops {kv_dtype}", flush=True)
    w = make_workload(cfg)
    base, _ = run_gpu(w)
    rng = np.random.default_rng(7)
    tail = cfg.kv_len - (cfg.n_pages - 1) * cfg.ps
    w.k[:, -1, tail:] = _junk_like(w.k[:, -1, tail:], kv_dtype, rng)
    w.v[:, -1, tail:] = _junk_like(w.v[:, -1, tail:], kv_dtype, rng)
    S = prep.supports(w.topk, cfg.n_pages)
    touched = np.zeros((cfg.nq, cfg.hkv), dtype=bool)
    n_single = 0
    for g in range(cfg.hkv):
        count = np.zeros(cfg.n_pages, dtype=np.int64)
        for s in S[g]:
            count[list(s)] += 1
        single = [p for p in range(cfg.n_pages - 1) if count[p] == 1]
        n_single += len(single)
        for p in single:
            w.k[g, p] = _junk_like(w.k[g, p], kv_dtype, rng)
            w.v[g, p] = _junk_like(w.v[g, p], kv_dtype, rng)
        for i in range(cfg.nq):
            touched[i, g] = any(p in S[g][i] for p in single)
    assert n_single > 0 and (~touched).any()
    junk, _ = run_gpu(w)
    G = cfg.hq // cfg.hkv
    keep = np.repeat(~touched, G, axis=1)                              # [nq, hq] rows not using junk pages
    assert np.array_equal(junk["out"][keep], base["out"][keep])
    assert np.array_equal(junk["lse"][keep], base["lse"][keep])
    O, L = oracle_attention(w, S)
    check_close(junk["out"][keep], O[keep], kv_dtype, "rows beside junk")
    check_lse(junk["lse"][keep], L[keep], "rows beside junk")


def _wide_cfg(**kw):
    base = dict(name="wide", hq=128, hkv=1, d=128, ps=64, kv_len=2048, nq=37, kv_dtype="bf16",
                support="uniform", k=5, forced=True, seed=71)
    base.update(kw)
    return Config(**base)


@pytest.mark.parametrize("kv_dtype,chunk", [("bf16", 2), ("fp8", 1)])
def test_page_union_more_than_64_heads_per_kv_head(kv_dtype, chunk):
    """128 query heads on one KV head: the direct KV-page union's merge gives every head its
    lse weights (the lanes of the merge wave loop over head columns)."""
    cfg = _wide_cfg(kv_dtype=kv_dtype)
    print(f"[contract] page union G=128 {kv_dtype} chunk={chunk}", flush=True)
    w = make_workload(cfg)
    d = device_inputs(w)
    plan = pw.PageUnionPrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                               page_size=cfg.ps, kv_len=cfg.kv_len, k=cfg.k, chunk=chunk)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    plan(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], out, d["k_scale"], d["v_scale"], lse)
    torch.cuda.synchronize()
    O, L = oracle_attention(w, prep.supports(w.topk, cfg.n_pages))
    check_close(out.float().cpu().numpy(), O, kv_dtype, "page union G=128")
    check_lse(lse.cpu().numpy(), L, "page union G=128")


@pytest.mark.parametrize("n_split", [2, 3])
def test_shared_table_more_than_64_heads_per_kv_head(n_split):
    """128 query heads on one KV head over a shared table cut into slices: the slices'
    partial rows are merged for every head."""
    cfg = _wide_cfg()
    print(f"[contract] shared table G=128 n_split={n_split}", flush=True)
    w = make_workload(cfg)
    d = device_inputs(w)
    tables = prep.block_tables(w.topk, cfg.n_pages)              # one union over every row
    off = torch.tensor([0, len(tables[0])], dtype=torch.int32, device="cuda")
    pages = torch.tensor(tables[0], dtype=torch.int32, device="cuda")
    max_group = 2
    rows = cfg.nq * cfg.hq * n_split
    part_o = torch.empty((rows, cfg.d), dtype=torch.bfloat16, device="cuda")
    part_lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    pw.pw_shared_table_prefill(d["q"], d["k"], d["v"], d["q_pos"], cfg.kv_len, off, pages, out,
                               hkv=cfg.hkv, max_group=max_group, n_split=n_split, partial_o=part_o,
                               partial_lse=part_lse, lse=lse)
    torch.cuda.synchronize()
    O, L = oracle_attention(w, attention.shared_supports(tables, cfg.nq))
    check_close(out.float().cpu().numpy(), O, "bf16", f"shared table G=128 n_split={n_split}")
    check_lse(lse.cpu().numpy(), L, f"shared table G=128 n_split={n_split}")
