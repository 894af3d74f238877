"""Sparse-prefill benchmark: queries/s and unique-KV HBM GB/s on one MI355X.

One step = one complete sparse-prefill call on one chunk of synthetic input:
page bitsets -> affinity grouping -> union tables -> union attention.  The
default workload is the long-context fp8 case (64K context, 4096-query chunk,
Hq=32, Hkv=8, d=128, 64-token pages, Top16 per (query, KV head), OCP e4m3 KV
with per-page fp32 scales).  Inputs are resident in HBM before timing starts.

Prints one JSON line.  ``roofline`` refers to the attention kernel (the
dominant one): achieved = unique-KV bytes (every group's union pages, K and V
plus their scales) / the kernel's mean duration from HIP events on its own
stream.  ``cpu_baseline`` times the CPU oracle on a bounded sample (the first
windows of the chunk), single-threaded.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "sparse-prefill queries/s + unique-KV HBM GB/s (% roofline), 64K ctx Top16 fp8"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the chip's clocks take some tens of milliseconds of steady work to settle: 200 untimed
    # calls of the 64K fp8 Top16 workload are about 80 ms
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c3_long_fp8")
    ap.add_argument("--window", type=int, default=None)
    ap.add_argument("--item-rows", type=int, default=None,
                    help="block-union workloads: query-head rows per work item over the shared table")
    ap.add_argument("--flush-steps", type=int, default=20,
                    help="replays per round, each timed after writing 512 MiB (L2/MALL flush)")
    ap.add_argument("--flush-rounds", type=int, default=7,
                    help="rounds of flushed replays (median of the round medians is reported)")
    ap.add_argument("--cpu-queries", type=int, default=4096,
                    help="oracle sample: the first N queries (whole windows), all KV heads")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--windows", default="256,512",
                    help="extra grouping windows measured beside the configured one (TopK workloads)")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the chunked-prefill leg (whole context in chunks of nq, overlap vs serial)")
    ap.add_argument("--profile-steps", type=int, default=None,
                    help="run only this many steps after warmup (for rocprofv3), no extras")
    ap.add_argument("--profile-path", choices=["union", "page"], default="union",
                    help="with --profile-steps: the query-union call (default) or the direct KV-page union")
    ap.add_argument("--calibrate-copy", type=int, default=None, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (counter calibration)")
    return ap.parse_args()


def calibrate_copy(mib: int) -> None:
    """A plain copy kernel of known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}))


def unique_kv_bytes(union_pages_total: int, cfg) -> int:
    esz = 1 if cfg.kv_dtype == "fp8" else 2
    per_page = 2 * cfg.ps * cfg.d * esz + (8 if cfg.kv_dtype == "fp8" else 0)
    return union_pages_total * per_page


def cpu_baseline(w, n_queries: int) -> dict:
    """The oracle as it stands on the first n_queries queries (whole windows), 1 thread."""
    from threadpoolctl import threadpool_limits

    from oracle import attention, prep
    cfg = w.cfg
    nqs = min(cfg.nq, max(cfg.window, (n_queries // cfg.window) * cfg.window))
    topk = w.topk[:nqs]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        bits = prep.page_bitsets(topk, cfg.n_pages)
        groups = [prep.group_affinity(b, cfg.window, cfg.max_group) for b in bits]
        prep.union_tables(bits, groups)
        t1 = time.perf_counter()
        S = prep.supports(topk, cfg.n_pages)
        attention.route_a(w.q[:nqs], w.k, w.v, w.k_scale, w.v_scale, cfg.kv_dtype, S, w.q_pos[:nqs],
                          cfg.kv_len, cfg.ps, 1.0 / math.sqrt(cfg.d))
        t2 = time.perf_counter()
    return {"value": nqs / (t2 - t0), "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"first {nqs} of {cfg.nq} queries ({nqs // cfg.window} windows of {cfg.window}), "
                      f"all {cfg.hkv} KV heads; prep {t1 - t0:.2f}s + attention {t2 - t1:.2f}s",
            "cpu": _cpu_model()}


def profiled_traffic(workload: str):
    """HBM-side bytes per attention launch from the committed rocprofv3 summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain-copy calibration), or None if the
    kernel source changed since the counters were taken."""
    import hashlib
    import re
    src = os.path.join(ROOT, "query_union_kv_amd", "csrc", "attn.hip")
    summ = os.path.join(ROOT, "profiles", f"k_attn_{workload}.md")
    if not os.path.exists(summ):
        return None
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    for line in open(summ):
        m = re.match(r"traffic_bytes_per_launch\[.*\] = ([0-9.eE+]+)\s+\(attn.hip sha256\[:16\] (\w+)\)", line)
        if m and m.group(2) == h:
            return float(m.group(1))
    return None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X with no sharding; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import query_union_kv_amd as pw
    from workloads import CONFIGS, make_workload

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    cfg = CONFIGS[args.workload]
    if args.window:
        cfg = cfg.scaled(window=args.window)
    if args.item_rows:
        cfg = cfg.scaled(item_rows=args.item_rows)
    w = make_workload(cfg)
    dev = torch.device("cuda:0")

    q = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if cfg.kv_dtype == "bf16":
        kc = torch.from_numpy(w.k.view(np.int16)).view(torch.bfloat16).to(dev)
        vc = torch.from_numpy(w.v.view(np.int16)).view(torch.bfloat16).to(dev)
        ks = vs = None
    else:
        kc, vc = torch.from_numpy(w.k).to(dev), torch.from_numpy(w.v).to(dev)
        ks, vs = torch.from_numpy(w.k_scale).to(dev), torch.from_numpy(w.v_scale).to(dev)
    q_pos = torch.from_numpy(w.q_pos).to(dev)
    ids_np = w.topk if w.topk is not None else w.mask_rows
    ids = torch.from_numpy(np.ascontiguousarray(ids_np)).to(dev)
    mode = "topk" if w.topk is not None else "block_union"
    max_group = cfg.max_group if mode == "topk" else max(1, cfg.item_rows // cfg.g)
    plan = pw.SparsePrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                            page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], window=cfg.window,
                            max_group=max_group, mode=mode,
                            n_rows=ids.shape[0] if mode == "block_union" else 0, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        plan.prepare(ids, stream)
        if evs:
            evs[1].record(stream)
        plan.attend(q, kc, vc, q_pos, out, ks, vs, stream=stream)
        if evs:
            evs[2].record(stream)

    if args.profile_steps is not None:
        run = step
        if args.profile_path == "page":
            pu = pw.PageUnionPrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                                     page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], device=dev)
            run = lambda: pu(ids, q, kc, vc, q_pos, out, ks, vs, stream=stream)   # noqa: E731
        for _ in range(args.warmup + args.profile_steps):
            run()
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "warmup": args.warmup, "workload": cfg.name,
                          "path": args.profile_path}))
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- the timed region: K complete steps back to back -------------------------------
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_prep = [evs[i][0].elapsed_time(evs[i][1]) for i in range(args.steps)]
    t_attn = [evs[i][1].elapsed_time(evs[i][2]) for i in range(args.steps)]
    ms_step = wall * 1e3 / args.steps
    value = cfg.nq / (ms_step / 1e3)

    def timed(fn, n=10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # ---- structure of this call's tables --------------------------------------------------
    off = plan.union_off.cpu().numpy()
    total_pages = int(off[-1])
    # page visits: every work item streams its table once (a shared per-KV-group table
    # is streamed by each of the KV head's groups)
    visits = total_pages if mode == "topk" else int(np.diff(off).sum()) * plan.n_groups
    Bu = unique_kv_bytes(visits, cfg)
    attn_ms = statistics.mean(t_attn)
    achieved = Bu / (attn_ms / 1e3) / 1e9
    extras = {"t_prep_ms_mean": statistics.mean(t_prep), "t_attn_ms_mean": attn_ms,
              "t_attn_ms_median": statistics.median(t_attn), "union_pages": total_pages,
              "page_visits": visits,
              "unique_kv_bytes": Bu}
    if mode == "topk":
        sizes = np.diff(off)
        gsz = plan.group_size.cpu().numpy().reshape(-1)
        qm = plan.union_qmask[:total_pages].cpu().numpy()
        selected = int(np.unpackbits(qm[:, None], axis=1).sum())      # retained selected edges
        slots = int((sizes * gsz).sum())                                # member x union-page slots
        orig = pw.SparsePrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                                page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], window=cfg.window,
                                max_group=cfg.max_group, grouping="original", device=dev)
        orig.prepare(ids)
        torch.cuda.synchronize()
        orig_pages = int(orig.union_off[-1].item())
        per_q = cfg.nq * cfg.hkv
        # useful work: keys each (query, head) row actually uses, |J| = sum over its support
        # pages of the tokens at or before its position and before the cache end
        tk = np.asarray(ids_np, dtype=np.int64)                            # [nq, hkv, K]
        valid = (tk >= 0) & (tk < cfg.n_pages)
        uniq = np.where(valid, tk, -1)
        uniq = np.sort(uniq, axis=2)
        first = np.concatenate([np.ones_like(uniq[:, :, :1], dtype=bool), uniq[:, :, 1:] != uniq[:, :, :-1]], axis=2)
        keep = first & (uniq >= 0)
        lim = np.minimum(w.q_pos.astype(np.int64)[:, None, None] + 1, cfg.kv_len)
        used = np.clip(lim - uniq * cfg.ps, 0, cfg.ps) * keep
        keys_used = int(used.sum()) * cfg.g                                # over all query heads
        useful_flops = 4.0 * cfg.d * keys_used
        page_bytes = cfg.ps * cfg.d * (1 if cfg.kv_dtype == "fp8" else 2) * 2 + (8 if cfg.kv_dtype == "fp8" else 0)
        extras.update({
            "useful_tflops": useful_flops / (attn_ms / 1e3) / 1e12,
            "bytes": {"B_u": Bu, "B_query": selected * page_bytes, "B_orig": orig_pages * page_bytes,
                      "B_distinct": int(len(np.unique(np.nonzero(keep)[1] * cfg.n_pages + uniq[keep]))) * page_bytes},
            "visits_per_query_kvh": {"per_query": selected / per_q, "original_union": orig_pages / per_q,
                                     "affinity_union": total_pages / per_q},
            "masked_slot_frac": (slots - selected) / slots if slots else 0.0,
            "selected_edges": selected,
        })

        # Fig. 6 / Eq. 7 decomposition: original-order Union call, attention over fixed
        # affinity tables, and the complete online affinity call.
        t_orig = timed(lambda: (orig.prepare(ids, stream),
                                orig.attend(q, kc, vc, q_pos, out, ks, vs, stream=stream)))
        t_orig_attn = timed(lambda: orig.attend(q, kc, vc, q_pos, out, ks, vs, stream=stream))
        t_fixed = timed(lambda: plan.attend(q, kc, vc, q_pos, out, ks, vs, stream=stream))
        t_online = timed(lambda: step())
        extras["fig6_ms"] = {"original_union_call": t_orig, "original_union_attention": t_orig_attn,
                             "fixed_affinity_attention": t_fixed, "online_affinity_call": t_online,
                             "execution_saving": t_orig_attn - t_fixed,
                             "online_cost": t_online - t_fixed, "net_saving": t_orig - t_online}
        exec_rows_pages = float((sizes * gsz).sum()) * cfg.g     # (row, union page) pairs

        # Grouping window sweep: a wider bounded search finds more same-community queries
        # (fewer page visits) but costs more preparation.
        sweep = {}
        for wn in [int(x) for x in args.windows.split(",") if x.strip()]:
            if wn == cfg.window or wn % cfg.max_group:
                continue
            pw_plan = pw.SparsePrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                                       page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], window=wn,
                                       max_group=cfg.max_group, device=dev)
            t_p = timed(lambda: pw_plan.prepare(ids, stream))
            t_a = timed(lambda: pw_plan.attend(q, kc, vc, q_pos, out, ks, vs, stream=stream))
            sweep[str(wn)] = {"visits_per_query_kvh": int(pw_plan.union_off[-1].item()) / per_q,
                              "prep_ms": t_p, "attn_ms": t_a}
            del pw_plan
        sweep[str(cfg.window)] = {"visits_per_query_kvh": total_pages / per_q,
                                  "prep_ms": statistics.mean(t_prep), "attn_ms": t_fixed}
        extras["window_sweep"] = sweep

        # Members arranged for 4-member row tiles (QUILT's cascaded sharing at row-tile
        # granularity): row tiles computed, from the member masks, and attention time.
        if cfg.g == 4 and cfg.max_group > 4:
            arr = pw.SparsePrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                                   page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], window=cfg.window,
                                   max_group=cfg.max_group, arrange=True, device=dev)
            t_arr_prep = timed(lambda: arr.prepare(ids, stream))
            t_arr_attn = timed(lambda: arr.attend(q, kc, vc, q_pos, out, ks, vs, stream=stream))

            def tiles_of(plan_):
                qm_ = plan_.union_qmask[:int(plan_.union_off[-1].item())].cpu().numpy()
                return int(((qm_ & 0x0F) != 0).sum() + ((qm_ & 0xF0) != 0).sum())
            extras["tile_arrangement"] = {
                "row_tiles_pick_order": tiles_of(plan), "row_tiles_arranged": tiles_of(arr),
                "prep_ms": t_arr_prep, "attn_ms": t_arr_attn, "attn_ms_pick_order": t_fixed}
            del arr

        # Wide groups (items of more than 32 rows, the two-wave form) run as two halves, each
        # over the union of its own members' pages: the same outputs bit for bit.
        if cfg.g * cfg.max_group > 32 and cfg.max_group % 2 == 0:
            hv = pw.SparsePrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                                  page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], window=cfg.window,
                                  max_group=cfg.max_group, halves=True, device=dev)
            out_hv = torch.empty_like(q)
            t_hv_prep = timed(lambda: hv.prepare(ids, stream))
            for _ in range(30):   # (a form not run so far: settle it before timing)
                hv.attend(q, kc, vc, q_pos, out_hv, ks, vs, stream=stream)
            t_hv_attn = timed(lambda: hv.attend(q, kc, vc, q_pos, out_hv, ks, vs, stream=stream), n=30)
            plan.attend(q, kc, vc, q_pos, out, ks, vs, stream=stream)   # whole groups, again
            torch.cuda.synchronize()
            extras["half_groups"] = {
                "prep_ms": t_hv_prep, "attn_ms": t_hv_attn, "call_ms": t_hv_prep + t_hv_attn,
                "queries_per_s": cfg.nq / ((t_hv_prep + t_hv_attn) / 1e3),
                "union_pages": int(hv.union_off[-1].item()), "union_pages_whole_groups": total_pages,
                "attn_ms_whole_groups": t_fixed,
                "bit_identical": bool(torch.equal(out_hv.view(torch.int16), out.view(torch.int16)))}
            del hv, out_hv

        # The direct KV-page union on the same inputs: every (KV head, page) once,
        # per-page partials, lse merge (a separate entry point, compared here).
        pu = pw.PageUnionPrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                                 page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], device=dev)
        out_pu = torch.empty_like(q)
        t_pu_prep = timed(lambda: pu.prepare(ids, stream))
        t_pu_attn = timed(lambda: pu.attend(q, kc, vc, q_pos, out_pu, ks, vs, stream=stream))
        t_pu_call = timed(lambda: pu(ids, q, kc, vc, q_pos, out_pu, ks, vs, stream=stream))
        n_items = pu.n_items
        distinct = int((np.diff(pu.item_off.cpu().numpy()) > 0).sum())  # (KV head, page) pairs used
        page_bytes = cfg.ps * cfg.d * (1 if cfg.kv_dtype == "fp8" else 2) * 2 + (8 if cfg.kv_dtype == "fp8" else 0)
        partial_bytes = 2 * selected * cfg.g * (cfg.d * 2 + 4)          # written, then read by the merge
        extras["direct_page_union"] = {
            "call_ms": t_pu_call, "prep_ms": t_pu_prep, "attn_and_merge_ms": t_pu_attn,
            "queries_per_s": cfg.nq / (t_pu_call / 1e3), "items": n_items, "chunk": pu.chunk,
            "distinct_kv_bytes": distinct * page_bytes, "partial_bytes": partial_bytes,
            "max_abs_vs_union": float((out_pu.float() - out.float()).abs().max().item())}
        del pu, out_pu
    else:
        exec_rows_pages = float(visits) * max_group * cfg.g      # item rows x its table pages
    # executed MFMA work: QK and PV, 2 flops per MAC, over every (row, union token)
    exec_flops = 4.0 * cfg.d * cfg.ps * exec_rows_pages
    extras["executed_tflops"] = exec_flops / (attn_ms / 1e3) / 1e12
    extras["attn_queries_per_s"] = cfg.nq / (attn_ms / 1e3)

    # ---- the step before attention: appending the chunk's own keys and values -------------
    # (into copies of the caches, so the attention inputs above stay as generated)
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    kn = torch.randn((cfg.nq, cfg.hkv, cfg.d), generator=gen, device=dev).to(torch.bfloat16)
    vn = torch.randn((cfg.nq, cfg.hkv, cfg.d), generator=gen, device=dev).to(torch.bfloat16)
    kc2, vc2 = kc.clone(), vc.clone()
    ks2, vs2 = (ks.clone(), vs.clone()) if ks is not None else (None, None)
    t_app = timed(lambda: pw.pw_append_kv(kn, vn, cfg.first_pos, kc2, vc2, ks2, vs2, stream=stream))
    esize = 1 if cfg.kv_dtype == "fp8" else 2
    n_app_pages = (cfg.kv_len - 1) // cfg.ps - cfg.first_pos // cfg.ps + 1
    app_bytes = 2 * cfg.nq * cfg.hkv * cfg.d * 2 + 2 * n_app_pages * cfg.hkv * cfg.ps * cfg.d * esize
    if esize == 1:
        app_bytes += 2 * n_app_pages * cfg.hkv * 4
    extras["append_kv"] = {"ms": t_app, "bytes": app_bytes, "GBs": app_bytes / (t_app / 1e3) / 1e9,
                           "hbm_frac": app_bytes / (t_app / 1e3) / 1e9 / HBM_PEAK_GBS}
    del kc2, vc2, ks2, vs2

    # ---- chunked prefill of the whole context: append -> prepare -> attend per chunk, the
    # next chunk's preparation overlapped on a second stream vs all on one stream ----------
    if mode == "topk" and not args.no_chunked and cfg.kv_len % cfg.nq == 0:
        from workloads import make_supports
        n_chunks = cfg.kv_len // cfg.nq
        runner = pw.ChunkedPrefill(hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages, page_size=cfg.ps,
                                   max_chunk=cfg.nq, k=cfg.k, window=cfg.window, max_group=cfg.max_group,
                                   device=dev)
        kc3, vc3 = kc.clone(), vc.clone()
        ks3, vs3 = (ks.clone(), vs.clone()) if ks is not None else (None, None)
        chunk_list = []
        for c in range(n_chunks):
            ccfg = cfg.scaled(kv_len=cfg.nq * (c + 1))
            qp, tk, _ = make_supports(ccfg, seed=cfg.seed * 1000 + c)
            chunk_list.append(dict(q=q, k_new=kn, v_new=vn, topk=torch.from_numpy(np.ascontiguousarray(tk)).to(dev),
                                   q_pos=torch.from_numpy(qp).to(dev), first_token=cfg.nq * c,
                                   out=torch.empty_like(q)))

        def chunked(overlap):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            runner.run(chunk_list, kc3, vc3, ks3, vs3, overlap=overlap, stream=stream)   # warm
            torch.cuda.synchronize()
            ts = []
            for _ in range(3):
                e0.record(stream)
                runner.run(chunk_list, kc3, vc3, ks3, vs3, overlap=overlap, stream=stream)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return statistics.median(ts)

        t_ser = chunked(False)
        t_ovl = chunked(True)
        extras["chunked_prefill"] = {
            "chunks": n_chunks, "chunk_queries": cfg.nq, "context": cfg.kv_len,
            "serial_ms": t_ser, "overlapped_ms": t_ovl, "saving_ms": t_ser - t_ovl,
            "queries_per_s_overlapped": cfg.kv_len / (t_ovl / 1e3)}
        del kc3, vc3, ks3, vs3, chunk_list, runner

    # ---- flushed timing: rounds of replays, 512 MiB written before each replay outside the
    # event pair; the median of the round medians and their range ---------------------------
    if args.flush_steps:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        rounds = []
        for _ in range(max(1, args.flush_rounds)):
            fl = []
            for _ in range(args.flush_steps):
                scratch.fill_(1)
                e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                step(e)
                torch.cuda.synchronize()
                fl.append((e[0].elapsed_time(e[2]), e[1].elapsed_time(e[2])))
            rounds.append((statistics.median(x[0] for x in fl), statistics.median(x[1] for x in fl)))
        del scratch
        f_call = statistics.median(r[0] for r in rounds)
        f_attn = statistics.median(r[1] for r in rounds)
        extras["flushed"] = {"rounds": len(rounds), "replays_per_round": args.flush_steps,
                             "ms_per_call_median": f_call, "ms_per_call_range": [min(r[0] for r in rounds),
                                                                                 max(r[0] for r in rounds)],
                             "attn_ms_median": f_attn, "attn_ms_range": [min(r[1] for r in rounds),
                                                                         max(r[1] for r in rounds)],
                             "queries_per_s": cfg.nq / (f_call / 1e3),
                             "unique_kv_GBs": Bu / (f_attn / 1e3) / 1e9}

    # ---- a measured copy peak beside the nominal 8 TB/s: 1 GiB device copy, best of 5 -------
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        best = t if best is None else min(best, t)
    del src, dst
    copy_gbs = 2 * (1 << 30) / (best / 1e3) / 1e9   # read + write bytes
    extras["copy_peak"] = {"GBs": copy_gbs, "unique_kv_frac_of_copy": achieved / copy_gbs,
                           "what": "1 GiB device-to-device copy, read + write bytes, best of 5"}

    # arithmetic of the attention's MFMAs: fp8 KV with d = 128 takes QK on the fp8 MFMA
    dtype = "fp8/bf16" if cfg.kv_dtype == "fp8" and cfg.d == 128 else "bf16"
    rec = {
        "metric": METRIC, "value": value, "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "hq": cfg.hq, "hkv": cfg.hkv, "d": cfg.d, "page_size": cfg.ps,
                   "kv_len": cfg.kv_len, "nq": cfg.nq, "topk": cfg.k, "kv_dtype": cfg.kv_dtype,
                   "window": cfg.window, "max_group": max_group, "seed": w.seed},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": profiled_traffic(cfg.name), "kernel": "k_attn",
                     "bytes_per_launch": Bu},
        "extra": extras,
    }
    if not args.no_cpu and mode == "topk":
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_queries)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
