"""Sparse-prefill benchmark: queries/s and unique-KV HBM GB/s on one MI355X.

One step = one complete sparse-prefill call on one chunk of synthetic input:
page bitsets -> affinity grouping -> union tables -> union attention.  The
default workload is the long-context fp8 case (64K context, 4096-query chunk,
Hq=32, Hkv=8, d=128, 64-token pages, Top16 per (query, KV head), OCP e4m3 KV
with per-page fp32 scales).  Inputs are resident in HBM before timing starts.

Warm-up: the W calls of ``--warmup``, then untimed calls until the warm-up has
lasted ``--settle-ms`` of wall time (1 s); the timed calls' HIP events are created
and recorded during it.  After the GPU has been idle the time of a call moves over
the first ~30 ms of steady work (a C3 call: about 0.42 ms, settling at 0.34 ms from
the ~100th call on), so a count of calls alone leaves short warm-ups inside that
transient; and the first timing events of the first process on a fresh box slowed
the calls around them.  The K calls right after the W warm-up calls are timed as
well and reported as ``extra.warmup.right_after_warmup``.

Prints one JSON line.  ``roofline`` refers to the attention kernel (the
dominant one, timed live with HIP events on its own stream) as a hierarchical
roofline: each level's traffic or work over that level's peak - L2 (the
algorithmic bytes through it against a measured L2-resident read of the same
load path), HBM (calibrated FETCH/WRITE counters), MFMA (MOPS counters against
the dense peaks) and VALU (issue cycles) - and ``bound`` names the level with
the largest fraction.  The counters come from the committed rocprofv3 summary
of the same kernel source (profiles/).  ``cpu_baseline`` times the CPU oracle
(route A, every row of the chunk, on the host's cores), and ``extra.accuracy``
compares the timed output with it.
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
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="after the --warmup calls, more untimed calls until the warm-up has lasted this "
                         "long (wall time): after idle the per-call time moves for about 30 ms of steady "
                         "work before it settles; the K calls right after the W warm-up calls are timed "
                         "too and reported as extra.right_after_warmup")
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


def item_members(group_qids, n_tables: int, max_group: int, nq: int) -> np.ndarray:
    """Member query IDs of every work item, int64 [n_tables, max_group], -1 padded: the
    listed groups, or consecutive groups of max_group IDs per KV head when group_qids is
    None (the original-order groups)."""
    if group_qids is not None:
        return np.asarray(group_qids, dtype=np.int64).reshape(n_tables, max_group)
    n_groups_g = -(-nq // max_group)
    j = np.arange(n_tables) % n_groups_g
    ids = j[:, None] * max_group + np.arange(max_group)[None, :]
    return np.where(ids < nq, ids, -1)


def union_table_stats(union_off, union_qmask, members) -> dict:
    """Page visits and member x page slots of query-union tables (PageWeaver Fig. 2 and
    Fig. 6 counts): visits = sum |U|, slots = sum |g| |U|, selected = member-mask bits set,
    masked = slots - selected."""
    sizes = np.diff(np.asarray(union_off, dtype=np.int64))
    gsz = (np.asarray(members) >= 0).sum(axis=1)
    qm = np.asarray(union_qmask[:int(sizes.sum())], dtype=np.uint8)
    selected = int(np.unpackbits(qm[:, None], axis=1).sum())
    slots = int((sizes * gsz).sum())
    return {"visits": int(sizes.sum()), "slots": slots, "selected": selected,
            "masked": slots - selected, "masked_frac": (slots - selected) / slots if slots else 0.0}


def row_tile_work(union_off, union_pages, union_qmask, members, q_pos, G: int, ps: int,
                  kv_len: int, shared_table: bool = False, n_split: int = 1) -> dict:
    """The attention's unit of MFMA work is a row tile (16 query-head rows: 16 / G members)
    against a 32-token tile of a union page.  It runs when some member of the row tile
    selected the page (member-mask bit) and the tile starts at or before the row tile's
    last usable token; otherwise it is skipped.  Counts both, from the tables alone.
    members: [n_items, max_group] query IDs (-1 padded); shared_table: every item of KV
    head g reads table g (then no member masks)."""
    members = np.asarray(members, dtype=np.int64)
    n_items, max_group = members.shape
    off = np.asarray(union_off, dtype=np.int64)
    rows = max_group * G
    n_rt = -(-rows // 16)
    # member bits of each row tile, and its last usable token (-1: no valid row)
    qp = np.asarray(q_pos, dtype=np.int64)
    lim_m = np.where(members >= 0, np.minimum(qp[np.maximum(members, 0)], kv_len - 1), -1)
    rt_bits = np.zeros(n_rt, dtype=np.int64)
    rt_lim = np.full((n_items, n_rt), -1, dtype=np.int64)
    for t in range(n_rt):
        ms = sorted({r // G for r in range(16 * t, min(16 * (t + 1), rows))})
        for m in ms:
            rt_bits[t] |= 1 << m
        rt_lim[:, t] = lim_m[:, ms].max(axis=1)
    n_tables = len(off) - 1
    active = total = 0
    sub = ps // 32
    for it in range(n_items):
        e = (it // (n_items // n_tables)) if shared_table else it
        pages = np.asarray(union_pages[off[e]:off[e + 1]], dtype=np.int64)
        if pages.size == 0:
            continue
        qm = (np.full(pages.size, 0xFF, dtype=np.int64) if union_qmask is None
              else np.asarray(union_qmask[off[e]:off[e + 1]], dtype=np.int64))
        tok0 = pages[:, None] * ps + 32 * np.arange(sub)[None, :]                 # [P, sub]
        for t in range(n_rt):
            if rt_lim[it, t] < 0:
                continue
            sel = (qm & (rt_bits[t] if union_qmask is not None else 0xFF)) != 0
            act = sel[:, None] & (tok0 <= rt_lim[it, t])
            active += int(act.sum())
            total += tok0.size
    return {"active_pairs": active, "pairs": total, "row_tiles": n_rt}


def unique_kv_bytes(union_pages_total: int, cfg) -> int:
    esz = 1 if cfg.kv_dtype == "fp8" else 2
    per_page = 2 * cfg.ps * cfg.d * esz + (8 if cfg.kv_dtype == "fp8" else 0)
    return union_pages_total * per_page


def host_cores() -> int:
    """Cores this process may run on, at most 16 (a one-GPU share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def blas_vendor() -> str:
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                if i.get("user_api") == "blas"]
        return ", ".join(libs) or "unknown"
    except Exception:          # the report only; never fails the run
        return "unknown"


def cpu_baseline(w, n_queries: int, cores: int) -> tuple:
    """The oracle as it stands on the first n_queries queries (whole windows): pure-Python
    bitsets, grouping and union tables, then route A (the definition) for every row with
    its KV heads and query batches spread over `cores` threads.  Returns the record and the
    route A output (fp64 [n, hq, d]) for the accuracy check."""
    from oracle import attention, prep
    cfg = w.cfg
    nqs = min(cfg.nq, max(cfg.window, (n_queries // cfg.window) * cfg.window))
    t0 = time.perf_counter()
    if w.topk is not None:
        topk = w.topk[:nqs]
        bits = prep.page_bitsets(topk, cfg.n_pages)
        groups = [prep.group_affinity(b, cfg.window, cfg.max_group) for b in bits]
        prep.union_tables(bits, groups)
        S = prep.supports(topk, cfg.n_pages)
    else:   # block union: the per-KV-group tables, every query over its group's table
        S = attention.shared_supports(prep.block_tables(w.mask_rows, cfg.n_pages), nqs)
    t1 = time.perf_counter()
    O, _ = attention.route_a_batched(w.q[:nqs], w.k, w.v, w.k_scale, w.v_scale, cfg.kv_dtype, S,
                                     w.q_pos[:nqs], cfg.kv_len, cfg.ps, 1.0 / math.sqrt(cfg.d),
                                     workers=cores)
    t2 = time.perf_counter()
    rec = {"value": nqs / (t2 - t0), "unit": "queries/s", "cores": min(cores, cfg.hkv * -(-nqs // 64)),
           "kind": "oracle",
           "sample": f"first {nqs} of {cfg.nq} queries ({nqs // cfg.window} windows of {cfg.window}), "
                     f"all {cfg.hkv} KV heads; prep {t1 - t0:.2f}s (pure Python, one thread) + "
                     f"attention {t2 - t1:.2f}s (numpy fp64 route A, {cores} threads)",
           "cpu": _cpu_model(), "blas": blas_vendor(), "prep_s": t1 - t0, "attention_s": t2 - t1}
    return rec, O


def accuracy(out_bf16, ref) -> dict:
    """max-abs, mean-abs and NRMS (PageWeaver Table 2: ||O - R|| / ||R|| over the whole
    output, in percent) of the GPU output against the oracle's rows."""
    got = out_bf16.astype(np.float64)
    err = np.abs(got - ref)
    den = float(np.sqrt((ref ** 2).sum()))
    return {"rows": int(ref.shape[0] * ref.shape[1]), "elements": int(ref.size),
            "max_abs": float(err.max()), "mean_abs": float(err.mean()),
            "nrms_pct": 100.0 * float(np.sqrt((err ** 2).sum())) / den if den else 0.0,
            "finite": bool(np.isfinite(got).all())}


MFMA_PEAK_FLOPS = {"bf16": 2.5e15, "fp8": 5.0e15}   # dense, per the MI355X specification
FLOPS_PER_MOP = 512                                   # SQ_INSTS_VALU_MFMA_MOPS_* unit


def attn_source_hash() -> str:
    import hashlib
    src = os.path.join(ROOT, "query_union_kv_amd", "csrc", "attn.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def profiled_counters(workload: str):
    """Per-launch counters of the attention kernel from the committed rocprofv3 summary
    profiles/k_attn_<workload>.md (a line `counters_per_launch = {json}  (attn.hip
    sha256[:16] H)`), or None when the summary is missing or the kernel source has changed
    since the counters were taken.  Keys: fetch_bytes and write_bytes (FETCH_SIZE and
    WRITE_SIZE scaled by a plain-copy calibration), mops_bf16 / mops_f8 (MFMA work, 512
    flops each), valu_busy (SQ_ACTIVE_INST_VALU x 4 cycles per SIMD over the kernel's
    cycles), l2_hit (TCC_HIT / (TCC_HIT + TCC_MISS)), mean_us (kernel trace)."""
    import re
    summ = os.path.join(ROOT, "profiles", f"k_attn_{workload}.md")
    if not os.path.exists(summ):
        return None
    h = attn_source_hash()
    for line in open(summ):
        m = re.match(r"counters_per_launch = (\{.*\})\s+\(attn.hip sha256\[:16\] (\w+)\)", line.strip())
        if m and m.group(2) == h:
            return json.loads(m.group(1))
    return None


def read_peaks(dev, reps: int = 5) -> dict:
    """Measured read rates of plain streaming-read kernels (libpw_probe.so) by the level
    that serves them, in GB/s (best of `reps` launches): `vec` = vector loads, `lds` =
    direct global->LDS loads (the attention's load path).  Working sets: 2 MiB (every XCD
    re-reads it from its L2), 128 MiB (re-read from the 256 MB last-level cache once
    warm: each XCD's share, 16 MiB, exceeds its 4 MB L2), 4 GiB (HBM)."""
    import ctypes

    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "query_union_kv_amd", "libpw_probe.so"))
    L.pwp_read.restype = ctypes.c_int
    L.pwp_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                           ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    out = {}
    for name, nbytes, seg, n_blocks in (("l2", 2 << 20, 64 << 10, 16384),
                                        ("mall", 128 << 20, 64 << 10, 8192),
                                        ("hbm", 4 << 30, 1 << 20, 4096)):
        buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        out[name] = {"buffer_bytes": nbytes, "bytes_per_launch": seg * n_blocks}
        for mode, key in ((0, "vec"), (1, "lds")):
            best = None
            for r in range(reps + 1):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                st = L.pwp_read(buf.data_ptr(), nbytes, seg, n_blocks, mode, sink.data_ptr(),
                                stream.cuda_stream)
                e1.record(stream)
                if st != 0:
                    raise RuntimeError(f"pwp_read failed: {st}")
                torch.cuda.synchronize()
                if r:   # the first launch warms the caches
                    t = e0.elapsed_time(e1)
                    best = t if best is None else min(best, t)
            out[name][key + "_GBs"] = seg * n_blocks / (best / 1e3) / 1e9
        del buf
    return out


def roofline_levels(Bu: float, qo_bytes: float, t_attn_s: float, ctr, peaks) -> dict:
    """The attention kernel against each resource that could bound it (a hierarchical
    roofline: each level's traffic over that level's peak).
      l2:      the algorithmic bytes that pass through the L2 - every group's union tiles once
               (B_u) plus the Q rows read and the output rows written - over the kernel time,
               against the measured read rate of a plain streaming read of an L2-resident
               buffer through the same direct-to-LDS load path (cross-checked against the
               counter-measured L2 requests, TCC_REQ x 128 B);
      hbm:     counter-measured bytes between the L2 and memory (FETCH_SIZE + WRITE_SIZE,
               calibrated) against 8 TB/s;
      mfma:    counter-measured MFMA work (MOPS) as the time the matrix cores need at their
               dense peaks (bf16 2.5, fp8 5.0 PFLOP/s) over the kernel time;
      valu:    counter-measured vector-ALU issue cycles over the kernel's SIMD cycles;
      simd:    vector-ALU issue cycles plus MFMA busy cycles over the SIMD cycles: the two
               pipes as one wave's dependent chain uses them (QK on MFMA -> softmax on the
               VALU -> PV on MFMA), which two waves per SIMD overlap only in part (an MFMA's
               issue cycle is counted in both terms: at most 0.05 on these kernels).
    The counter fractions are taken over the profiled launches and rescaled to the live kernel
    time (same cycles of work in the live duration).
    Not bounds (reported for reference): `logical` = the union bytes B_u over the kernel
    time against the 8 TB/s HBM peak (re-reads of pages other groups also read come from
    the L2, so this exceeds 1), and `llc` = B_u against the measured read rate of a buffer
    resident in the 256 MB last-level cache (also exceeded: most of B_u is served by L2)."""
    ach = Bu / t_attn_s / 1e9
    lv = {"logical": {"achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                      "bound": False, "what": "union bytes B_u / kernel time vs HBM peak (not a bound)"}}
    if peaks:
        p_llc = peaks["mall"]["lds_GBs"]
        lv["llc"] = {"achieved": ach, "peak": p_llc, "unit": "GB/s", "frac": ach / p_llc, "bound": False,
                     "what": "B_u / kernel time vs a measured last-level-cache-resident read (not a bound: L2 "
                             "serves most of B_u)"}
    if peaks:
        l2b = Bu + qo_bytes
        p_l2 = peaks["l2"]["lds_GBs"]
        lv["l2"] = {"achieved": l2b / t_attn_s / 1e9, "peak": p_l2, "unit": "GB/s",
                    "frac": l2b / t_attn_s / 1e9 / p_l2, "bytes_per_launch": l2b,
                    "what": "(B_u + Q + O bytes) per launch / kernel time vs the measured L2-resident read "
                            "rate of the direct-to-LDS load path"}
        if ctr and ctr.get("l2_requests"):
            lv["l2"]["counter_bytes_per_launch"] = ctr["l2_requests"] * 128.0
            lv["l2"]["l2_hit"] = ctr.get("l2_hit")
    if ctr:
        hb = ctr["fetch_bytes"] + ctr["write_bytes"]
        lv["hbm"] = {"achieved": hb / t_attn_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": hb / t_attn_s / 1e9 / HBM_PEAK_GBS, "bytes_per_launch": hb,
                     "what": "FETCH_SIZE + WRITE_SIZE (calibrated) per launch / kernel time"}
        fb, f8 = ctr["mops_bf16"] * FLOPS_PER_MOP, ctr["mops_f8"] * FLOPS_PER_MOP
        t_peak = fb / MFMA_PEAK_FLOPS["bf16"] + f8 / MFMA_PEAK_FLOPS["fp8"]
        lv["mfma"] = {"achieved": (fb + f8) / t_attn_s / 1e12,
                      "peak": (fb + f8) / t_peak / 1e12 if t_peak else MFMA_PEAK_FLOPS["bf16"] / 1e12,
                      "unit": "TFLOP/s", "frac": t_peak / t_attn_s, "flops_per_launch": fb + f8,
                      "flops_bf16": fb, "flops_fp8": f8,
                      "what": "MFMA MOPS x 512 per launch; peak = the dtype-weighted dense peak"}
        scale = ctr["mean_us"] / (t_attn_s * 1e6) if ctr.get("mean_us") else 1.0
        if ctr.get("valu_busy") is not None:
            v = ctr["valu_busy"] * scale
            lv["valu"] = {"achieved": v, "peak": 1.0, "unit": "fraction of SIMD cycles", "frac": v,
                          "what": "vector-ALU issue cycles / SIMD cycles (counters)"}
            if ctr.get("mfma_busy") is not None:
                sm = (ctr["valu_busy"] + ctr["mfma_busy"]) * scale
                lv["simd"] = {"achieved": sm, "peak": 1.0, "unit": "fraction of SIMD cycles", "frac": sm,
                              "what": "(vector-ALU issue + MFMA busy cycles) / SIMD cycles (counters)"}
    return lv


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

    # The timed calls' HIP events are created and recorded during the warm-up: the first
    # timing events of a process on a freshly leased GPU slowed the calls around them (one
    # C3 call 0.34 -> 0.40 ms with the events first used in the timed region, in the first
    # process on a box only); recorded once before, they cost nothing measurable.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_warm = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the same K calls timed right after the W warm-up calls (with few warm-up calls the GPU is
    # still leaving its idle state), then untimed calls until the warm-up has lasted settle_ms
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    settle_calls = 0
    while (time.perf_counter() - t_warm) * 1e3 < args.settle_ms or settle_calls < args.steps:
        for _ in range(10):
            step(evs[settle_calls % args.steps])   # (the same events as the timed calls)
            settle_calls += 1
        torch.cuda.synchronize()
    warm_wall_ms = (time.perf_counter() - t_warm) * 1e3

    # ---- the timed region: K complete steps back to back -------------------------------
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    t_enq = time.perf_counter() - t0          # host time to enqueue the K calls
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    out_final = out.float().cpu().numpy()       # the timed calls' output (every call writes the same)
    t_prep = [evs[i][0].elapsed_time(evs[i][1]) for i in range(args.steps)]
    t_attn = [evs[i][1].elapsed_time(evs[i][2]) for i in range(args.steps)]
    ms_step = wall * 1e3 / args.steps
    value = cfg.nq / (ms_step / 1e3)
    settle = {"host_enqueue_ms_per_step": t_enq * 1e3 / args.steps, "warmup_calls": args.warmup, "right_after_warmup_calls": args.steps,
              "settle_calls": settle_calls, "untimed_wall_ms": warm_wall_ms, "settle_ms": args.settle_ms,
              "right_after_warmup": {"ms_per_step": first_ms, "queries_per_s": cfg.nq / (first_ms / 1e3)}}

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
              "unique_kv_bytes": Bu, "warmup": settle}
    n_items = len(off) - 1 if mode == "topk" else cfg.hkv * plan.n_groups
    halves = mode == "topk" and plan.halves
    members = item_members((plan.half_qids if halves else plan.group_qids).cpu().numpy()
                           if plan.group_qids is not None else None,
                           n_items, plan.width if halves else max_group, cfg.nq)
    pages_np = plan.union_pages[:total_pages].cpu().numpy()
    qm_np = plan.union_qmask[:total_pages].cpu().numpy() if plan.union_qmask is not None else None
    work = row_tile_work(off, pages_np, qm_np, members, w.q_pos, cfg.g, cfg.ps, cfg.kv_len,
                         shared_table=(mode != "topk"))
    if mode == "topk":
        st = union_table_stats(off, qm_np, members)
        selected, slots = st["selected"], st["slots"]                  # retained edges, member x page slots
        orig = pw.SparsePrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                                page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], window=cfg.window,
                                max_group=cfg.max_group, grouping="original", device=dev)
        orig.prepare(ids)
        torch.cuda.synchronize()
        orig_pages = int(orig.union_off[-1].item())
        per_q = cfg.nq * cfg.hkv
        group_pages = total_pages          # pages of the affinity groups' unions
        if halves:                         # (the timed tables are the halves' unions)
            whole = pw.SparsePrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                                     page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], window=cfg.window,
                                     max_group=cfg.max_group, halves=False, device=dev)
            whole.prepare(ids)
            torch.cuda.synchronize()
            group_pages = int(whole.union_off[-1].item())
            w_off = whole.union_off.cpu().numpy()
            st_group = union_table_stats(
                w_off, whole.union_qmask[:group_pages].cpu().numpy(),
                item_members(whole.group_qids.cpu().numpy(), len(w_off) - 1, cfg.max_group, cfg.nq))
            del whole
        else:
            st_group = st
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
            "bytes": {"B_u": unique_kv_bytes(group_pages, cfg), "B_streamed": Bu,
                      "B_query": selected * page_bytes, "B_orig": orig_pages * page_bytes,
                      "B_distinct": int(len(np.unique(np.nonzero(keep)[1] * cfg.n_pages + uniq[keep]))) * page_bytes},
            "visits_per_query_kvh": {"per_query": selected / per_q, "original_union": orig_pages / per_q,
                                     "affinity_union": group_pages / per_q,
                                     "streamed": total_pages / per_q},
            "execution": "two halves per group, each over its own union" if halves else "whole groups",
            "masked_slot_frac": st_group["masked_frac"],
            "masked_slot_frac_streamed": (slots - selected) / slots if slots else 0.0,
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

        # Wide groups (more than 32 query-head rows) run as two halves by default, each half
        # over the union of its own members' pages; the whole-group execution (the two-wave
        # form over the group's union) is timed beside it: the same outputs bit for bit.
        if plan.halves:
            wh = pw.SparsePrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                                  page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], window=cfg.window,
                                  max_group=cfg.max_group, halves=False, device=dev)
            out_wh = torch.empty_like(q)
            t_wh_prep = timed(lambda: wh.prepare(ids, stream))
            for _ in range(30):   # (a form not run so far: settle it before timing)
                wh.attend(q, kc, vc, q_pos, out_wh, ks, vs, stream=stream)
            t_wh_attn = timed(lambda: wh.attend(q, kc, vc, q_pos, out_wh, ks, vs, stream=stream), n=30)
            torch.cuda.synchronize()
            wh_pages = int(wh.union_off[-1].item())
            extras["whole_groups"] = {
                "prep_ms": t_wh_prep, "attn_ms": t_wh_attn, "call_ms": t_wh_prep + t_wh_attn,
                "queries_per_s": cfg.nq / ((t_wh_prep + t_wh_attn) / 1e3),
                "union_pages": wh_pages, "union_pages_halves": total_pages,
                "union_bytes": unique_kv_bytes(wh_pages, cfg),
                "attn_ms_halves": t_fixed,
                "bit_identical": bool(torch.equal(out_wh.view(torch.int16), out.view(torch.int16)))}
            del wh, out_wh

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
        # CompactAttention's shared per-KV-group tables: the timed form cuts each table into
        # plan.n_split slices (partial rows merged by lse); the same attention with no
        # partials at all (one workgroup streams a whole table) is timed beside it
        one = pw.SparsePrefill(nq=cfg.nq, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, n_pages=cfg.n_pages,
                               page_size=cfg.ps, kv_len=cfg.kv_len, k=ids.shape[2], max_group=max_group,
                               mode=mode, n_rows=ids.shape[0], n_split=1, device=dev)
        one.prepare(ids, stream)
        out_one = torch.empty_like(q)
        for _ in range(20):
            one.attend(q, kc, vc, q_pos, out_one, ks, vs, stream=stream)
        t_one = timed(lambda: one.attend(q, kc, vc, q_pos, out_one, ks, vs, stream=stream), n=20)
        extras["shared_table"] = {
            "timed_form": f"table cut into {plan.n_split} slices, partial rows merged by lse"
                          if plan.n_split > 1 else "one workgroup per table slice: no partials",
            "n_split": plan.n_split, "attn_ms": attn_ms,
            "no_partials": {"n_split": 1, "attn_ms": t_one, "call_ms": statistics.mean(t_prep) + t_one,
                            "queries_per_s": cfg.nq / ((statistics.mean(t_prep) + t_one) / 1e3),
                            "max_abs_vs_timed": float((out_one.float() - out.float()).abs().max().item())}}
        del one, out_one
    # executed MFMA work: QK and PV over every row tile x 32-token tile the kernel runs (the
    # tables' member masks and causal limits decide which); skipped pairs are not counted.
    # (fp8 K at d = 128 runs QK as two fp8 MFMAs, hi and lo parts of Q: the counters count both)
    exec_flops = 2 * 2.0 * 16 * 32 * cfg.d * work["active_pairs"]
    extras["executed_mfma"] = {"row_tile_key_tile_pairs": work["active_pairs"],
                               "pairs_in_tables": work["pairs"],
                               "skipped": work["pairs"] - work["active_pairs"],
                               "flops_per_launch": exec_flops,
                               "tflops": exec_flops / (attn_ms / 1e3) / 1e12}
    if mode == "topk":
        extras["executed_mfma"]["executed_over_useful"] = exec_flops / useful_flops
    extras["attn_queries_per_s"] = cfg.nq / (attn_ms / 1e3)

    # ---- the complete call captured once in a HIP graph and replayed, against eager calls
    # (PageWeaver times graph replays beside eager rounds: Table 1, Fig. 8) -----------------
    out_g = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.prepare(ids)
        plan.attend(q, kc, vc, q_pos, out_g, ks, vs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.prepare(ids)
        plan.attend(q, kc, vc, q_pos, out_g, ks, vs)
    for _ in range(20):
        graph.replay()
    t_graph = timed(graph.replay, n=50)
    t_eager = timed(step, n=50)
    torch.cuda.synchronize()
    extras["hip_graph"] = {"graph_call_ms": t_graph, "eager_call_ms": t_eager,
                           "queries_per_s_graph": cfg.nq / (t_graph / 1e3),
                           "bit_identical": bool(torch.equal(out_g.view(torch.int16), out.view(torch.int16))),
                           "what": "bitsets, grouping, union tables and attention as one graph, 50 replays"}
    del graph, out_g

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

    # ---- measured read rates of each memory level, and the roofline levels -------------------
    peaks = read_peaks(dev)
    extras["read_peaks_GBs"] = peaks
    ctr = profiled_counters(cfg.name)
    qo_bytes = 2.0 * cfg.nq * cfg.hq * cfg.d * 2                    # Q read and O written, bf16
    levels = roofline_levels(Bu, qo_bytes, attn_ms / 1e3, ctr, peaks)
    bounds = {k: v for k, v in levels.items() if v.get("bound", True)}
    bound = max(bounds, key=lambda k: bounds[k]["frac"]) if bounds else "logical"
    top = levels[bound]
    if ctr:
        levels["counters"] = {"source": f"profiles/k_attn_{cfg.name}.md", "attn_sha16": attn_source_hash(),
                              "profiled_mean_us": ctr.get("mean_us"),
                              "frac_at_profiled_time": {k: v["frac"] * attn_ms * 1e3 / ctr["mean_us"]
                                                        for k, v in bounds.items() if ctr.get("mean_us")}}
    else:
        levels["counters"] = {"source": None, "note": "no counters for this kernel source: the hbm, mfma "
                                                      "and valu levels are unknown"}

    # arithmetic of the attention's MFMAs: fp8 KV with d = 128 takes QK on the fp8 MFMA
    dtype = "fp8/bf16" if cfg.kv_dtype == "fp8" and cfg.d == 128 else "bf16"
    rec = {
        "metric": METRIC, "value": value, "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "hq": cfg.hq, "hkv": cfg.hkv, "d": cfg.d, "page_size": cfg.ps,
                   "kv_len": cfg.kv_len, "nq": cfg.nq, "topk": cfg.k, "kv_dtype": cfg.kv_dtype,
                   "window": cfg.window, "max_group": max_group, "seed": w.seed,
                   "attention": ("query unions with member masks (pw_sparse_prefill)" if mode == "topk" else
                                 f"shared per-KV-group tables, {plan.n_split} slices per table merged by lse"
                                 if plan.n_split > 1 else "shared per-KV-group tables, no partials")},
        "roofline": {"bound": bound, "achieved": top["achieved"], "peak": top["peak"], "unit": top["unit"],
                     "frac": top["frac"],
                     "traffic": (ctr["fetch_bytes"] + ctr["write_bytes"]) if ctr else None,
                     "kernel": "k_attn", "kernel_ms": attn_ms, "union_bytes_per_launch": Bu,
                     "levels": levels},
        "extra": extras,
    }
    if not args.no_cpu:
        cpu, ref = cpu_baseline(w, args.cpu_queries, host_cores())
        rec["cpu_baseline"] = cpu
        n = ref.shape[0]
        acc = accuracy(out_final[:n], ref)
        tol = (2e-2, 2e-3) if cfg.kv_dtype == "bf16" else (6e-2, None)
        acc["within_tolerance"] = bool(acc["finite"] and acc["max_abs"] <= tol[0]
                                       and (tol[1] is None or acc["mean_abs"] <= tol[1]))
        acc["tolerance"] = {"max_abs": tol[0], "mean_abs": tol[1]}
        acc["oracle"] = "route A (per-query gather, fp64), every row of the sample"
        extras["accuracy"] = acc
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
