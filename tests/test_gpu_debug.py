"""GPU: the debug build (libpw_debug.so, -DPW_DEBUG).  Its kernels count index and
LDS-ring invariant violations instead of trapping.  On valid inputs it counts none and
gives the release build's bits; on a table damaged from the host (a page ID past the
cache, an offset past the capacity) it counts them, and the kernels still clamp and skip
as the release build does."""
import numpy as np
import pytest
import torch

import query_union_kv_amd as pw
from gpu_util import device_inputs, make_plan
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_lib():
    release = pw.LIB_PATH
    pw.use_library(pw.DEBUG_LIB_PATH)
    assert pw.pw_debug_violations() >= 0          # a debug build; clears the counters
    yield
    pw.use_library(release)


def _run(w, halves=False):
    d = device_inputs(w)
    plan = make_plan(w, halves=halves)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    plan(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], out, d["k_scale"], d["v_scale"], lse)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu(), lse.cpu(), plan, d


CASES = [("c3_long_fp8", {}, False), ("c2_gqa_bf16", dict(nq=512, kv_len=4096 + 512), False),
         ("c4_block_union", dict(nq=256, kv_len=16384), False),
         ("c5_adversarial", dict(nq=512, kv_len=8192), True), ("c1_tiny", {}, False)]


@pytest.mark.parametrize("name,kw,halves", CASES, ids=[c[0] for c in CASES])
def test_debug_build_counts_nothing_and_matches_release(name, kw, halves):
    cfg = CONFIGS[name].scaled(**kw) if kw else CONFIGS[name]
    print(f"[debug] {name} {kw}", flush=True)
    w = make_workload(cfg)
    ref_out, ref_lse, _, _ = _run(w, halves)
    release = pw.LIB_PATH
    pw.use_library(pw.DEBUG_LIB_PATH)
    try:
        assert pw.pw_debug_violations() >= 0
        out, lse, _, _ = _run(w, halves)
        n = pw.pw_debug_violations()
    finally:
        pw.use_library(release)
    assert n == 0, f"{n} invariant violations"
    assert torch.equal(out, ref_out) and torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))


def test_debug_build_counts_a_damaged_table(debug_lib):
    """A union table entry past the cache (the kernel reads no such page: it skips the
    entry) and a prefix sum past the capacity (clamped) are counted."""
    cfg = CONFIGS["c2_gqa_bf16"].scaled(nq=256, kv_len=2048 + 256)
    w = make_workload(cfg)
    _, _, plan, d = _run(w)
    assert pw.pw_debug_violations() == 0
    plan.union_pages[3] = cfg.n_pages + 7                       # a page ID past the cache
    out = torch.empty_like(d["q"])
    plan.attend(d["q"], d["k"], d["v"], d["q_pos"], out)
    torch.cuda.synchronize()
    assert pw.pw_debug_violations() > 0
    plan.prepare(d["ids"])                                       # a clean table again
    cap = plan.union_pages.numel()
    plan.union_off[-1] = cap + 100                               # the last table past the capacity
    plan.attend(d["q"], d["k"], d["v"], d["q_pos"], out)
    torch.cuda.synchronize()
    assert pw.pw_debug_violations() > 0
    assert np.isfinite(out.float().cpu().numpy()).all()
