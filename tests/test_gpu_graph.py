"""GPU: the complete call (bitsets, grouping, union tables, attention) captured once in a
HIP graph and replayed.  The library enqueues kernels only (no allocation, no memset, no
synchronisation), so a captured call replays; every replay is compared bit for bit with
the eager call, with eager work and host synchronisation between the replays."""
import numpy as np
import pytest
import torch

from gpu_util import device_inputs, make_plan
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu


CASES = [("c3_long_fp8", dict(nq=512, kv_len=8192)), ("c2_gqa_bf16", dict(nq=256, kv_len=4096 + 256)),
         ("c4_block_union", dict(nq=256, kv_len=16384)), ("c1_tiny", {})]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_eager(name, kw):
    cfg = CONFIGS[name].scaled(**kw) if kw else CONFIGS[name]
    print(f"[graph] {name} {kw}", flush=True)
    w = make_workload(cfg)
    d = device_inputs(w)
    plan = make_plan(w)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    plan(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], out, d["k_scale"], d["v_scale"], lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()

    g_out = torch.full_like(d["q"], float("nan"))
    g_lse = torch.full_like(lse, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):        # one call on the capturing side before capture
        plan(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], g_out, d["k_scale"], d["v_scale"], g_lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], g_out, d["k_scale"], d["v_scale"], g_lse)
    other = make_plan(w, grouping="original") if w.topk is not None else None
    for r in range(3):
        g_out.fill_(float("nan"))
        g_lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_out.view(torch.int16), ref_out.view(torch.int16)), f"replay {r}: out"
        assert torch.equal(g_lse.view(torch.int32), ref_lse.view(torch.int32)), f"replay {r}: lse"
        if other is not None:   # eager work on the same inputs between replays
            tmp = torch.empty_like(d["q"])
            other(d["ids"], d["q"], d["k"], d["v"], d["q_pos"], tmp, d["k_scale"], d["v_scale"])
            torch.cuda.synchronize()
            assert np.isfinite(tmp.float().cpu().numpy()).all()
