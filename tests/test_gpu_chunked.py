"""GPU: chunked prefill of one sequence (append -> prepare -> attend per chunk), with the
next chunk's preparation on a second stream, against the oracle and against the same
run without overlap."""
import math

import numpy as np
import pytest
import torch

import query_union_kv_amd as pw
from gpu_util import oracle_workers
from oracle import attention, kvcache, prep
from workloads import make_workload
from workloads.configs import Config

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _make_chunks(kv_dtype, bounds, hq=8, hkv=2, d=128, ps=64, k=8, seed=0):
    """One sequence of bounds[-1] tokens prefilled in chunks [bounds[i], bounds[i+1])."""
    total = bounds[-1]
    n_pages = -(-total // ps)
    rng = np.random.default_rng(seed)
    chunks = []
    for i, (lo, hi) in enumerate(zip(bounds[:-1], bounds[1:])):
        cfg = Config(name="chunk", hq=hq, hkv=hkv, d=d, ps=ps, kv_len=hi, nq=hi - lo, kv_dtype="bf16",
                     support="uniform", k=k, forced=True, seed=100 + seed * 10 + i)
        w = make_workload(cfg)                    # its Q, positions and TopK pages
        chunks.append(dict(q_bits=w.q, q_pos=w.q_pos.astype(np.int32), topk=w.topk, first_token=lo,
                           k_bits=_bf16_bits(rng.standard_normal((hi - lo, hkv, d)) * (1 + i)),
                           v_bits=_bf16_bits(rng.standard_normal((hi - lo, hkv, d)))))
    return chunks, n_pages


def _run(chunks, n_pages, kv_dtype, overlap, hq=8, hkv=2, d=128, ps=64, k=8):
    if kv_dtype == "fp8":
        kc = torch.zeros((hkv, n_pages, ps, d), dtype=torch.uint8, device="cuda")
        ks = torch.ones((hkv, n_pages), dtype=torch.float32, device="cuda")
        vc, vs = kc.clone(), ks.clone()
    else:
        kc = torch.zeros((hkv, n_pages, ps, d), dtype=torch.bfloat16, device="cuda")
        vc, ks, vs = kc.clone(), None, None
    max_chunk = max(c["q_bits"].shape[0] for c in chunks)
    runner = pw.ChunkedPrefill(hq=hq, hkv=hkv, d=d, n_pages=n_pages, page_size=ps, max_chunk=max_chunk, k=k)
    dev = []
    for c in chunks:
        dev.append(dict(q=_dev_bf16(c["q_bits"]), k_new=_dev_bf16(c["k_bits"]), v_new=_dev_bf16(c["v_bits"]),
                        topk=torch.from_numpy(np.ascontiguousarray(c["topk"])).cuda(),
                        q_pos=torch.from_numpy(c["q_pos"]).cuda(), first_token=c["first_token"],
                        out=torch.full((c["q_bits"].shape[0], hq, d), float("nan"), dtype=torch.bfloat16,
                                       device="cuda")))
    runner.run(dev, kc, vc, ks, vs, overlap=overlap)
    torch.cuda.synchronize()
    return [x["out"].float().cpu().numpy() for x in dev]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_chunked_prefill_matches_oracle_and_serial(kv_dtype):
    bounds = [0, 1000, 2048, 3100, 4096]          # ragged: chunks share boundary pages
    chunks, n_pages = _make_chunks(kv_dtype, bounds)
    got = _run(chunks, n_pages, kv_dtype, overlap=True)
    ser = _run(chunks, n_pages, kv_dtype, overlap=False)
    for a, b in zip(got, ser):
        assert np.array_equal(a, b)
    _check_against_oracle(chunks, got, n_pages, kv_dtype)


def test_chunked_prefill_wide_groups_as_halves():
    """Eight query heads per KV head make 64-row groups, which every chunk's plan runs as
    two halves (the fused half-table preparation on the side stream): overlap equals
    serial bit for bit, and every row matches the oracle."""
    bounds = [0, 700, 1500, 2200]
    chunks, n_pages = _make_chunks("fp8", bounds, hq=16, seed=3)
    got = _run(chunks, n_pages, "fp8", overlap=True, hq=16)
    ser = _run(chunks, n_pages, "fp8", overlap=False, hq=16)
    for a, b in zip(got, ser):
        assert np.array_equal(a, b)
    _check_against_oracle(chunks, got, n_pages, "fp8")


def _check_against_oracle(chunks, got, n_pages, kv_dtype, hkv=2, ps=64, d=128):
    # oracle: append chunk by chunk; attend each chunk on the cache as it stood then
    if kv_dtype == "fp8":
        k = np.zeros((hkv, n_pages, ps, d), np.uint8)
        ks = np.ones((hkv, n_pages), np.float32)
    else:
        k = np.zeros((hkv, n_pages, ps, d), np.uint16)
        ks = None
    v, vs = k.copy(), (ks.copy() if ks is not None else None)
    for c, o in zip(chunks, got):
        kvcache.append_kv(k, v, ks, vs, c["k_bits"], c["v_bits"], c["first_token"], ps, kv_dtype)
        n = c["q_bits"].shape[0]
        S = prep.supports(c["topk"], n_pages)
        # every row of the chunk (route A indexes q_pos / q by chunk-local query number)
        O, _ = attention.route_a_batched(c["q_bits"], k, v, ks, vs, kv_dtype, S, c["q_pos"],
                                         c["first_token"] + n, ps, 1.0 / math.sqrt(d),
                                         workers=oracle_workers())
        err = np.abs(o - O)
        assert np.isfinite(o).all()
        assert err.max() <= (6e-2 if kv_dtype == "fp8" else 2e-2), err.max()
        if kv_dtype == "bf16":
            assert err.mean() <= 2e-3, err.mean()
