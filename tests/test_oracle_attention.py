"""Pins for the oracle's attention: brute force, a library attention on the dense
case, closed forms, and independence of the result from the grouping."""
import math
import random

import numpy as np
import pytest
import torch

from oracle import attention, numerics, prep
from helpers import add_padding_and_duplicates, tiny_workload


def _route_a(w, S, queries=None):
    c = w.cfg
    return attention.route_a(w.q, w.k, w.v, w.k_scale, w.v_scale, c.kv_dtype, S, w.q_pos,
                             c.kv_len, c.ps, 1.0 / math.sqrt(c.d), queries)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("seed", [0, 1])
def test_route_a_equals_brute_force(kv_dtype, seed):
    w = tiny_workload(kv_dtype=kv_dtype, seed=20 + seed, k=3)
    topk = add_padding_and_duplicates(w.topk, seed)
    c = w.cfg
    S = prep.supports(topk, c.n_pages)
    O, L = _route_a(w, S)
    Ob, Lb = attention.brute_force(w.q, w.k, w.v, w.k_scale, w.v_scale, kv_dtype, S, w.q_pos,
                                   c.kv_len, c.ps, 1.0 / math.sqrt(c.d))
    assert np.allclose(O, Ob, rtol=0, atol=1e-12)
    fin = np.isfinite(Lb)
    assert (np.isfinite(L) == fin).all()
    assert np.allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)


def _sdpa_dense(w):
    """torch SDPA (fp64, CPU) over the whole cache with a bottom-right causal mask."""
    c = w.cfg
    G = c.hq // c.hkv
    q = torch.from_numpy(numerics.bf16_bits_to_f64(w.q)).permute(1, 0, 2)[None]        # [1,hq,nq,d]
    k = numerics.decode_kv(w.k, w.k_scale, c.kv_dtype).reshape(c.hkv, -1, c.d)[:, :c.kv_len]
    v = numerics.decode_kv(w.v, w.v_scale, c.kv_dtype).reshape(c.hkv, -1, c.d)[:, :c.kv_len]
    k = torch.from_numpy(k).repeat_interleave(G, dim=0)[None]
    v = torch.from_numpy(v).repeat_interleave(G, dim=0)[None]
    t = torch.arange(c.kv_len)[None, :]
    mask = t <= torch.from_numpy(w.q_pos.astype(np.int64))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=1.0 / math.sqrt(c.d))
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_dense_support_equals_library_attention(kv_dtype):
    w = tiny_workload(kv_dtype=kv_dtype, hq=6, hkv=2, d=16, ps=8, kv_len=61, nq=13, seed=5)
    c = w.cfg
    S = attention.dense_supports(c.nq, c.hkv, c.n_pages)
    O, _ = _route_a(w, S)
    assert np.allclose(O, _sdpa_dense(w), rtol=0, atol=1e-12)


def test_dense_support_positions_past_cache_end():
    # Positions beyond the cache end still see only tokens t < kv_len.
    w = tiny_workload(kv_dtype="bf16", hq=4, hkv=2, d=16, ps=8, kv_len=61, nq=13, seed=6)
    w.q_pos = w.q_pos + 5
    c = w.cfg
    S = attention.dense_supports(c.nq, c.hkv, c.n_pages)
    O, _ = _route_a(w, S)
    assert np.allclose(O, _sdpa_dense(w), rtol=0, atol=1e-12)


def test_closed_form_single_key():
    # Query at the first token of its own page with support {own page}: J = {that token}.
    w = tiny_workload(ps=4, kv_len=24, nq=8, hq=2, hkv=1, d=8)
    c = w.cfg
    S = [[frozenset({int(p) // c.ps}) for p in w.q_pos]]
    O, L = _route_a(w, S)
    Vd = numerics.decode_kv(w.v, None, "bf16").reshape(1, -1, c.d)[0]
    Kd = numerics.decode_kv(w.k, None, "bf16").reshape(1, -1, c.d)[0]
    Q = numerics.bf16_bits_to_f64(w.q)
    for n, p in enumerate(w.q_pos):
        if p % c.ps == 0:
            assert np.array_equal(O[n, 0], Vd[p]) and np.array_equal(O[n, 1], Vd[p])
            assert L[n, 0] == pytest.approx(Q[n, 0] @ Kd[p] / math.sqrt(c.d), abs=1e-13)


def test_closed_form_zero_query_is_mean():
    w = tiny_workload(seed=7, k=4)
    w.q[:] = 0
    c = w.cfg
    S = prep.supports(w.topk, c.n_pages)
    O, _ = _route_a(w, S)
    G = c.hq // c.hkv
    Vd = numerics.decode_kv(w.v, None, "bf16").reshape(c.hkv, -1, c.d)
    for i in range(c.nq):
        for h in range(c.hq):
            g = h // G
            J = [t for t in range(c.kv_len) if t // c.ps in S[g][i] and t <= w.q_pos[i]]
            want = Vd[g, J].mean(axis=0) if J else np.zeros(c.d)
            assert np.allclose(O[i, h], want, atol=1e-13)


def test_closed_form_identical_keys_is_mean():
    w = tiny_workload(seed=8, k=4)
    w.k[:] = w.k[0, 0, 0]                     # every key row identical
    c = w.cfg
    S = prep.supports(w.topk, c.n_pages)
    O, _ = _route_a(w, S)
    Vd = numerics.decode_kv(w.v, None, "bf16").reshape(c.hkv, -1, c.d)
    G = c.hq // c.hkv
    for i in range(c.nq):
        for h in range(c.hq):
            J = [t for t in range(c.kv_len) if t // c.ps in S[h // G][i] and t <= w.q_pos[i]]
            if J:
                assert np.allclose(O[i, h], Vd[h // G, J].mean(axis=0), atol=1e-13)


def test_own_page_only_is_local_causal_attention():
    w = tiny_workload(seed=9, ps=8, kv_len=40, nq=16, hq=2, hkv=1, d=8)
    c = w.cfg
    S = [[frozenset({int(p) // c.ps}) for p in w.q_pos]]
    O, _ = _route_a(w, S)
    Kd = torch.from_numpy(numerics.decode_kv(w.k, None, "bf16").reshape(-1, c.d))
    Vd = torch.from_numpy(numerics.decode_kv(w.v, None, "bf16").reshape(-1, c.d))
    Q = torch.from_numpy(numerics.bf16_bits_to_f64(w.q))
    for n, p in enumerate(w.q_pos):
        lo = (int(p) // c.ps) * c.ps
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[n][:, None, :], Kd[lo:p + 1][None].expand(2, -1, -1), Vd[lo:p + 1][None].expand(2, -1, -1),
            scale=1.0 / math.sqrt(c.d))
        assert np.allclose(O[n], ref[:, 0].numpy(), atol=1e-13)


def test_empty_support_and_future_pages():
    w = tiny_workload(seed=10, ps=4, kv_len=40, nq=6)
    c = w.cfg
    future = [[frozenset({c.n_pages - 1}) if int(p) < (c.n_pages - 1) * c.ps else frozenset()
               for p in w.q_pos] for _ in range(c.hkv)]
    O, L = _route_a(w, future)
    for n, p in enumerate(w.q_pos):
        if int(p) < (c.n_pages - 1) * c.ps:
            assert np.array_equal(O[n], np.zeros_like(O[n]))
            assert np.isneginf(L[n]).all()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_grouping_invariance_route_b(kv_dtype):
    w = tiny_workload(kv_dtype=kv_dtype, hq=4, hkv=2, d=16, ps=8, kv_len=200, nq=40, k=5, seed=12)
    c = w.cfg
    S = prep.supports(w.topk, c.n_pages)
    bits = prep.page_bitsets(w.topk, c.n_pages)
    sm = 1.0 / math.sqrt(c.d)
    OA, LA = _route_a(w, S)
    rng = random.Random(0)
    perm = list(range(c.nq))
    rng.shuffle(perm)
    groupings = {
        "affinity": [prep.group_affinity(b, 16, 4) for b in bits],
        "original": [prep.group_original(c.nq, 4) for _ in bits],
        "singletons": [[[i] for i in range(c.nq)] for _ in bits],
        "random": [[perm[j:j + 5] for j in range(0, c.nq, 5)] for _ in bits],
    }
    for name, grp in groupings.items():
        OB, LB = attention.route_b(w.q, w.k, w.v, w.k_scale, w.v_scale, kv_dtype, S, grp,
                                   w.q_pos, c.kv_len, c.ps, sm)
        assert not np.isnan(OB).any(), name
        assert np.allclose(OB, OA, rtol=0, atol=1e-12), name
        assert np.allclose(LB, LA, rtol=0, atol=1e-12), name


def test_query_subset_matches_full():
    w = tiny_workload(seed=13, k=3)
    c = w.cfg
    S = prep.supports(w.topk, c.n_pages)
    O, L = _route_a(w, S)
    sel = [7, 0, 3]
    Os, Ls = _route_a(w, S, sel)
    assert np.array_equal(Os, O[sel]) and np.array_equal(Ls, L[sel])


def test_nrms_definition():
    ref = np.array([3.0, 4.0])
    assert attention.nrms(ref, ref) == 0.0
    assert attention.nrms(np.array([3.0, 4.5]), ref) == pytest.approx(10.0)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_direct_page_union_route_c_equals_definition(kv_dtype):
    """The direct KV-page union (partials per (query, page), merged by their lse)
    reaches the definition, including empty supports, pages wholly in a query's
    future and positions past the cache end."""
    w = tiny_workload(kv_dtype=kv_dtype, hq=4, hkv=2, d=16, ps=8, kv_len=197, nq=40, k=5, seed=14)
    c = w.cfg
    topk = add_padding_and_duplicates(w.topk, 3)
    topk[0, 0, :] = -1                                        # an empty support
    topk[1, 1, 0] = c.n_pages - 1                             # a page after the query
    S = prep.supports(topk, c.n_pages)
    OA, LA = _route_a(w, S)
    OC, LC = attention.route_c(w.q, w.k, w.v, w.k_scale, w.v_scale, kv_dtype, S, w.q_pos,
                               c.kv_len, c.ps, 1.0 / math.sqrt(c.d))
    assert np.allclose(OC, OA, rtol=0, atol=1e-12)
    assert (np.isneginf(LC) == np.isneginf(LA)).all()
    fin = np.isfinite(LA)
    assert np.allclose(LC[fin], LA[fin], rtol=0, atol=1e-12)
    assert np.isneginf(LC[0, :2]).all() and not OC[0, :2].any()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("batch,workers", [(1, 1), (5, 2), (64, 3)])
def test_route_a_batched_equals_route_a(kv_dtype, batch, workers):
    """The batched route A (padded gathers with an explicit J(i, g) mask, threads over KV
    heads) gives route A's result: supports of different sizes with padding slots and
    duplicates, an empty support, a page wholly after its query, positions past the
    cache end and a cache end inside a page."""
    w = tiny_workload(kv_dtype=kv_dtype, hq=6, hkv=3, d=16, ps=8, kv_len=197, nq=41, k=5, seed=15)
    c = w.cfg
    topk = add_padding_and_duplicates(w.topk, 4)
    topk[0, 0, :] = -1                                        # an empty support
    topk[1, 1, :2] = -1                                       # a shorter support
    topk[2, 2, 0] = c.n_pages - 1                             # a page after the query
    w.q_pos = w.q_pos.copy()
    w.q_pos[-3:] += 9                                         # positions past the cache end
    S = prep.supports(topk, c.n_pages)
    OA, LA = _route_a(w, S)
    OB, LB = attention.route_a_batched(w.q, w.k, w.v, w.k_scale, w.v_scale, kv_dtype, S, w.q_pos,
                                       c.kv_len, c.ps, 1.0 / math.sqrt(c.d), batch=batch,
                                       workers=workers)
    assert np.allclose(OB, OA, rtol=0, atol=1e-12)
    assert (np.isneginf(LB) == np.isneginf(LA)).all()
    fin = np.isfinite(LA)
    assert np.allclose(LB[fin], LA[fin], rtol=0, atol=1e-12)
    assert not OB[0, :2].any() and np.isneginf(LB[0, :2]).all()
    sel = [40, 3, 0, 17]
    Os, Ls = attention.route_a_batched(w.q, w.k, w.v, w.k_scale, w.v_scale, kv_dtype, S, w.q_pos,
                                       c.kv_len, c.ps, 1.0 / math.sqrt(c.d), queries=sel, batch=batch)
    assert np.allclose(Os, OA[sel], rtol=0, atol=1e-12)


def test_route_a_batched_shared_table_equals_route_a():
    """A batch whose queries share one support (a per-KV-group block table) is gathered
    once and still masked per query: the same result as route A, also against the
    dense library attention when the table holds every page."""
    w = tiny_workload(kv_dtype="bf16", hq=4, hkv=2, d=16, ps=8, kv_len=150, nq=30, seed=16)
    c = w.cfg
    tables = [[0, 3, 5, 6, 7, 9, 12, 15, 17, 18], [1, 2, 4, 8, 11, 16, 18]]
    S = attention.shared_supports(tables, c.nq)
    OA, LA = _route_a(w, S)
    OB, LB = attention.route_a_batched(w.q, w.k, w.v, w.k_scale, w.v_scale, "bf16", S, w.q_pos,
                                       c.kv_len, c.ps, 1.0 / math.sqrt(c.d), batch=8, workers=2)
    assert np.allclose(OB, OA, rtol=0, atol=1e-12)
    assert np.allclose(LB[np.isfinite(LA)], LA[np.isfinite(LA)], rtol=0, atol=1e-12)
    Sd = attention.dense_supports(c.nq, c.hkv, c.n_pages)
    Od, _ = attention.route_a_batched(w.q, w.k, w.v, None, None, "bf16", Sd, w.q_pos, c.kv_len, c.ps,
                                      1.0 / math.sqrt(c.d), batch=7)
    assert np.allclose(Od, _sdpa_dense(w), rtol=0, atol=1e-12)
