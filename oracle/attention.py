"""Causal softmax attention of every query over exactly its own pages, in fp64.

The union method is exact: masked query-page slots are excluded and every
selected edge is retained (PageWeaver Fig. 2 caption), each query keeps its
original support and owns its complete output row (abstract).  So the result
is the plain definition below; grouping only changes how it is reached.

Notation (readings where the pages are silent are listed in the design notes):
query i sits at position p_i = q_pos[i]; query head h reads KV head
g = h // G; token t lies on page t // ps; the allowed keys of (i, g) are

    J(i, g) = { t : t // ps in S(i, g),  t <= p_i,  t < kv_len }

and, with s_t = sigma * <Q[i, h], K[g, t]>,

    O[i, h] = sum_{t in J} exp(s_t - m) V[g, t] / sum_{t in J} exp(s_t - m),
    lse[i, h] = m + log sum_{t in J} exp(s_t - m),   m = max_{t in J} s_t,

with O = 0 and lse = -inf when J is empty.  K and V are the decoded cache
values (bf16 exact, or e4m3fn code times the page scale, exact in fp64).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np

from .numerics import bf16_bits_to_f64, decode_kv


def _softmax_pv(s: np.ndarray, v: np.ndarray):
    """s [R, n] scores, v [n, d] -> (O [R, d], lse [R]); n == 0 gives zeros / -inf."""
    R, n = s.shape
    if n == 0:
        return np.zeros((R, v.shape[1])), np.full(R, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ v) / l, (m + np.log(l))[:, 0]


def route_a(q_bits, k_data, v_data, k_scale, v_scale, kv_dtype: str,
            S: List[List[frozenset]], q_pos, kv_len: int, ps: int, sm_scale: float,
            queries: Optional[Sequence[int]] = None):
    """Per-query gather of the selected pages: the definition.

    q_bits uint16 [nq, hq, d]; k_data/v_data [hkv, n_pages, ps, d]; S[g][i] sets.
    Returns O fp64 [n_sel, hq, d] and lse fp64 [n_sel, hq] for ``queries``
    (default: all) in the order given.
    """
    nq, hq, d = q_bits.shape
    hkv = k_data.shape[0]
    G = hq // hkv
    queries = list(range(nq)) if queries is None else list(queries)
    O = np.zeros((len(queries), hq, d))
    L = np.full((len(queries), hq), -np.inf)
    for g in range(hkv):
        Kg = decode_kv(k_data[g], None if k_scale is None else k_scale[g], kv_dtype)
        Vg = decode_kv(v_data[g], None if v_scale is None else v_scale[g], kv_dtype)
        for n, i in enumerate(queries):
            pages = np.asarray(sorted(S[g][i]), dtype=np.int64)
            t = (pages[:, None] * ps + np.arange(ps)[None, :]).reshape(-1)
            keep = (t <= int(q_pos[i])) & (t < kv_len)
            kk = Kg[pages].reshape(-1, d)[keep]
            vv = Vg[pages].reshape(-1, d)[keep]
            qh = bf16_bits_to_f64(q_bits[i, g * G:(g + 1) * G])          # [G, d]
            o, lse = _softmax_pv(sm_scale * (qh @ kk.T), vv)
            O[n, g * G:(g + 1) * G] = o
            L[n, g * G:(g + 1) * G] = lse
    return O, L


def _route_a_batch(Kg, Vg, g, G, q_bits, S, q_pos, kv_len, ps, sm_scale, ids):
    """Route A for the queries `ids` and the query heads of KV head g (its decoded K and V
    given): returns O [len(ids), G, d] and lse [len(ids), G]."""
    d = q_bits.shape[2]
    sets = [S[g][i] for i in ids]
    qh = bf16_bits_to_f64(q_bits[ids, g * G:(g + 1) * G])                  # [B, G, d]
    pos = np.asarray([int(q_pos[i]) for i in ids], dtype=np.int64)
    if sets[0] and all(s == sets[0] for s in sets):
        # one support for the whole batch (a per-KV-group table): gathered once
        pages = np.asarray(sorted(sets[0]), dtype=np.int64)[None, :]
    else:
        width = max(1, max(len(s) for s in sets))
        pages = np.full((len(ids), width), -1, dtype=np.int64)              # -1: padding
        for n, s in enumerate(sets):
            pages[n, :len(s)] = sorted(s)
    t = pages[:, :, None] * ps + np.arange(ps)[None, None, :]              # token of each slot
    keep = (pages[:, :, None] >= 0) & (t <= pos[:, None, None]) & (t < kv_len)
    keep = np.broadcast_to(keep.reshape(keep.shape[0], -1), (len(ids), t[0].size))
    safe = np.maximum(pages, 0)
    kk = Kg[safe].reshape(pages.shape[0], -1, d)                             # [1 or B, n, d]
    vv = Vg[safe].reshape(pages.shape[0], -1, d)
    s_t = sm_scale * np.matmul(qh, kk.transpose(0, 2, 1))                   # [B, G, n]
    s_t = np.where(keep[:, None, :], s_t, -np.inf)                          # keys outside J(i, g)
    has = keep.any(axis=1)
    m = np.where(has[:, None, None], s_t.max(axis=2, keepdims=True), 0.0)
    e = np.exp(s_t - m)                                                     # 0 outside J
    l = e.sum(axis=2, keepdims=True)
    o = np.matmul(e, vv) / np.where(has[:, None, None], l, 1.0)
    O = np.where(has[:, None, None], o, 0.0)
    L = np.where(has[:, None], (m + np.log(np.where(has[:, None, None], l, 1.0)))[:, :, 0], -np.inf)
    return O, L


def route_a_batched(q_bits, k_data, v_data, k_scale, v_scale, kv_dtype: str,
                    S: List[List[frozenset]], q_pos, kv_len: int, ps: int, sm_scale: float,
                    queries: Optional[Sequence[int]] = None, batch: int = 64, workers: int = 1):
    """Route A (the definition) with `batch` queries per numpy call, the (KV head, batch)
    pieces spread over `workers` threads.  Each query's scores, softmax and PV still use
    its own keys J(i, g) only: its gathered support slots outside J (padding of a shorter
    support, keys after its position or past the cache end) are excluded by an explicit
    mask.  A batch whose queries share one support gathers it once (the per-KV-group block
    table of CompactAttention's "Approach").  Same outputs as ``route_a`` (up to rounding
    order); sized for whole chunks."""
    nq, hq, d = q_bits.shape
    hkv = k_data.shape[0]
    G = hq // hkv
    queries = list(range(nq)) if queries is None else list(queries)
    O = np.zeros((len(queries), hq, d))
    L = np.full((len(queries), hq), -np.inf)

    def decode(g):
        return (decode_kv(k_data[g], None if k_scale is None else k_scale[g], kv_dtype),
                decode_kv(v_data[g], None if v_scale is None else v_scale[g], kv_dtype))

    def piece(task):
        g, b0 = task
        Kg, Vg = heads[g]
        o, l = _route_a_batch(Kg, Vg, g, G, q_bits, S, q_pos, kv_len, ps, sm_scale,
                              queries[b0:b0 + batch])
        O[b0:b0 + batch, g * G:(g + 1) * G] = o
        L[b0:b0 + batch, g * G:(g + 1) * G] = l

    tasks = [(g, b0) for g in range(hkv) for b0 in range(0, len(queries), batch)]
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor

        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
            heads = list(ex.map(decode, range(hkv)))
            list(ex.map(piece, tasks))
    else:
        heads = [decode(g) for g in range(hkv)]
        for task in tasks:
            piece(task)
    return O, L


def route_b(q_bits, k_data, v_data, k_scale, v_scale, kv_dtype: str,
            S: List[List[frozenset]], groups_per_g: List[List[List[int]]], q_pos,
            kv_len: int, ps: int, sm_scale: float):
    """Through group unions: every group's union pages are visited once for all
    members, and each member masks out pages it did not select and future keys.
    Returns O fp64 [nq, hq, d], lse [nq, hq]; rows are written by original ID."""
    nq, hq, d = q_bits.shape
    hkv = k_data.shape[0]
    G = hq // hkv
    O = np.full((nq, hq, d), np.nan)
    L = np.full((nq, hq), np.nan)
    for g in range(hkv):
        Kg = decode_kv(k_data[g], None if k_scale is None else k_scale[g], kv_dtype)
        Vg = decode_kv(v_data[g], None if v_scale is None else v_scale[g], kv_dtype)
        for members in groups_per_g[g]:
            union = sorted(frozenset().union(*(S[g][m] for m in members)))
            pages = np.asarray(union, dtype=np.int64)
            t = (pages[:, None] * ps + np.arange(ps)[None, :]).reshape(-1)
            tok_page = np.repeat(pages, ps)
            kk = Kg[pages].reshape(-1, d)
            vv = Vg[pages].reshape(-1, d)
            for m in members:
                sel = np.isin(tok_page, np.asarray(sorted(S[g][m]), dtype=np.int64))
                keep = sel & (t <= int(q_pos[m])) & (t < kv_len)
                qh = bf16_bits_to_f64(q_bits[m, g * G:(g + 1) * G])
                o, lse = _softmax_pv(sm_scale * (qh @ kk[keep].T), vv[keep])
                O[m, g * G:(g + 1) * G] = o
                L[m, g * G:(g + 1) * G] = lse
    return O, L


def route_c(q_bits, k_data, v_data, k_scale, v_scale, kv_dtype: str,
            S: List[List[frozenset]], q_pos, kv_len: int, ps: int, sm_scale: float):
    """Through the direct KV-page union (PageWeaver abstract, its complementary
    page-major study): every (KV head, page) is visited once for all queries that
    selected it; each (query, head, page) gives a partial softmax over that page's
    usable keys - a normalised output o_i and its lse_i - and each row's partials
    are merged by their lse:  lse = log sum_i exp(lse_i),
    O = sum_i exp(lse_i - lse) o_i  (empty rows: O = 0, lse = -inf).
    Returns O fp64 [nq, hq, d], lse [nq, hq]."""
    nq, hq, d = q_bits.shape
    hkv = k_data.shape[0]
    G = hq // hkv
    n_pages = k_data.shape[1]
    parts = {}
    for g in range(hkv):
        Kg = decode_kv(k_data[g], None if k_scale is None else k_scale[g], kv_dtype)
        Vg = decode_kv(v_data[g], None if v_scale is None else v_scale[g], kv_dtype)
        lists = [[] for _ in range(n_pages)]
        for i in range(nq):
            for p in sorted(S[g][i]):
                lists[p].append(i)
        for p in range(n_pages):
            t = p * ps + np.arange(ps)
            for i in lists[p]:
                keep = (t <= int(q_pos[i])) & (t < kv_len)
                qh = bf16_bits_to_f64(q_bits[i, g * G:(g + 1) * G])
                o, lse = _softmax_pv(sm_scale * (qh @ Kg[p][keep].T), Vg[p][keep])
                parts.setdefault((i, g), []).append((lse, o))
    O = np.zeros((nq, hq, d))
    L = np.full((nq, hq), -np.inf)
    for (i, g), lst in parts.items():
        lses = np.stack([x[0] for x in lst])            # [n_parts, G]
        outs = np.stack([x[1] for x in lst])            # [n_parts, G, d]
        m = lses.max(axis=0)
        ok = np.isfinite(m)
        w = np.where(ok[None, :], np.exp(lses - np.where(ok, m, 0.0)[None, :]), 0.0)
        tot = w.sum(axis=0)
        O[i, g * G:(g + 1) * G] = np.where(ok[:, None], (w[:, :, None] * outs).sum(axis=0)
                                           / np.where(ok, tot, 1.0)[:, None], 0.0)
        L[i, g * G:(g + 1) * G] = np.where(ok, m + np.log(np.where(ok, tot, 1.0)), -np.inf)
    return O, L


def brute_force(q_bits, k_data, v_data, k_scale, v_scale, kv_dtype: str,
                S: List[List[frozenset]], q_pos, kv_len: int, ps: int, sm_scale: float):
    """Explicit scalar loops with math.exp over every (query, head, token): tiny inputs only."""
    nq, hq, d = q_bits.shape
    hkv, n_pages = k_data.shape[0], k_data.shape[1]
    G = hq // hkv
    K = [decode_kv(k_data[g], None if k_scale is None else k_scale[g], kv_dtype).tolist() for g in range(hkv)]
    V = [decode_kv(v_data[g], None if v_scale is None else v_scale[g], kv_dtype).tolist() for g in range(hkv)]
    Q = bf16_bits_to_f64(q_bits).tolist()
    O = [[[0.0] * d for _ in range(hq)] for _ in range(nq)]
    L = [[-math.inf] * hq for _ in range(nq)]
    for i in range(nq):
        for h in range(hq):
            g = h // G
            scores = []
            for t in range(n_pages * ps):
                if (t // ps) in S[g][i] and t <= q_pos[i] and t < kv_len:
                    p, r = divmod(t, ps)
                    dot = 0.0
                    for c in range(d):
                        dot += Q[i][h][c] * K[g][p][r][c]
                    scores.append((sm_scale * dot, p, r))
            if not scores:
                continue
            m = max(s for s, _, _ in scores)
            den = 0.0
            acc = [0.0] * d
            for s, p, r in scores:
                w = math.exp(s - m)
                den += w
                for c in range(d):
                    acc[c] += w * V[g][p][r][c]
            O[i][h] = [a / den for a in acc]
            L[i][h] = m + math.log(den)
    return np.asarray(O), np.asarray(L)


def dense_supports(nq: int, hkv: int, n_pages: int) -> List[List[frozenset]]:
    """Every query selects every page (TopK = all pages)."""
    full = frozenset(range(n_pages))
    return [[full] * nq for _ in range(hkv)]


def shared_supports(tables: List[List[int]], nq: int) -> List[List[frozenset]]:
    """Every query of KV head g attends to the whole per-KV-group table T_g."""
    return [[frozenset(t)] * nq for t in tables]


def nrms(out: np.ndarray, ref: np.ndarray) -> float:
    """||O - R||_2 / ||R||_2 over all output elements, in percent."""
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.sqrt((ref ** 2).sum()))
    num = float(np.sqrt(((np.asarray(out, dtype=np.float64) - ref) ** 2).sum()))
    return 100.0 * num / den if den else 0.0
