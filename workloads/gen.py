"""Seeded input generators.

Every array is drawn from ``numpy.random.Generator(PCG64)`` children of
``SeedSequence(seed)``, spawned in a fixed order (communities, assignment,
picks, Q, K, V), so a (config, seed) pair always yields the same bytes.

Supports are TopK sets of page IDs per (query, KV head), as in PageWeaver's
"fixed TopK pages" (Fig. 1 caption).  Community-structured supports give
neighbouring queries different but overlapping page sets, the situation the
regrouping of Fig. 2 exploits; the uniform mode has no such structure; the
block-union mode draws 2-D block-sparse mask rows per (head, Q-block) as in
CompactAttention's chunked prefill.

Values: Q, K, V ~ N(0, 1) in fp32, rounded to bf16 (round-to-nearest-even,
torch CPU cast).  For fp8 caches each (KV head, page) of K and of V gets its
own fp32 scale = max|x| / 448 and codes e4m3fn(clamp(x / scale, +-448)); the
clamp matters because torch's e4m3fn cast maps out-of-range values to NaN.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import Config

FP8_MAX = 448.0


@dataclass
class Workload:
    cfg: Config
    q: np.ndarray                    # uint16 bf16 bits [nq, hq, d]
    k: np.ndarray                    # bf16 bits uint16 or fp8 codes uint8 [hkv, n_pages, ps, d]
    v: np.ndarray                    # same as k
    k_scale: Optional[np.ndarray]    # float32 [hkv, n_pages] (fp8 only)
    v_scale: Optional[np.ndarray]
    q_pos: np.ndarray                # int32 [nq]
    topk: Optional[np.ndarray]       # int32 [nq, hkv, K], -1 = empty slot (None for block_union)
    mask_rows: Optional[np.ndarray]  # block_union: int32 [n_qblocks * G, hkv, Kmax], -1 padded
    seed: int

    @property
    def n_pages(self) -> int:
        return self.cfg.n_pages


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _to_fp8_codes(x: np.ndarray):
    """Per-(head, page) scaled OCP e4m3fn encoding of x [hkv, n_pages, ps, d]."""
    amax = np.abs(x).max(axis=(2, 3))
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale[:, :, None, None], -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale


def _kv_tensor(rng: np.random.Generator, cfg: Config):
    shape = (cfg.hkv, cfg.n_pages, cfg.ps, cfg.d)
    x = rng.standard_normal(shape, dtype=np.float32)
    if cfg.kv_dtype == "bf16":
        return _to_bf16_bits(x), None
    if cfg.kv_dtype == "fp8":
        return _to_fp8_codes(x)
    raise ValueError(f"kv_dtype {cfg.kv_dtype!r}")


def _community_supports(cfg: Config, q_pos: np.ndarray, r_comm, r_assign, r_picks) -> np.ndarray:
    nq, hkv, K, ps = cfg.nq, cfg.hkv, cfg.k, cfg.ps
    last_prefix_page = cfg.first_pos // ps - 1          # prefix pages 1 .. last_prefix_page
    pool = np.arange(1, max(last_prefix_page, 0) + 1)
    csize = min(cfg.comm_size, len(pool))
    comms = np.zeros((hkv, max(cfg.n_comm, 1), csize), dtype=np.int64)
    for g in range(hkv):
        for c in range(cfg.n_comm):
            comms[g, c] = r_comm.choice(pool, size=csize, replace=False) if csize else []
    assign = r_assign.integers(0, max(cfg.n_comm, 1), size=(nq, hkv))
    out = np.full((nq, hkv, K), -1, dtype=np.int32)
    n_comm_picks = K - (2 if cfg.forced else 0) - cfg.n_uniform
    for i in range(nq):
        own = int(q_pos[i]) // ps
        for g in range(hkv):
            chosen = []
            if cfg.forced:
                chosen = [0] if own == 0 else [0, own]
            members = [int(p) for p in comms[g, assign[i, g]] if int(p) not in chosen]
            take = min(max(n_comm_picks, 0), len(members))
            if take:
                chosen += [int(p) for p in r_picks.choice(members, size=take, replace=False)]
            if cfg.n_uniform:
                rest = np.setdiff1d(np.arange(own + 1), np.asarray(chosen, dtype=np.int64))
                take = min(cfg.n_uniform, len(rest))
                if take:
                    chosen += [int(p) for p in r_picks.choice(rest, size=take, replace=False)]
            chosen = chosen[:K]
            perm = r_picks.permutation(len(chosen))
            out[i, g, :len(chosen)] = np.asarray(chosen, dtype=np.int32)[perm]
    return out


def _uniform_supports(cfg: Config, q_pos: np.ndarray, r_picks) -> np.ndarray:
    nq, hkv, K, ps = cfg.nq, cfg.hkv, cfg.k, cfg.ps
    out = np.full((nq, hkv, K), -1, dtype=np.int32)
    for i in range(nq):
        own = int(q_pos[i]) // ps
        n = own + 1
        take = min(K, n)
        for g in range(hkv):
            out[i, g, :take] = r_picks.choice(n, size=take, replace=False)
    return out


def _block_union_rows(cfg: Config, r_comm, r_picks) -> np.ndarray:
    """Block-sparse mask rows per (Q-block b, head-in-group hh) and KV head g.

    Row r = b * G + hh holds the blocks selected by query head g * G + hh for the
    queries of Q-block b: sink block 0 and the diagonal block are forced, the
    rest are drawn from a per-KV-group pool so that rows of one group are
    correlated (the union is then far from dense, as the page reports for real
    masks).  Blocks are ``cfg.ps`` tokens; Q-blocks are ``cfg.ps`` queries.
    """
    ps, G, hkv = cfg.ps, cfg.g, cfg.hkv
    n_qb = (cfg.nq + ps - 1) // ps
    n_prefix = cfg.first_pos // ps                       # blocks 0 .. n_prefix-1 precede the chunk
    cand = np.arange(1, n_prefix)
    pool_size = int(np.floor(cfg.pool_frac * len(cand) + 0.5))
    rows = []
    kmax = 0
    for g in range(hkv):
        pool = r_comm.choice(cand, size=pool_size, replace=False) if pool_size else np.zeros(0, np.int64)
        per_g = []
        for b in range(n_qb):
            diag = (cfg.first_pos + b * ps) // ps
            target = int(np.floor(cfg.density * (diag + 1) + 0.5))
            for _hh in range(G):
                row = [0] if diag == 0 else [0, diag]
                take = min(max(target - len(row), 0), len(pool))
                if take:
                    row += [int(p) for p in r_picks.choice(pool, size=take, replace=False)]
                per_g.append(row)
                kmax = max(kmax, len(row))
        rows.append(per_g)
    out = np.full((n_qb * G, hkv, kmax), -1, dtype=np.int32)
    for g in range(hkv):
        for r, row in enumerate(rows[g]):
            out[r, g, :len(row)] = np.asarray(row, dtype=np.int32)[r_picks.permutation(len(row))]
    return out


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(6)]


def _supports(cfg: Config, q_pos, r_comm, r_assign, r_picks):
    topk = mask_rows = None
    if cfg.support == "community":
        topk = _community_supports(cfg, q_pos, r_comm, r_assign, r_picks)
    elif cfg.support == "uniform":
        topk = _uniform_supports(cfg, q_pos, r_picks)
    elif cfg.support == "block_union":
        mask_rows = _block_union_rows(cfg, r_comm, r_picks)
    else:
        raise ValueError(f"support {cfg.support!r}")
    return topk, mask_rows


def make_supports(cfg: Config, seed: Optional[int] = None):
    """(q_pos, topk, mask_rows) exactly as make_workload draws them, without Q, K and V."""
    seed = cfg.seed if seed is None else seed
    r_comm, r_assign, r_picks, _, _, _ = _streams(seed)
    q_pos = np.arange(cfg.first_pos, cfg.kv_len, dtype=np.int32)
    return (q_pos,) + _supports(cfg, q_pos, r_comm, r_assign, r_picks)


def make_workload(cfg: Config, seed: Optional[int] = None) -> Workload:
    seed = cfg.seed if seed is None else seed
    if cfg.hq % cfg.hkv:
        raise ValueError("hq must be a multiple of hkv")
    r_comm, r_assign, r_picks, r_q, r_k, r_v = _streams(seed)
    q_pos = np.arange(cfg.first_pos, cfg.kv_len, dtype=np.int32)
    topk, mask_rows = _supports(cfg, q_pos, r_comm, r_assign, r_picks)
    q = _to_bf16_bits(r_q.standard_normal((cfg.nq, cfg.hq, cfg.d), dtype=np.float32))
    k, k_scale = _kv_tensor(r_k, cfg)
    v, v_scale = _kv_tensor(r_v, cfg)
    return Workload(cfg=cfg, q=q, k=k, v=v, k_scale=k_scale, v_scale=v_scale, q_pos=q_pos,
                    topk=topk, mask_rows=mask_rows, seed=seed)
