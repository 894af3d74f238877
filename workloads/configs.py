"""The five synthetic workload shapes and their knobs.

Shapes follow the pages' workloads: PageWeaver measures 16K-query chunks of
64K-context captures with Top16 page supports, groups of eight and FP8 KV
(PageWeaver abstract; Table 1; Fig. 1 caption); CompactAttention measures
chunked prefill at 128K with chunk 1024 and block-sparse masks turned into
per-KV-group block tables (CompactAttention summary, "Approach" and "Key
results").  Model captures and benchmark suites are not available, so these
seeded synthetic inputs stand in for them.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    hq: int                 # query heads
    hkv: int                # KV heads (GQA ratio G = hq // hkv)
    d: int                  # head dimension
    ps: int                 # page size in tokens
    kv_len: int             # tokens in the cache, the chunk's own tokens included
    nq: int                 # queries in the chunk (the last nq positions)
    kv_dtype: str           # "bf16" or "fp8" (OCP e4m3 + fp32 scale per (kv head, page))
    support: str            # "community", "uniform" or "block_union"
    k: int                  # pages per (query, KV head) support (block_union: unused)
    n_comm: int = 0         # communities per KV head
    comm_size: int = 0      # pages per community
    n_uniform: int = 0      # picks drawn uniformly from the causal prefix
    forced: bool = True     # sink page 0 and the query's own page always selected
    density: float = 0.0    # block_union: per-row block density
    pool_frac: float = 0.0  # block_union: fraction of prefix blocks in a KV group's pool
    window: int = 64        # grouping window W (consecutive query IDs)
    max_group: int = 8      # queries per group
    item_rows: int = 128    # block_union: query-head rows per work item over a shared table
    seed: int = 1

    @property
    def g(self) -> int:
        return self.hq // self.hkv

    @property
    def n_pages(self) -> int:
        return (self.kv_len + self.ps - 1) // self.ps

    @property
    def first_pos(self) -> int:
        return self.kv_len - self.nq

    def scaled(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # Tiny single-head case: 16 pages of 64, the last 256 positions are queries,
    # Top4 = sink + own page + 2 from one of 4 communities of 4 pages.
    "c1_tiny": Config(
        name="c1_tiny", hq=1, hkv=1, d=64, ps=64, kv_len=1024, nq=256, kv_dtype="bf16",
        support="community", k=4, n_comm=4, comm_size=4, n_uniform=0, seed=1),
    # GQA chunk: 16K prefix + 2048 queries, Top16 from 16 communities of 24 pages.
    "c2_gqa_bf16": Config(
        name="c2_gqa_bf16", hq=32, hkv=8, d=128, ps=64, kv_len=16384 + 2048, nq=2048,
        kv_dtype="bf16", support="community", k=16, n_comm=16, comm_size=24, n_uniform=0,
        seed=2),
    # Long-context fp8: 64K context, 4096 queries, Top16 with 20% of picks uniform
    # over the causal prefix and the rest from 32 communities of 48 pages.
    "c3_long_fp8": Config(
        name="c3_long_fp8", hq=32, hkv=8, d=128, ps=64, kv_len=65536, nq=4096, kv_dtype="fp8",
        support="community", k=16, n_comm=32, comm_size=48, n_uniform=3, seed=3),
    # Block-union chunked prefill: 128K cache, 1024 queries, 128x128 blocks at 20%
    # density, sink + diagonal forced; pages are the 128-token blocks.
    "c4_block_union": Config(
        name="c4_block_union", hq=32, hkv=8, d=128, ps=128, kv_len=131072, nq=1024,
        kv_dtype="bf16", support="block_union", k=0, density=0.20, pool_frac=0.30, seed=4),
    # Adversarial low affinity: Top64 uniform over the causal prefix, G = 8.
    "c5_adversarial": Config(
        name="c5_adversarial", hq=64, hkv=8, d=128, ps=64, kv_len=65536, nq=4096,
        kv_dtype="fp8", support="uniform", k=64, forced=False, seed=5),
}

HEADLINE = "c3_long_fp8"


def get_config(name: str) -> Config:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None
