"""Seeded synthetic workloads for query-union sparse prefill.

This package only draws inputs: query/KV tensors, per-query TopK page supports,
query positions and the optional fp8 encoding of the KV cache that the pages
take as given ("FP8 KV throughout", PageWeaver abstract).  It holds none of the
method's arithmetic (no bitsets, grouping, unions or attention), so both the
CPU oracle and the HIP path may consume what it returns.
"""
from .configs import CONFIGS, Config, get_config
from .gen import Workload, make_supports, make_workload

__all__ = ["CONFIGS", "Config", "get_config", "Workload", "make_supports", "make_workload"]
