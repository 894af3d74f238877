"""Small-input builders shared by the tests (no method arithmetic here)."""
import numpy as np

from workloads import make_workload
from workloads.configs import Config


def tiny_config(**kw) -> Config:
    base = dict(name="tiny", hq=4, hkv=2, d=8, ps=4, kv_len=30, nq=9, kv_dtype="bf16",
                support="uniform", k=3, forced=False, window=8, max_group=4, seed=11)
    base.update(kw)
    return Config(**base)


def tiny_workload(**kw):
    return make_workload(tiny_config(**kw))


def add_padding_and_duplicates(topk: np.ndarray, seed: int = 0) -> np.ndarray:
    """Append -1 slots and repeat some IDs: supports are sets, so nothing changes."""
    rng = np.random.default_rng(seed)
    n, h, k = topk.shape
    extra = np.full((n, h, 3), -1, dtype=np.int32)
    dup = rng.integers(0, k, size=(n, h))
    extra[:, :, 0] = np.take_along_axis(topk, dup[:, :, None], axis=2)[:, :, 0]
    out = np.concatenate([topk, extra], axis=2)
    for i in range(n):
        for g in range(h):
            out[i, g] = out[i, g][rng.permutation(out.shape[2])]
    return out
