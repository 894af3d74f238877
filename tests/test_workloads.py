"""The generators draw what the workload recipes state (structure, not method arithmetic)."""
import numpy as np
import pytest

from workloads import CONFIGS, make_workload


def test_deterministic():
    a = make_workload(CONFIGS["c1_tiny"])
    b = make_workload(CONFIGS["c1_tiny"])
    for f in ("q", "k", "v", "topk", "q_pos"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_c1_structure():
    cfg = CONFIGS["c1_tiny"]
    w = make_workload(cfg)
    assert w.q.shape == (256, 1, 64) and w.k.shape == (1, 16, 64, 64)
    assert list(w.q_pos) == list(range(768, 1024))
    for i in range(cfg.nq):
        s = [int(x) for x in w.topk[i, 0]]
        assert len(set(s)) == 4 and 0 in s and (768 + i) // 64 in s
        rest = set(s) - {0, (768 + i) // 64}
        assert all(1 <= p <= 11 for p in rest)


def test_fp8_encoding_is_scaled_and_finite():
    cfg = CONFIGS["c1_tiny"].scaled(kv_dtype="fp8", name="c1_fp8")
    w = make_workload(cfg)
    assert w.k.dtype == np.uint8 and w.k_scale.shape == (1, 16)
    codes = w.k.reshape(-1)
    assert not np.isin(codes, [0x7F, 0xFF]).any()          # no NaN codes
    # each page reaches the top code magnitude 448 (0x7E / 0xFE) exactly once-ish
    top = (w.k & 0x7F).reshape(1, 16, -1).max(axis=2)
    assert (top == 0x7E).all()


@pytest.mark.parametrize("name", ["c1_tiny"])
def test_supports_are_causal(name):
    cfg = CONFIGS[name]
    w = make_workload(cfg)
    own = w.q_pos // cfg.ps
    assert (w.topk.max(axis=2) <= own[:, None]).all()


def test_make_supports_draws_the_workloads_supports():
    from workloads import make_supports
    for name in ("c1_tiny", "c4_block_union"):
        cfg = CONFIGS[name].scaled(kv_len=CONFIGS[name].kv_len // 4, nq=CONFIGS[name].nq // 4) \
            if name == "c4_block_union" else CONFIGS[name]
        w = make_workload(cfg)
        q_pos, topk, rows = make_supports(cfg)
        assert np.array_equal(q_pos, w.q_pos)
        assert (topk is None and w.topk is None) or np.array_equal(topk, w.topk)
        assert (rows is None and w.mask_rows is None) or np.array_equal(rows, w.mask_rows)
