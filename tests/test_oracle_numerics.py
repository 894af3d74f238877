"""Pins for the oracle's number decoding: library casts of torch (CPU)."""
import math

import numpy as np
import torch

from oracle import numerics


def test_e4m3fn_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = numerics.E4M3FN_TABLE
    nan_ref, nan_ours = np.isnan(ref), np.isnan(ours)
    assert (nan_ref == nan_ours).all()
    assert nan_ours.sum() == 2                      # S.1111.111, both signs
    assert np.array_equal(ref[~nan_ref], ours[~nan_ours])


def test_e4m3fn_special_values():
    assert numerics.e4m3fn_value(0x7E) == 448.0     # largest finite
    assert numerics.e4m3fn_value(0x01) == 2.0 ** -9  # smallest subnormal
    assert numerics.e4m3fn_value(0x08) == 2.0 ** -6  # smallest normal
    assert numerics.e4m3fn_value(0x38) == 1.0
    assert numerics.e4m3fn_value(0x80) == 0.0 and math.copysign(1, numerics.e4m3fn_value(0x80)) < 0
    assert math.isnan(numerics.e4m3fn_value(0xFF))


def test_bf16_decode_matches_torch_cast():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = numerics.bf16_bits_to_f64(bits)
    both = ~np.isnan(ref)
    assert (np.isnan(ours) == ~both).all()
    assert np.array_equal(ours[both], ref[both])


def test_decode_kv_fp8_applies_page_scale():
    codes = np.full((2, 3, 4), 0x38, dtype=np.uint8)   # 1.0
    scale = np.array([0.5, 2.0], dtype=np.float32)
    out = numerics.decode_kv(codes, scale, "fp8")
    assert np.array_equal(out[0], np.full((3, 4), 0.5))
    assert np.array_equal(out[1], np.full((3, 4), 2.0))
