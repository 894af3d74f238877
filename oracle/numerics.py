"""Number formats of the inputs, decoded from their definitions (fp64 exact).

bf16: the upper 16 bits of an IEEE-754 binary32 value.
OCP fp8 E4M3 ("e4m3fn", OCP 8-bit floating point specification): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals 2^-6 * m/8; S.1111.111 is NaN; there is no infinity; the largest
finite magnitude is 2^8 * 1.75 = 448.  PageWeaver keeps the KV cache in FP8
throughout (abstract); each (KV head, page) carries an fp32 scale and the
decoded value is code * scale.
"""
from __future__ import annotations

import math

import numpy as np


def e4m3fn_value(code: int) -> float:
    """Value of one OCP e4m3fn byte, from the format's definition."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = math.ldexp(m / 8.0, 1 - 7)
    else:
        mag = math.ldexp(1.0 + m / 8.0, e - 7)
    return -mag if s else mag


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN payloads stay NaN
        return b.view(np.float32).astype(np.float64)


def decode_kv(data: np.ndarray, scale, kv_dtype: str) -> np.ndarray:
    """Decode a cache slab [..., n_pages, ps, d] to fp64.

    ``scale`` is None for bf16, else fp32 [..., n_pages] applied per page.
    """
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(data)
    if kv_dtype == "fp8":
        vals = E4M3FN_TABLE[np.asarray(data, dtype=np.uint8)]
        return vals * np.asarray(scale, dtype=np.float64)[..., None, None]
    raise ValueError(f"kv_dtype {kv_dtype!r}")
