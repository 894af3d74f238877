"""Writing a prefill chunk's keys and values into the paged cache (test oracle).

PageWeaver keeps the KV cache in FP8 throughout (abstract) and its chunked
prefill appends each chunk's keys and values before attending; CompactAttention
runs in place over the paged cache in a KV-head-major layout ("Approach").
Neither page fixes how a per-page scale evolves when a chunk starts part way
into a page, so this oracle takes the plainest reading that keeps every stored
value representable:

* token ``t = first_token + i`` of the chunk goes to page ``t // ps``, slot
  ``t % ps`` of every KV head; the new values are bf16 (the projection's type);
* bf16 cache: the bits are copied;
* fp8 cache, separately for K and V and for each touched (KV head, page):
  ``a`` = max |x| over the chunk's tokens on the page (fp32);
  a page the chunk starts on (slots before the chunk hold earlier tokens) keeps
  its scale if ``a / 448 <= scale_old``, else takes ``a / 448``; any other
  touched page gets ``a / 448``, or 1.0 when ``a == 0``;
  new slots get ``e4m3fn(clamp(x / scale, -448, 448))``; when a page's scale
  grew, its earlier slots are re-encoded from their decoded fp32 values
  ``code * scale_old`` the same way;
* slots after the chunk's last token on its last page are zeroed, so that a
  page never holds stale or non-finite values past the end of the cache.

The scale and every code are decided in fp32 (the kernel's precision): the
quotient ``x / scale`` is the correctly rounded fp32 division, and the code is
that quotient rounded to the nearest e4m3fn value, ties to the even code.  The
decision is then exact in fp64 below.  Plain numpy, slow on purpose.
"""
from __future__ import annotations

import numpy as np

from .numerics import E4M3FN_TABLE

FP8_MAX = np.float32(448.0)

# Finite non-negative e4m3fn values by code 0x00..0x7E (ascending in code order).
_POS_VALUES = E4M3FN_TABLE[:0x7F]


def e4m3fn_encode(y) -> np.ndarray:
    """Round fp32 values to OCP e4m3fn codes: nearest finite value, ties to the
    even code; |y| must not exceed 448 (callers clamp first).  Sign is kept,
    so values rounding to zero from below give the negative-zero code 0x80."""
    y = np.asarray(y, dtype=np.float32)
    if not np.isfinite(y).all():
        raise ValueError("e4m3fn_encode: non-finite input")
    a = np.abs(y).astype(np.float64)
    if (a > 448.0).any():
        raise ValueError("e4m3fn_encode: |value| > 448 (clamp first)")
    hi = np.searchsorted(_POS_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    exact = d_hi == 0
    pick_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


def quantize(x32: np.ndarray, scale: np.float32) -> np.ndarray:
    """Codes of fp32 values under one page scale: e4m3fn(clamp(x / scale))."""
    q = (np.asarray(x32, dtype=np.float32) / np.float32(scale)).astype(np.float32)
    return e4m3fn_encode(np.clip(q, -FP8_MAX, FP8_MAX))


def _append_one(cache, scale, new_bits, first_token, ps, kv_dtype):
    """One tensor (K or V): cache [hkv, n_pages, ps, d] (uint16 bf16 bits or
    uint8 codes), scale [hkv, n_pages] fp32 or None, new_bits uint16 [n_tok, hkv, d]."""
    n_tok, hkv, d = new_bits.shape
    if n_tok == 0:
        return
    last = first_token + n_tok - 1
    for p in range(first_token // ps, last // ps + 1):
        base = p * ps
        s0 = max(first_token - base, 0)                 # first slot written by the chunk
        s1 = min(last - base, ps - 1) + 1               # one past the last written slot
        rows = slice(base + s0 - first_token, base + s1 - first_token)
        for g in range(hkv):
            if kv_dtype == "bf16":
                cache[g, p, s0:s1] = new_bits[rows, g]
                cache[g, p, s1:] = 0
                continue
            x = (new_bits[rows, g].astype(np.uint32) << np.uint32(16)).view(np.float32)
            a = np.float32(np.abs(x).max())
            s_new = np.float32(a / FP8_MAX)
            if s0 > 0:
                s_old = np.float32(scale[g, p])
                if s_new > s_old:
                    old = (E4M3FN_TABLE[cache[g, p, :s0]].astype(np.float32) * s_old).astype(np.float32)
                    cache[g, p, :s0] = quantize(old, s_new)
                else:
                    s_new = s_old
            elif a == 0:
                s_new = np.float32(1.0)
            scale[g, p] = s_new
            cache[g, p, s0:s1] = quantize(x, s_new)
            cache[g, p, s1:] = 0


def append_kv(k_cache, v_cache, k_scale, v_scale, k_new, v_new, first_token, ps, kv_dtype):
    """Write the chunk's keys and values into the caches in place.

    k_cache, v_cache  [hkv, n_pages, ps, d]: uint16 bf16 bits, or uint8 e4m3fn codes
    k_scale, v_scale  fp32 [hkv, n_pages] (fp8) or None (bf16)
    k_new, v_new      uint16 bf16 bits [n_tok, hkv, d] (token-major)
    first_token       position of the chunk's first token
    """
    n_tok = k_new.shape[0]
    if first_token < 0 or (n_tok and (first_token + n_tok - 1) // ps >= k_cache.shape[1]):
        raise ValueError("append_kv: chunk does not fit the cache")
    for cache, scale, new in ((k_cache, k_scale, k_new), (v_cache, v_scale, v_new)):
        _append_one(cache, scale, np.asarray(new, dtype=np.uint16), first_token, ps, kv_dtype)
