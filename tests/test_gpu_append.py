"""GPU parity of pw_append_kv (chunk K/V append with per-page fp8 quantisation)
against the oracle, bit for bit: codes, scales and every untouched byte."""
import numpy as np
import pytest
import torch

import query_union_kv_amd as pw
from oracle import kvcache
from oracle.numerics import E4M3FN_TABLE

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _initial_cache(rng, hkv, n_pages, ps, d, dtype):
    """A cache already holding arbitrary content (earlier tokens and stale bytes)."""
    if dtype == "bf16":
        k = _bf16_bits(rng.standard_normal((hkv, n_pages, ps, d)))
        v = _bf16_bits(rng.standard_normal((hkv, n_pages, ps, d)))
        return k, v, None, None
    k = rng.integers(0, 0x7F, (hkv, n_pages, ps, d), dtype=np.uint8) | \
        (rng.integers(0, 2, (hkv, n_pages, ps, d), dtype=np.uint8) << 7)
    v = rng.integers(0, 0x7F, (hkv, n_pages, ps, d), dtype=np.uint8)
    ks = (rng.uniform(0.001, 0.02, (hkv, n_pages))).astype(np.float32)
    vs = (rng.uniform(0.001, 0.02, (hkv, n_pages))).astype(np.float32)
    return k, v, ks, vs


def _chunk(rng, n_tok, hkv, d, mag):
    x = rng.standard_normal((n_tok, hkv, d)) * mag
    x[rng.random(x.shape) < 0.01] = 0.0
    return _bf16_bits(x)


def _to_dev(a, dtype):
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _from_dev(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _run_both(state, chunks, ps, dtype, qkv_stride=False):
    """Apply the same sequence of appends on the GPU and in the oracle."""
    k, v, ks, vs = state
    dev = [_to_dev(a, dtype) for a in (k, v, ks, vs)]
    ref = [a.copy() if a is not None else None for a in (k, v, ks, vs)]
    for first, kb, vb in chunks:
        kvcache.append_kv(ref[0], ref[1], ref[2], ref[3], kb, vb, first, ps, dtype)
        if qkv_stride:
            # keys and values as slices of one fused [n_tok, 3*hkv, d] projection output
            n, hkv, d = kb.shape
            fused = torch.zeros((n, 3 * hkv, d), dtype=torch.bfloat16, device="cuda")
            fused[:, hkv:2 * hkv] = _to_dev(kb, "bf16")
            fused[:, 2 * hkv:] = _to_dev(vb, "bf16")
            kt, vt = fused[:, hkv:2 * hkv], fused[:, 2 * hkv:]
        else:
            kt, vt = _to_dev(kb, "bf16"), _to_dev(vb, "bf16")
        pw.pw_append_kv(kt, vt, first, dev[0], dev[1], dev[2], dev[3])
    torch.cuda.synchronize()
    got = [_from_dev(t) for t in dev]
    for name, g, r in zip(("k_cache", "v_cache", "k_scale", "v_scale"), got, ref):
        if r is None:
            continue
        if g.dtype == np.float32:
            bad = np.flatnonzero(g.view(np.uint32) != r.view(np.uint32))
        else:
            bad = np.flatnonzero(g != r)
        assert bad.size == 0, f"{name}: {bad.size} mismatches, first at {np.unravel_index(bad[0], g.shape)}"


# (first_token, n_tok) cases over a 12-page cache: page-aligned, mid-page start and end,
# a single token, a chunk inside one page, a chunk ending on a page boundary, the whole cache.
CASES = [(0, 64), (64, 200), (70, 3), (130, 1), (100, 28), (33, 95), (0, 768), (765, 3), (1, 766)]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("first,n_tok", CASES)
def test_append_parity(dtype, first, n_tok):
    hkv, n_pages, ps, d = 3, 12, 64, 128
    rng = np.random.default_rng(1000 + first * 7 + n_tok)
    state = _initial_cache(rng, hkv, n_pages, ps, d, dtype)
    mag = 10.0 if first % 2 else 0.05          # grow some mid-page scales, keep others
    _run_both(state, [(first, _chunk(rng, n_tok, hkv, d, mag), _chunk(rng, n_tok, hkv, d, mag))], ps, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("ps,d", [(64, 64), (128, 128), (16, 8), (64, 136), (256, 128)])
def test_append_sequence_of_chunks(dtype, ps, d):
    """Chunked prefill: consecutive ragged chunks, magnitudes varying so that some
    pages keep and some grow their scales; a strided (fused QKV) source."""
    hkv, n_pages = 2, 10
    rng = np.random.default_rng(ps + d)
    state = _initial_cache(rng, hkv, n_pages, ps, d, dtype)
    total = n_pages * ps
    cuts = [c for c in (0, 37, 37, 100, 101, 300, 512) if c < total - 5] + [total - 5]
    chunks = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        mag = float(rng.choice([0.01, 1.0, 30.0]))
        chunks.append((lo, _chunk(rng, hi - lo, hkv, d, mag), _chunk(rng, hi - lo, hkv, d, mag)))
    _run_both(state, chunks, ps, dtype, qkv_stride=(ps == 64))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_append_full_size_chunk(dtype):
    """A 4096-token chunk into a 64K-token cache with 8 KV heads of d=128 (the
    long-context workload's own chunk), compared over the whole cache."""
    hkv, ps, d, kv_len, n_tok = 8, 64, 128, 65536, 4096
    n_pages = kv_len // ps
    rng = np.random.default_rng(77)
    state = _initial_cache(rng, hkv, n_pages, ps, d, dtype)
    _run_both(state, [(kv_len - n_tok, _chunk(rng, n_tok, hkv, d, 1.0), _chunk(rng, n_tok, hkv, d, 3.0))],
              ps, dtype)


@pytest.mark.parametrize("scale", [0.125, 0.3, 2.0 ** -20])
def test_append_rounding_ties(scale):
    """Values at, and one bf16 step either side of, every e4m3fn rounding midpoint times
    the page scale (exact ties when the scale is a power of two), appended part way
    into a page whose scale they do not raise."""
    fin = E4M3FN_TABLE[:0x7F]
    mids = ((fin[1:] + fin[:-1]) / 2 * np.float32(scale)).astype(np.float32)
    b = _bf16_bits(mids).astype(np.int32)
    vals = np.concatenate([b, b - 1, b + 1]).astype(np.uint16)
    vals = np.concatenate([vals, vals | 0x8000])
    hkv, n_pages, ps, d = 1, 2, 64, 128
    n_tok = -(-vals.size // d)
    chunk = np.zeros(n_tok * d, np.uint16)
    chunk[:vals.size] = vals
    chunk = chunk.reshape(n_tok, hkv, d)
    rng = np.random.default_rng(3)
    k, v, ks, vs = _initial_cache(rng, hkv, n_pages, ps, d, "fp8")
    ks[:] = np.float32(scale)
    vs[:] = np.float32(scale)
    _run_both((k, v, ks, vs), [(5, chunk, chunk[::-1].copy())], ps, "fp8")


def test_append_nothing_is_a_noop():
    k = torch.zeros((1, 2, 64, 64), dtype=torch.uint8, device="cuda")
    s = torch.ones((1, 2), dtype=torch.float32, device="cuda")
    e = torch.zeros((0, 1, 64), dtype=torch.bfloat16, device="cuda")
    pw.pw_append_kv(e, e, 5, k, k.clone(), s, s.clone())
    torch.cuda.synchronize()
    assert int(k.sum()) == 0


def test_append_rejects_overflow():
    k = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((10, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pw.PWError, match="PW_ERR_CAPACITY"):
        pw.pw_append_kv(x, x, 120, k, k.clone())
