"""Pins of the KV-append oracle (oracle/kvcache.py) against what the number
format, a library cast and the workload generator's independent quantisation
fix (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import kvcache
from oracle.numerics import E4M3FN_TABLE
from workloads.gen import _to_fp8_codes


def _bf16_round(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.float().numpy(), t.view(torch.int16).numpy().view(np.uint16)


def _torch_e4m3(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-13, np.log2(448.0), 200_000)).astype(np.float32)
    y = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    fin = E4M3FN_TABLE[:0x7F]
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)       # exact in fp32: ties
    y = np.concatenate([y, mids, -mids, fin.astype(np.float32), [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    assert (kvcache.e4m3fn_encode(y) == _torch_e4m3(y)).all()


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if np.isfinite(E4M3FN_TABLE[c])], dtype=np.uint8)
    assert (kvcache.e4m3fn_encode(E4M3FN_TABLE[codes].astype(np.float32)) == codes).all()


def test_encode_ties_go_to_even_code():
    # 1.0625 lies half way between 1.0 (0x38) and 1.125 (0x39); 1.1875 between 0x39 and 1.25 (0x3A);
    # 3 * 2^-10 between the subnormals 2^-9 (0x01) and 2^-8 (0x02); 2^-10 between 0 and 2^-9.
    y = np.array([1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, -1.0625, 464.0 - 16.0], dtype=np.float32)
    assert list(kvcache.e4m3fn_encode(y)) == [0x38, 0x3A, 0x02, 0x00, 0xB8, 0x7E]


def _fresh(hkv, n_pages, ps, d, dtype):
    if dtype == "bf16":
        z = np.zeros((hkv, n_pages, ps, d), dtype=np.uint16)
        return z, z.copy(), None, None
    z = np.zeros((hkv, n_pages, ps, d), dtype=np.uint8)
    return z, z.copy(), np.ones((hkv, n_pages), np.float32), np.ones((hkv, n_pages), np.float32)


def test_full_append_matches_generator_quantisation():
    hkv, n_pages, ps, d = 2, 5, 16, 32
    rng = np.random.default_rng(3)
    xk, bk = _bf16_round(rng.standard_normal((n_pages * ps, hkv, d)) * 3)
    xv, bv = _bf16_round(rng.standard_normal((n_pages * ps, hkv, d)) / 7)
    xk[5 * ps // 2:3 * ps] = 0.0                      # an all-zero page takes scale 1.0
    bk[5 * ps // 2:3 * ps] = 0
    kc, vc, ks, vs = _fresh(hkv, n_pages, ps, d, "fp8")
    kvcache.append_kv(kc, vc, ks, vs, bk, bv, 0, ps, "fp8")
    for x, c, s in ((xk, kc, ks), (xv, vc, vs)):
        paged = x.reshape(n_pages, ps, hkv, d).transpose(2, 0, 1, 3)
        codes, scale = _to_fp8_codes(paged)
        assert (c == codes).all() and (s == scale).all()


def test_decode_error_within_format_bound():
    hkv, n_pages, ps, d = 1, 3, 64, 64
    rng = np.random.default_rng(11)
    x, b = _bf16_round(rng.standard_normal((n_pages * ps, hkv, d)) * np.exp2(rng.integers(-8, 8, (1, 1, d))))
    kc, vc, ks, vs = _fresh(hkv, n_pages, ps, d, "fp8")
    kvcache.append_kv(kc, vc, ks, vs, b, b, 0, ps, "fp8")
    paged = x.reshape(n_pages, ps, hkv, d).transpose(2, 0, 1, 3).astype(np.float64)
    dec = E4M3FN_TABLE[kc] * ks[..., None, None].astype(np.float64)
    s = ks[..., None, None].astype(np.float64)
    # Half an ulp: 2^-4 relative for normals (3 mantissa bits), 2^-10 * scale for subnormals,
    # plus the fp32 quotient's own rounding.
    bound = np.maximum(np.abs(paged) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert (np.abs(dec - paged) <= bound).all()
    assert np.isclose(np.abs(dec).max(axis=(2, 3)), np.abs(paged).max(axis=(2, 3)), rtol=1e-6).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_append_in_pieces_equals_one_chunk(dtype):
    """With each page's largest value in its first slot, no page's scale grows
    after its first piece, so any split of the chunk gives the one-shot cache."""
    hkv, n_pages, ps, d = 2, 6, 16, 16
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, n_pages * ps, hkv, d))
    x[:, ::ps] = 8.0
    _, kb = _bf16_round(x[0])
    _, vb = _bf16_round(-x[1])
    one = _fresh(hkv, n_pages, ps, d, dtype)
    kvcache.append_kv(*one, kb, vb, 0, ps, dtype)
    for cuts in ([0, 5, 40, 41, 96], [0, 16, 33, 70, 96], [0, 1, 2, 3, 96]):
        many = _fresh(hkv, n_pages, ps, d, dtype)
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            kvcache.append_kv(*many, kb[lo:hi], vb[lo:hi], lo, ps, dtype)
        for got, want in zip(many, one):
            if want is not None:
                assert (got == want).all()


def test_scale_growth_reencodes_earlier_slots():
    hkv, n_pages, ps, d = 1, 2, 16, 8
    rng = np.random.default_rng(9)
    _, b1 = _bf16_round(rng.standard_normal((5, hkv, d)))
    _, b2 = _bf16_round(rng.standard_normal((20, hkv, d)) * 10)
    kc, vc, ks, vs = _fresh(hkv, n_pages, ps, d, "fp8")
    kvcache.append_kv(kc, vc, ks, vs, b1, b1, 0, ps, "fp8")
    old_codes, old_scale = kc[0, 0, :5].copy(), ks[0, 0]
    kvcache.append_kv(kc, vc, ks, vs, b2, b2, 5, ps, "fp8")
    x2 = (b2.astype(np.uint32) << 16).view(np.float32)
    a = np.float32(np.abs(x2[:11, 0]).max())
    assert ks[0, 0] == np.float32(a / np.float32(448)) > old_scale
    # earlier slots: their decoded fp32 values re-rounded under the new scale
    dec = (E4M3FN_TABLE[old_codes].astype(np.float32) * old_scale).astype(np.float32)
    want = _torch_e4m3(np.clip(dec / ks[0, 0], -448, 448))
    assert (kc[0, 0, :5] == want).all()
    # the second page is fresh: scale from its own 9 tokens
    assert ks[0, 1] == np.float32(np.float32(np.abs(x2[11:, 0]).max()) / np.float32(448))


def test_scale_kept_when_chunk_is_smaller():
    hkv, n_pages, ps, d = 1, 1, 16, 8
    _, b1 = _bf16_round(np.full((4, hkv, d), 100.0))
    _, b2 = _bf16_round(np.full((4, hkv, d), 1.0))
    kc, vc, ks, vs = _fresh(hkv, n_pages, ps, d, "fp8")
    kvcache.append_kv(kc, vc, ks, vs, b1, b1, 0, ps, "fp8")
    before = kc[0, 0, :4].copy()
    kvcache.append_kv(kc, vc, ks, vs, b2, b2, 4, ps, "fp8")
    assert ks[0, 0] == np.float32(np.float32(100.0) / np.float32(448))
    assert (kc[0, 0, :4] == before).all()
    assert (kc[0, 0, 4:8] == _torch_e4m3(np.float32(1.0) / ks[0, 0])).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_tail_zeroed_and_other_pages_untouched(dtype):
    hkv, n_pages, ps, d = 2, 4, 16, 8
    kc, vc, ks, vs = _fresh(hkv, n_pages, ps, d, dtype)
    kc[:] = 0x33
    vc[:] = 0x33
    _, b = _bf16_round(np.ones((10, hkv, d)))
    kvcache.append_kv(kc, vc, ks, vs, b, b, 20, ps, dtype)     # tokens 20..29: page 1, slots 4..13
    for c in (kc, vc):
        assert (c[:, 0] == 0x33).all() and (c[:, 2:] == 0x33).all()
        assert (c[:, 1, :4] != 0).all()              # earlier slots (re-encoded or kept), never zeroed
        assert (c[:, 1, 14:] == 0).all()
        if dtype == "bf16":
            assert (c[:, 1, 4:14] == 0x3F80).all()


def test_append_rejects_overflow_and_nonfinite():
    kc, vc, ks, vs = _fresh(1, 2, 16, 8, "fp8")
    _, b = _bf16_round(np.ones((10, 1, 8)))
    with pytest.raises(ValueError):
        kvcache.append_kv(kc, vc, ks, vs, b, b, 25, 16, "fp8")
    with pytest.raises(ValueError):
        kvcache.e4m3fn_encode(np.array([np.nan], np.float32))
