"""Pins of the oracle's fp8 encoder, quantise-on-insert and paged addressing."""
import numpy as np
import pytest
import torch

from context_mla_prefill_amd import synth
from oracle import kvcache as ok
from oracle import numerics as on

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _brute_encode(x):
    """Argmin over every finite code of |value - x|; of equal distances the even code,
    then the code whose sign matches x (so -0.0 -> 0x80)."""
    vals = on.e4m3fn_decode(FINITE)
    out = np.empty(len(x), dtype=np.uint8)
    for i, v in enumerate(np.asarray(x, dtype=np.float32).astype(np.float64)):
        d = np.abs(vals - v)
        best = FINITE[d == d.min()]
        even = best[(best & 1) == 0]
        best = even if len(even) else best
        want_neg = np.signbit(np.float32(v))
        signed = best[((best & 0x80) != 0) == want_neg]
        out[i] = (signed if len(signed) else best)[0]
    return out


def test_encode_round_trips_every_finite_code():
    vals = on.e4m3fn_decode(FINITE).astype(np.float32)
    assert np.array_equal(on.e4m3fn_encode_rne(vals), FINITE)


def test_encode_matches_brute_force_at_midpoints():
    mags = on.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    mid = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)  # exact in binary32
    assert np.all(mid.astype(np.float64) == (mags[:-1] + mags[1:]) / 2)
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    x = np.concatenate([mid, up, dn, -mid, -up, -dn, [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    assert np.array_equal(on.e4m3fn_encode_rne(x), _brute_encode(x))


def test_encode_ties_go_to_even_code():
    # 0x08 = 2^-6, 0x09 = 2^-6 * 9/8, 0x0A = 2^-6 * 10/8
    m89 = np.float32(2.0 ** -6 * 17 / 16)
    m9a = np.float32(2.0 ** -6 * 19 / 16)
    assert list(on.e4m3fn_encode_rne(np.array([m89, m9a, -m89]))) == [0x08, 0x0A, 0x88]
    # subnormal tie: halfway between 0 and the smallest subnormal 2^-9 goes to 0
    assert list(on.e4m3fn_encode_rne(np.array([2.0 ** -10, 3 * 2.0 ** -10], np.float32))) == [0x00, 0x02]


def test_encode_matches_torch_cast():
    """A library routine: torch's float8_e4m3fn conversion (round to nearest even)."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * 60, rng.standard_normal(5000) * 0.01,
                        rng.uniform(-448, 448, 5000)]).clip(-448, 448).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(on.e4m3fn_encode_rne(x), lib)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        on.e4m3fn_encode_rne(np.array([449.0], np.float32))
    with pytest.raises(ValueError):
        on.e4m3fn_encode_rne(np.array([np.nan], np.float32))


def _fresh(N, D):
    return np.full((N, D), 0x7F, np.uint8), np.full((N + 63) // 64, np.nan, np.float32)


def test_quantize_closed_form_power_of_two_scale():
    """Rows that are E4M3FN values times 2^-3 with a block maximum of 448 * 2^-3: the scale
    is exactly 2^-3 and every code comes back unchanged."""
    rng = np.random.default_rng(1)
    D = 64
    codes = rng.choice(FINITE, size=(64, D))
    codes[5, 9] = 0x7E  # 448: the block maximum
    x = (on.e4m3fn_decode(codes) * 0.125).astype(np.float32)
    bits = synth.bf16_bits(x)  # exact: 4 significant bits
    cache, sc = _fresh(128, D)
    c2, s2 = ok.quantize_insert_fp8(cache, sc, bits, np.arange(64, 128))
    assert s2[1] == np.float32(0.125) and np.isnan(s2[0])
    got = c2[64:]
    # +-0 codes of a zero value keep its sign; compare values and the nonzero codes
    assert np.array_equal(on.e4m3fn_decode(got), on.e4m3fn_decode(codes))
    assert np.array_equal(got[x != 0], codes[x != 0])
    assert np.all(c2[:64] == 0x7F)  # untouched rows


def test_quantize_scale_per_block_and_zero_block():
    D = 16
    x = np.zeros((192, D), np.float32)
    x[:64] = 3.0
    x[10, 2] = -7.0  # block 0 amax 7
    x[64:128] = 0.5  # block 1 amax 0.5
    # block 2 all zero
    cache, sc = _fresh(192, D)
    c2, s2 = ok.quantize_insert_fp8(cache, sc, synth.bf16_bits(x), np.arange(192))
    # 7/448 = 2^-6 is a power of two; 0.5/448 lies in (2^-10, 2^-9]
    assert s2[0] == np.float32(2.0 ** -6) and s2[1] == np.float32(2.0 ** -9)
    assert s2[2] == 1.0 and np.all(c2[128:] == 0)
    assert c2[10, 2] == 0xFE  # -448 after dividing by the block's own scale
    assert np.all(c2[64:128] == 0x78)  # every element is the block maximum, 0.5 / 2^-9 = 256


def test_quantize_later_rows_use_the_stored_scale():
    """A block opened by a first call (rows 0..9) keeps its scale when a second call writes
    rows 10..63; a value beyond 448 * scale saturates. (2/448 lies in (2^-8, 2^-7].)"""
    D = 8
    cache, sc = _fresh(64, D)
    a = np.full((10, D), 2.0, np.float32)
    c1, s1 = ok.quantize_insert_fp8(cache, sc, synth.bf16_bits(a), np.arange(10))
    assert s1[0] == np.float32(2.0 ** -7)
    b = np.full((54, D), 1.0, np.float32)
    b[3, 1] = 5.0  # 5 / 2^-7 = 640 -> saturates
    b[4, 2] = -5.0
    c2, s2 = ok.quantize_insert_fp8(c1, s1, synth.bf16_bits(b), np.arange(10, 64))
    assert s2[0] == s1[0] and np.array_equal(c2[:10], c1[:10])
    assert c2[13, 1] == 0x7E and c2[14, 2] == 0xFE
    assert on.e4m3fn_decode(c2[10:11, 0])[0] == 128.0  # 1 / 2^-7


def test_quantize_skips_rows_outside_the_cache():
    cache, sc = _fresh(64, 8)
    x = np.ones((3, 8), np.float32)
    c2, s2 = ok.quantize_insert_fp8(cache, sc, synth.bf16_bits(x), np.array([-1, 64, 0]))
    # 1/448 lies in (2^-9, 2^-8]: scale 2^-8, code of 256
    assert np.all(c2[0] == 0x78) and np.all(c2[1:] == 0x7F) and s2[0] == np.float32(2.0 ** -8)


def test_quantize_error_bound():
    """|decode(code) * scale - x| <= 2^-4 |x| + 2^-10 scale (half an ulp of a 3-bit
    mantissa, or of the subnormal step 2^-9) for every element of fresh blocks."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((256, 512)) * np.exp(rng.standard_normal((256, 1)))).astype(np.float32)
    bits = synth.bf16_bits(x)
    xe = on.bf16_to_f64(bits)
    cache, sc = _fresh(256, 512)
    c2, s2 = ok.quantize_insert_fp8(cache, sc, bits, np.arange(256))
    s = s2[np.arange(256) // 64].astype(np.float64)[:, None]
    err = np.abs(on.e4m3fn_decode(c2) * s - xe)
    assert np.all(err <= 2.0 ** -4 * np.abs(xe) + 2.0 ** -10 * s * (1 + 1e-6))
    # the block scale is a power of two with max|x| / 448 <= scale < 2 max|x| / 448 (the
    # smallest such power; the block's largest element lands in (224, 448])
    for B in range(4):
        a = np.abs(xe[64 * B:64 * B + 64]).max() / 448.0
        m, _ = np.frexp(np.float64(s2[B]))
        assert m == 0.5 and a * (1 - 2.0 ** -23) <= s2[B] < 2 * a


def test_pow2_at_least():
    """Powers of two map to themselves, anything above one to the next, and everything at or
    below 2^-126 (zero and subnormals included) to 2^-126."""
    for e in (-126, -40, -6, 0, 1, 100):
        p = np.float32(2.0 ** e)
        assert ok.pow2_at_least(p) == p
        up = np.nextafter(p, np.float32(np.inf))
        assert ok.pow2_at_least(up) == np.float32(2.0 ** (e + 1))
        if e > -126:
            assert ok.pow2_at_least(np.nextafter(p, np.float32(0))) == p
    for r in (0.0, 1e-45, 2.0 ** -130):
        assert ok.pow2_at_least(r) == np.float32(2.0 ** -126)
    assert ok.pow2_at_least(0.3) == 0.5 and ok.pow2_at_least(200.0) == 256.0


def test_paged_rows():
    bt = np.array([[5, 2, 9], [0, 7, -1]])
    assert list(ok.paged_rows(bt, 0, [0, 63, 64, 130])) == [320, 383, 128, 578]
    assert list(ok.paged_rows(bt, 1, [1, 127])) == [1, 511]
    # identity table of a 64-aligned packed layout reproduces packed rows
    kv_start = np.array([0, 192])
    ident = np.array([[0, 1, 2, 3], [3, 4, 5, 6]])
    pos = np.arange(250)
    assert np.array_equal(ok.paged_rows(ident, 1, pos), kv_start[1] + pos)
