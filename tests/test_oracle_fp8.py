"""Pins of the oracle's E4M3 context cache (oracle/kv_fp8.py) to things other than itself:
the OCP E4M3 format's defining values, torch's float8_e4m3fn conversions (a library
routine) inside the finite range, exact round trips, the rounding error bound, and a
dequantised decode step whose values are exactly fp32 (power-of-two scales), checked
against the plain fp32 oracle path."""
import numpy as np
import pytest
import torch

import oracle
from oracle import kv_fp8 as f8

CODES = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_float8_e4m3fn():
    d = f8.e4m3_decode(CODES)
    t = _torch_decode(CODES).astype(np.float64)
    same = (d == t) | (np.isnan(d) & np.isnan(t))
    assert same.all(), CODES[~same]
    assert np.array_equal(np.signbit(d[~np.isnan(d)]), np.signbit(t[~np.isnan(t)]))


def test_decode_format_values():
    d = f8.e4m3_decode(CODES)
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0          # largest finite
    assert d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9  # subnormals m/8 * 2^-6
    assert d[0x08] == 2.0 ** -6                              # smallest normal
    assert d[0x38] == 1.0 and d[0xB8] == -1.0                # exponent field 7 = bias
    assert d[0x3C] == 1.5 and d[0x40] == 2.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])           # the only NaNs, no infinities
    assert np.isnan(d).sum() == 2
    assert d[0x00] == 0.0 and not np.signbit(d[0x00]) and np.signbit(d[0x80])
    fin = d[:0x7F]
    assert np.all(np.diff(fin) > 0)                          # codes 0..0x7E increase


def test_encode_matches_torch_inside_the_finite_range():
    rng = np.random.default_rng(5)
    mags = _torch_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (mags[:-1] + mags[1:]) / 2                         # exact ties, fp32 numbers
    xs = [mags, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
          np.nextafter(mids.astype(np.float32), np.float32(1e9)),
          np.exp2(rng.uniform(-13, np.log2(447.9), 200000)) * rng.choice([-1, 1], 200000)]
    x = np.concatenate([np.asarray(v, np.float64) for v in xs]).astype(np.float32)
    x = x[np.abs(x) < 448]
    x = np.concatenate([x, -x])
    assert np.array_equal(f8.e4m3_encode(x), _torch_encode(x))


def test_encode_ties_saturation_and_specials():
    e = lambda *v: [int(c) for c in f8.e4m3_encode(np.float32(v))]
    assert e(1.0625, 1.1875) == [0x38, 0x3A]            # ties to the even mantissa
    assert e(2.0 ** -10, 3 * 2.0 ** -10) == [0x00, 0x02]  # subnormal ties
    assert e(15 * 2.0 ** -10) == [0x08]                 # 7.5 * 2^-9 rounds up into the normals
    assert e(448, 449, 464, 500, 1e30, np.inf) == [0x7E] * 6
    assert e(-448, -1e30, -np.inf) == [0xFE] * 3
    assert e(np.nan) == [0x7F]
    assert e(0.0, -0.0, -2.0 ** -11) == [0x00, 0x80, 0x80]


def test_encode_round_trips_every_finite_code():
    d = f8.e4m3_decode(CODES)
    ok = ~np.isnan(d)
    assert np.array_equal(f8.e4m3_encode(d[ok].astype(np.float32)), CODES[ok])


def test_rounding_error_within_half_a_step():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-12, 8, 100000))).astype(np.float32)
    x = x[np.abs(x) < 448]
    y = f8.e4m3_decode(f8.e4m3_encode(x))
    a = np.abs(x.astype(np.float64))
    # spacing of E4M3 values around a: 2^(e-3) for a normal with exponent e, 2^-9 below 2^-6
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(y - x) <= step / 2)


def test_absmax_scales_map_each_heads_largest_element_to_448():
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((3, 50, 64)).astype(np.float32)).to(torch.bfloat16)
    x[2].zero_()
    s = f8.kv_absmax_scales(x)
    assert s.dtype == np.float32 and s[2] == 1.0
    codes = f8.kv_quantize(x, s)
    xw = x.float().numpy()
    for g in range(2):
        i = np.unravel_index(np.abs(xw[g]).argmax(), xw[g].shape)
        assert codes[g][i] in (0x7E, 0xFE)
        assert np.abs(f8.e4m3_decode(codes[g])).max() == 448.0
    assert np.all(codes[2] == 0)
    # a code's value times the scale is within half a step of the input
    deq = f8.kv_dequantize(codes, s)
    assert np.all(np.abs(deq[:2] - xw[:2]) <= np.abs(xw[:2]) / 16 + s[:2, None, None] * 2.0 ** -10)


def test_kv8_decode_equals_plain_oracle_on_fp32_exact_values():
    """Power-of-two scales, different per head and between K and V, make every dequantised
    value an fp32 number: the E4M3 decode step must equal the plain fp32 oracle step on
    those values (a scale applied to the wrong head or tensor fails this)."""
    rng = np.random.default_rng(11)
    hq, hkv, L, d, lq = 8, 2, 300, 64, 5
    k8 = rng.integers(0, 256, (hkv, L, d)).astype(np.uint8)
    v8 = rng.integers(0, 256, (hkv, L, d)).astype(np.uint8)
    for c in (k8, v8):                               # no NaN codes in a cache
        c[(c & 0x7F) == 0x7F] ^= 1
    ks = np.float32([2.0 ** -6, 2.0 ** -4])
    vs = np.float32([2.0 ** 3, 2.0 ** -2])
    q = rng.standard_normal((hq, d)).astype(np.float32)
    kt = rng.standard_normal((hkv, lq, d)).astype(np.float32)
    vt = rng.standard_normal((hkv, lq, d)).astype(np.float32)
    bounds = [0, 100, 100, 300]
    o8, l8 = f8.phase2_decode_kv8(q, k8, v8, ks, vs, bounds, kt, vt, lq)
    kd = f8.kv_dequantize(k8, ks).astype(np.float32)
    vd = f8.kv_dequantize(v8, vs).astype(np.float32)
    assert np.array_equal(kd.astype(np.float64), f8.kv_dequantize(k8, ks))
    o, l = oracle.phase2_decode(q, kd, vd, bounds, kt, vt, lq)
    np.testing.assert_allclose(o8, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l8, l, rtol=1e-14, atol=0)
    # swapping the two kv heads' K scales changes the result
    o_sw, _ = f8.phase2_decode_kv8(q, k8, v8, ks[::-1].copy(), vs, bounds, kt, vt, lq)
    assert np.abs(o_sw - o).max() > 1e-3


@pytest.mark.parametrize("scale", [None, 0.125])
def test_kv8_decode_against_dense_softmax(scale):
    """Brute force on a tiny case: the dequantised context plus the tail, one dense softmax."""
    rng = np.random.default_rng(17)
    hq, hkv, L, d, lq = 4, 2, 40, 16, 3
    k8 = rng.integers(0, 0x7E, (hkv, L, d)).astype(np.uint8) | (rng.integers(0, 2, (hkv, L, d)) << 7).astype(np.uint8)
    v8 = rng.integers(0, 0x7E, (hkv, L, d)).astype(np.uint8)
    ks, vs = np.float32([0.01, 0.02]), np.float32([0.03, 0.005])
    q = rng.standard_normal((hq, d)).astype(np.float32)
    kt = rng.standard_normal((hkv, lq, d)).astype(np.float32)
    vt = rng.standard_normal((hkv, lq, d)).astype(np.float32)
    o8, l8 = f8.phase2_decode_kv8(q, k8, v8, ks, vs, [0, 17, 40], kt, vt, lq, scale=scale)
    sc = 1 / np.sqrt(d) if scale is None else scale
    G = hq // hkv
    for h in range(hq):
        g = h // G
        keys = np.concatenate([float(ks[g]) * f8.e4m3_decode(k8[g]), kt[g].astype(np.float64)])
        vals = np.concatenate([float(vs[g]) * f8.e4m3_decode(v8[g]), vt[g].astype(np.float64)])
        x = sc * keys @ q[h].astype(np.float64)
        w = np.exp(x - x.max())
        np.testing.assert_allclose(o8[h], w @ vals / w.sum(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(l8[h], x.max() + np.log(w.sum()), rtol=1e-13)


def test_kv8_query_equals_plain_oracle_on_fp32_exact_values():
    """Power-of-two scales (different per head and between K and V) make the dequantised
    context fp32-exact: the E4M3 query phase must equal the plain oracle's query phase on
    those values, and swapping the heads' V scales must change it."""
    rng = np.random.default_rng(19)
    hq, hkv, L, d, lq = 8, 2, 260, 32, 7
    k8 = rng.integers(0, 256, (hkv, L, d)).astype(np.uint8)
    v8 = rng.integers(0, 256, (hkv, L, d)).astype(np.uint8)
    for c in (k8, v8):
        c[(c & 0x7F) == 0x7F] ^= 1
    ks = np.float32([2.0 ** -5, 2.0 ** -3])
    vs = np.float32([2.0 ** 2, 2.0 ** -1])
    q = rng.standard_normal((hq, lq, d)).astype(np.float32)
    kt = rng.standard_normal((hkv, lq, d)).astype(np.float32)
    vt = rng.standard_normal((hkv, lq, d)).astype(np.float32)
    bounds = [0, 90, 90, 260]
    o8, l8 = f8.phase2_query_kv8(q, k8, v8, ks, vs, bounds, kt, vt, lq)
    kd = f8.kv_dequantize(k8, ks).astype(np.float32)
    vd = f8.kv_dequantize(v8, vs).astype(np.float32)
    o, l = oracle.phase2_query(q, kd, vd, bounds, kt, vt)
    np.testing.assert_allclose(o8, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l8, l, rtol=1e-14, atol=0)
    o_sw, _ = f8.phase2_query_kv8(q, k8, v8, ks, vs[::-1].copy(), bounds, kt, vt, lq)
    assert np.abs(o_sw - o).max() > 1e-3


def test_kv8_query_rows_after_cached_tokens_against_dense_softmax():
    """Brute force: query rows that are the last 3 of 8 cached tokens see the whole
    dequantised context and the cache causally (row i up to position 5 + i), one dense
    softmax per row."""
    rng = np.random.default_rng(23)
    hq, hkv, L, d, rows, tail_len, cap = 6, 3, 30, 16, 3, 8, 11
    k8 = rng.integers(0, 0x7E, (hkv, L, d)).astype(np.uint8) | (rng.integers(0, 2, (hkv, L, d)) << 7).astype(np.uint8)
    v8 = rng.integers(0, 0x7E, (hkv, L, d)).astype(np.uint8) | (rng.integers(0, 2, (hkv, L, d)) << 7).astype(np.uint8)
    ks, vs = np.float32([0.01, 0.02, 0.004]), np.float32([0.03, 0.005, 0.1])
    q = rng.standard_normal((hq, rows, d)).astype(np.float32)
    kt = rng.standard_normal((hkv, cap, d)).astype(np.float32)
    vt = rng.standard_normal((hkv, cap, d)).astype(np.float32)
    o8, l8 = f8.phase2_query_kv8(q, k8, v8, ks, vs, [0, 11, 30], kt, vt, tail_len)
    sc = 1 / np.sqrt(d)
    G = hq // hkv
    for h in range(hq):
        g = h // G
        for i in range(rows):
            vis = tail_len - rows + i + 1
            keys = np.concatenate([float(ks[g]) * f8.e4m3_decode(k8[g]), kt[g, :vis].astype(np.float64)])
            vals = np.concatenate([float(vs[g]) * f8.e4m3_decode(v8[g]), vt[g, :vis].astype(np.float64)])
            x = sc * keys @ q[h, i].astype(np.float64)
            w = np.exp(x - x.max())
            np.testing.assert_allclose(o8[h, i], w @ vals / w.sum(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(l8[h, i], x.max() + np.log(w.sum()), rtol=1e-13)


@pytest.mark.parametrize("off", [-1, 3])
def test_kv8_partial_equals_plain_oracle_on_fp32_exact_values(off):
    """Power-of-two scales: the E4M3 partial over tokens [lo, hi) equals the plain partial on
    the exact dequantised values, with and without a causal offset; swapping the heads' K
    scales changes it."""
    rng = np.random.default_rng(29)
    hq, hkv, T, d, rows, lo, hi = 4, 2, 150, 32, 6, 20, 140
    k8 = rng.integers(0, 256, (hkv, T, d)).astype(np.uint8)
    v8 = rng.integers(0, 256, (hkv, T, d)).astype(np.uint8)
    for c in (k8, v8):
        c[(c & 0x7F) == 0x7F] ^= 1
    ks = np.float32([2.0 ** -6, 2.0 ** -2])
    vs = np.float32([2.0 ** 1, 2.0 ** -3])
    q = rng.standard_normal((hq, rows, d)).astype(np.float32)
    a8, m8, l8 = f8.partial_kv8(q, k8, v8, ks, vs, lo, hi, off)
    kd = f8.kv_dequantize(k8, ks).astype(np.float32)
    vd = f8.kv_dequantize(v8, vs).astype(np.float32)
    a, m, l = oracle.partial(q, kd, vd, lo, hi, off)
    np.testing.assert_allclose(a8, a, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m8, m, rtol=1e-14, atol=0)
    np.testing.assert_allclose(l8, l, rtol=1e-13, atol=0)
    a_sw, _, _ = f8.partial_kv8(q, k8, v8, ks[::-1].copy(), vs, lo, hi, off)
    assert np.abs(a_sw - a).max() > 1e-3


def test_kv8_partial_against_brute_force():
    """Tiny case, one row at a time: A is the softmax-weighted mean of the dequantised values
    over the visible tokens, m their largest scaled score and l the sum of exp(score - m)."""
    rng = np.random.default_rng(31)
    hq, hkv, T, d, rows, lo, hi, off = 4, 2, 25, 16, 3, 5, 21, 7
    k8 = rng.integers(0, 0x7E, (hkv, T, d)).astype(np.uint8) | (rng.integers(0, 2, (hkv, T, d)) << 7).astype(np.uint8)
    v8 = rng.integers(0, 0x7E, (hkv, T, d)).astype(np.uint8)
    ks, vs = np.float32([0.02, 0.007]), np.float32([0.05, 0.3])
    q = rng.standard_normal((hq, rows, d)).astype(np.float32)
    a8, m8, l8 = f8.partial_kv8(q, k8, v8, ks, vs, lo, hi, off)
    sc = 1 / np.sqrt(d)
    G = hq // hkv
    for h in range(hq):
        g = h // G
        for i in range(rows):
            toks = [t for t in range(lo, hi) if t - lo <= off + i]
            keys = float(ks[g]) * f8.e4m3_decode(k8[g, toks])
            vals = float(vs[g]) * f8.e4m3_decode(v8[g, toks])
            x = sc * keys @ q[h, i].astype(np.float64)
            w = np.exp(x - x.max())
            np.testing.assert_allclose(a8[h, i], w @ vals / w.sum(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(m8[h, i], x.max(), rtol=1e-13)
            np.testing.assert_allclose(l8[h, i], w.sum(), rtol=1e-13)
