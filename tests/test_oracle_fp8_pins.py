"""Pins of the oracle's FP8 prefix-cache functions (CPU only).

The E4M3 codec is pinned to the format's definition by closed-form values of chosen codes,
brute force over all 256 codes, and tie cases; the per-(token, head) quantisation by its error
bound and exactness cases; the cache-size function by the pages' "V-only saves about 25%".
Planted mistakes in a copy of the codec (wrong bias, ties away from zero, no subnormals) are
caught.
"""
import numpy as np
import pytest

import bca_workloads as W
from oracle import bca_oracle as O


def finite_codes():
    return [c for c in range(256) if not np.isnan(O.e4m3_value_table()[c])]


def brute_encode(x, table):
    """Nearest finite value over the whole table; ties to the even code; saturating."""
    fin = [c for c in range(256) if not np.isnan(table[c])]
    best = None
    for c in fin:
        d = abs(table[c] - x)
        key = (d, c & 1, c)  # nearest, then even code, then a fixed order
        if best is None or key < best[0]:
            best = (key, c)
    code = best[1]
    if abs(x) > 448:
        code = 0x7E | (0x80 if x < 0 else 0)
    if table[code] == 0 and x < 0:
        code = 0x80
    return code


def check_table(table):
    assert table[0x38] == 1.0                        # exponent field 7 = bias, mantissa 0
    assert table[0x7E] == 448.0                      # largest finite: 1.75 * 2^8
    assert table[0x08] == 2.0 ** -6                  # smallest normal
    assert table[0x01] == 2.0 ** -9                  # smallest subnormal
    assert table[0x07] == 7 * 2.0 ** -9              # largest subnormal
    assert np.isnan(table[0x7F]) and np.isnan(table[0xFF])
    assert table[0x80] == 0.0 and np.signbit(table[0x80])
    pos = table[:0x7F]
    assert (np.diff(pos) > 0).all() and len(pos) == 127
    assert np.array_equal(table[0x80:0xFF], -pos)


def check_encoder(encode, table):
    for c in finite_codes():
        if c == 0x80:
            continue
        assert encode(np.array([table[c]]))[0] == c, hex(c)
    pos = table[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    got = encode(mids)
    for i, g in enumerate(got):
        want = i if i % 2 == 0 else i + 1          # the even one of codes i, i + 1
        assert g == want, (i, mids[i], g)
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.normal(0, 30, 300), rng.normal(0, 0.01, 200), [500, -1e6, 448.5]])
    got = encode(xs)
    for x, g in zip(xs, got):
        assert g == brute_encode(x, table), (x, g)


def test_e4m3_table():
    check_table(O.e4m3_value_table())


def test_e4m3_encoder():
    check_encoder(O.e4m3_encode, O.e4m3_value_table())


def brute_scale(amax):
    """The smallest power of two 2^k, k >= -126, with amax <= 448 * 2^k, by a search in exact
    rational arithmetic (1 for amax = 0)."""
    from fractions import Fraction
    a = Fraction(float(amax))
    if a == 0:
        return 1.0
    k = -126
    while a > 448 * Fraction(2) ** k:
        k += 1
    return float(Fraction(2) ** k)


def test_quantize_rows_error_bound_and_scale():
    rng = np.random.default_rng(4)
    x = W.bf16_bits_to_f32(W.draw_bf16(rng, (3, 50, 2, 128), scaled=False))
    codes, scales = O.quantize_fp8_rows(x)
    assert scales.dtype == np.float32 and scales.shape == (3, 50, 2)
    amax = np.abs(x).max(axis=-1)
    want = np.array([brute_scale(a) for a in amax.ravel()], np.float32).reshape(amax.shape)
    np.testing.assert_array_equal(scales, want)
    # the element that attains amax lands in E4M3's top binade: no range is wasted
    top = O.e4m3_decode(codes).__abs__().max(axis=-1)
    assert ((top >= 224.0) & (top <= 448.0)).all()
    back = O.dequantize_fp8_rows(codes, scales)
    # 3 mantissa bits: half an ulp is 1/16 relative for normal values; subnormal steps are
    # 2^-9 * scale absolute
    err = np.abs(back - x)
    bound = np.maximum(np.abs(x) / 16, 2.0 ** -10 * scales[..., None]) * (1 + 1e-6)
    assert (err <= bound).all()


def test_quantize_exact_values_roundtrip():
    """Rows whose values are already E4M3 values times a power of two come back exactly."""
    rng = np.random.default_rng(5)
    table = O.e4m3_value_table()
    fin = np.array([table[c] for c in finite_codes()])
    rows = rng.choice(fin, size=(4, 128))
    rows[:, 0] = 448.0                              # amax 448 -> scale 1
    rows = rows * 2.0 ** rng.integers(-3, 4, size=(4, 1))
    codes, scales = O.quantize_fp8_rows(rows.astype(np.float32))
    np.testing.assert_array_equal(O.dequantize_fp8_rows(codes, scales), rows)
    zc, zs = O.quantize_fp8_rows(np.zeros((2, 128), np.float32))
    assert (zs == 1.0).all() and (O.e4m3_decode(zc) == 0).all()


def test_cache_size_v_only_saves_about_a_quarter():
    bf16 = O.prefix_cache_bytes_fp8(32, 1, 4096, 32, 128, O.CACHE_BF16)
    v_only = O.prefix_cache_bytes_fp8(32, 1, 4096, 32, 128, O.CACHE_FP8_V)
    kv = O.prefix_cache_bytes_fp8(32, 1, 4096, 32, 128, O.CACHE_FP8_KV)
    assert bf16 == O.prefix_cache_bytes(32, 1, 4096, 32, 128, 2) == 2 * 2 ** 30
    assert abs((1 - v_only / bf16) - 0.25) < 0.01   # "about 25%"
    assert kv < v_only < bf16


def test_decode_cached_equals_decode_on_exact_cache():
    """With every cached value exactly representable, the FP8 decode is the plain decode."""
    rng = np.random.default_rng(6)
    ids = W.TINY.block_ids()
    P, N, _ = O.prefix_split(ids)
    table = O.e4m3_value_table()
    fin = np.array([table[c] for c in finite_codes()])
    k = rng.choice(fin, size=(1, 146, 2, 128)) / 64.0
    v = rng.choice(fin, size=(1, 146, 2, 128)) / 64.0
    k[..., 0] = 448.0 / 64.0
    v[..., 0] = 448.0 / 64.0                        # per-row amax 7 -> scale 1/64 exactly
    q = rng.standard_normal((1, 146, 2, 128))
    ref = O.decode(q[:, P:], k[:, :P], v[:, :P], k[:, P:], v[:, P:])
    for fmt in (O.CACHE_FP8_V, O.CACHE_FP8_KV):
        cache = O.prefix_cache_fp8(k.astype(np.float32), v.astype(np.float32), ids, fmt)
        got = O.decode_cached(q[:, P:], cache, k[:, P:], v[:, P:])
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------------------------
def _table_bias8():
    t = O.e4m3_value_table().copy()
    return t / 2.0


def _table_no_subnormals():
    t = O.e4m3_value_table().copy()
    for c in range(256):
        if (c >> 3) & 0xF == 0:
            t[c] = 0.0 * (-1 if c & 0x80 else 1)
    return t


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    pos = O.e4m3_value_table()[:0x7F]
    a = np.abs(x)
    hi = np.clip(np.searchsorted(pos, a), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    code = np.where(np.abs(pos[hi] - a) <= np.abs(a - pos[lo]), hi, lo).astype(np.uint8)
    code = np.where(a > 448, np.uint8(0x7E), code)
    return np.where(x < 0, code | 0x80, code).astype(np.uint8)


@pytest.mark.parametrize("bad_table", [_table_bias8, _table_no_subnormals])
def test_planted_table_mistakes_are_caught(bad_table):
    with pytest.raises(AssertionError):
        check_table(bad_table())


def test_planted_rounding_mistake_is_caught():
    with pytest.raises(AssertionError):
        check_encoder(_encode_ties_away, O.e4m3_value_table())


def test_quantize_tiny_rows_keep_a_normal_scale():
    """Rows of tiny values: the scale stays a normal fp32 number, its reciprocal finite, no
    code is NaN, and every value comes back within half a step of the coarsest grid."""
    x = np.zeros((4, 128), np.float32)
    x[0, :3] = [2.0 ** -130, -2.0 ** -128, 2.0 ** -133]      # bf16 subnormals
    x[1, 5] = 2.0 ** -118                                    # amax / 448 = 2^-126.8
    x[2, 7] = 448 * 2.0 ** -126                              # exactly at the floor
    x[3, :] = 2.0 ** -100                                    # well above it
    codes, scales = O.quantize_fp8_rows(x)
    assert (scales >= np.float32(2.0 ** -126)).all()
    assert np.isfinite(np.float32(1) / scales).all()
    assert not np.isnan(O.e4m3_decode(codes)).any()
    assert scales[1] == np.float32(2.0 ** -126) and scales[2] == np.float32(2.0 ** -126)
    assert scales[3] == np.float32(2.0 ** -108)              # 2^-100 / 448 = 2^-108.8
    back = O.dequantize_fp8_rows(codes, scales)
    step = 2.0 ** -9 * scales[:, None].astype(np.float64)    # finest E4M3 step times the scale
    assert (np.abs(back - x) <= np.maximum(np.abs(x) / 16, step / 2)).all()
    nz = back != 0
    assert (np.sign(back[nz]) == np.sign(x[nz])).all()


@pytest.mark.parametrize("amax", [448.0, 448.0 * 2.0 ** 5, 448.0 * 2.0 ** -7, np.nextafter(448.0, 1e9),
                                  np.nextafter(448.0, 0), 224.0, 224.5, 1.0, 7.0, 3.0e38,
                                  2.0 ** -118, 2.0 ** -133, 448 * 2.0 ** -126, 0.0])
def test_scale_is_the_smallest_power_of_two_in_range(amax):
    """Edge amax values: exactly 448 times a power of two, one fp32 ulp either side of one, the
    top of the fp32 range, values at and below the floor, zero."""
    a = np.float32(amax)
    got = O.fp8_row_scale(np.array([a]))[0]
    assert got == np.float32(brute_scale(a))
    if a > 448 * 2.0 ** -126:
        assert 224 < float(a) / float(got) <= 448            # the top binade of E4M3


def test_planted_scale_mistake_is_caught():
    """A scale one power of two too large (amax / 448 rounded up twice) fails the scale pin."""
    rng = np.random.default_rng(8)
    amax = np.abs(rng.normal(0, 3, 200)).astype(np.float32)
    wrong = (O.fp8_row_scale(amax) * 2).astype(np.float32)
    want = np.array([brute_scale(a) for a in amax], np.float32)
    assert not np.array_equal(wrong, want)
    np.testing.assert_array_equal(O.fp8_row_scale(amax), want)
