"""Pins of the FP8 (E4M3) oracle: values the format's definition fixes, and the
scaled append's rounding, independently of the encoder's search."""
import math

import numpy as np
import pytest

from oracle import fp8


def test_decode_table_closed_forms():
    t = fp8.DECODE_TABLE
    assert t[0x00] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0
    assert t[0x01] == 2.0 ** -9                       # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9                   # largest subnormal
    assert t[0x08] == 2.0 ** -6                       # smallest normal
    assert t[0x38] == 1.0 and t[0x39] == 1.125 and t[0x40] == 2.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0     # largest finite
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    finite = t[:0x7F]
    assert np.all(np.diff(finite) > 0)                # codes 0x00..0x7E increase
    assert np.array_equal(t[0x80:0xFF], -finite)      # sign bit


def test_every_finite_code_round_trips():
    for c in list(range(0x00, 0x7F)) + list(range(0x80, 0xFF)):
        assert fp8.encode_value(fp8.DECODE_TABLE[c]) == c, hex(c)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),        # halfway between 1 and 1.125: even mantissa (1.0)
    (1.1875, 0x3A),        # halfway between 1.125 and 1.25: even mantissa (1.25)
    (1.06, 0x38), (1.07, 0x39),
    (0.5 * 2.0 ** -9, 0x00), (0.75 * 2.0 ** -9, 0x01), (1.5 * 2.0 ** -9, 0x02),
    (15.5 * 2.0 ** -10, 0x08),  # 7.75 * 2^-9 rounds up into the first normal
    (464.0, 0x7E), (1e30, 0x7E), (math.inf, 0x7E), (-math.inf, 0xFE), (-500.0, 0xFE),
    (-0.0, 0x80), (0.0, 0x00),
])
def test_encode_points(x, code):
    assert fp8.encode_value(x) == code


def test_nan_encodes_to_0x7f():
    assert fp8.encode_value(math.nan) == 0x7F


def test_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(2000) * 40, rng.standard_normal(500) * 0.01])
    finite = fp8.DECODE_TABLE[:0x7F]
    for x in xs:
        c = fp8.encode_value(float(x))
        v = fp8.DECODE_TABLE[c]
        best = np.min(np.abs(np.abs(x) - finite))
        assert abs(abs(x) - abs(v)) == best or abs(x) >= 448
        assert (c & 0x80 != 0) == (x < 0)


def test_quantize_uses_one_fp32_product():
    """The append's product is rounded to fp32 before encoding: 1.0625 is exactly
    halfway in E4M3, and x * (1/3) lands on either side of it depending on that rounding."""
    x = np.float32(3.1875)
    inv = np.float32(1.0) / np.float32(3.0)
    prod = np.float32(x * inv)
    assert fp8.quantize_for_append(np.array([x]), 3.0)[0] == fp8.encode_value(float(prod))


def test_fp8_decode_reduces_to_plain_attention():
    """With codes that are exact small integers and unit scales, decode_fp8 equals the
    16-bit oracle fed the same values."""
    from oracle import attention
    from workloads import f32_to_bits
    rng = np.random.default_rng(3)
    N, Hkv, bs, D, Hq = 4, 2, 16, 64, 4
    codes_k = rng.integers(0x30, 0x48, size=(N, Hkv, bs, D)).astype(np.uint8)
    codes_v = rng.integers(0xB0, 0xC8, size=(N, Hkv, bs, D)).astype(np.uint8)
    q = f32_to_bits(rng.standard_normal((2, Hq, D)).astype(np.float32), "bf16")
    tables = np.array([[2, 0], [1, 3]])
    lens = np.array([20, 31])
    got = fp8.decode(q, codes_k, codes_v, 1.0, 1.0, tables, lens, 0.125, q_dtype="bf16", num_blocks=N,
                     num_kv_heads=Hkv, block_size=bs)
    kb = f32_to_bits(fp8.DECODE_TABLE[codes_k].astype(np.float32), "bf16")   # exact: E4M3 fits in bf16
    vb = f32_to_bits(fp8.DECODE_TABLE[codes_v].astype(np.float32), "bf16")
    ref = attention.decode(q, kb.ravel(), vb.ravel(), tables, lens, 0.125, dtype="bf16", num_blocks=N,
                           num_kv_heads=Hkv, block_size=bs)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    # and the scales multiply through: K scale into the scores, V scale into the output
    got2 = fp8.decode(q, codes_k, codes_v, 2.0, 0.5, tables, lens, 0.0625, q_dtype="bf16", num_blocks=N,
                      num_kv_heads=Hkv, block_size=bs)
    assert np.allclose(got2, 0.5 * ref, rtol=1e-12, atol=1e-12)


def test_append_scatters_codes_and_leaves_the_rest():
    from workloads import f32_to_bits
    rng = np.random.default_rng(1)
    N, Hkv, bs, D = 3, 2, 16, 8
    k = f32_to_bits(rng.standard_normal((4, Hkv, D)).astype(np.float32) * 5, "bf16")
    v = f32_to_bits(rng.standard_normal((4, Hkv, D)).astype(np.float32) * 5, "bf16")
    kp = np.full((N, Hkv, bs, D), 0x55, dtype=np.uint8)
    vp = kp.copy()
    slots = np.array([17, -1, 2, 47])
    fp8.append(k, v, "bf16", slots, kp, vp, 0.5, 2.0, num_blocks=N, block_size=bs)
    from oracle.numerics import bits_to_f64
    for t, s in enumerate(slots):
        if s < 0:
            continue
        n, off = divmod(int(s), bs)
        # 16-bit inputs times a power-of-two inverse scale are exact in fp32, so the codes are
        # the nearest codes to x / scale
        assert np.array_equal(kp[n, :, off], fp8.encode(bits_to_f64(k[t], "bf16") / 0.5))
        assert np.array_equal(vp[n, :, off], fp8.encode(bits_to_f64(v[t], "bf16") / 2.0))
    touched = {(int(s) // bs, int(s) % bs) for s in slots if s >= 0}
    for n in range(N):
        for off in range(bs):
            if (n, off) not in touched:
                assert np.all(kp[n, :, off] == 0x55) and np.all(vp[n, :, off] == 0x55)


def test_array_encode_matches_the_scalar_definition():
    """encode (all elements at once) against encode_value one by one: every code's value,
    every midpoint between neighbouring codes and a little either side of it, random
    values over the whole range, and the special values."""
    finite = fp8.DECODE_TABLE[:0x7F]
    mids = (finite[1:] + finite[:-1]) / 2
    rng = np.random.default_rng(3)
    xs = np.concatenate([finite, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                         rng.standard_normal(3000) * 50, rng.standard_normal(1000) * 1e-3,
                         [448.0, 464.0, 479.9, 480.0, 1e30, math.inf, -math.inf, math.nan, -math.nan, 0.0, -0.0]])
    xs = np.concatenate([xs, -xs])
    want = np.array([fp8.encode_value(float(v)) for v in xs], dtype=np.uint8)
    got = fp8.encode(xs.reshape(2, -1)).ravel()
    assert np.array_equal(got, want), xs[got != want][:8]
