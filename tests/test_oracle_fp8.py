"""Pins of the oracle's FP8 cache codec (OCP 8-bit floating point, E4M3).

The pages say inference runs in FP8 but do not define the format; the oracle
takes the OCP E4M3 definition (bias 7, 3 mantissa bits, no infinities, NaN =
S.1111.111, largest finite 448).  These pins fix it from that definition and
from arithmetic independent of the oracle's own code:
  - code values printed in the definition (1.0, 448, the smallest subnormal
    and normal values, the NaN codes);
  - the shape of the value table (126 positive finite values, increasing);
  - round trips code -> value -> code;
  - every tie (each midpoint between neighbouring values) goes to the even
    code, and points just off each midpoint go to the nearer value;
  - agreement with an exponent/mantissa rounding written here (not a table
    search) on random values from the subnormals to past saturation;
  - saturation of finite overflow and of infinities to +-448;
  - the quantizer divides by the scale (round trip through a scale).
Planted mistakes in a copy of the codec must each fail a pin.
"""
import inspect

import numpy as np
import pytest

import oracle


def independent_encode(x):
    """Nearest-even E4M3 by exponent/mantissa arithmetic, saturating."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)  # 8 lands on code 0x08
    f, ex = np.frexp(np.where(sub, 1.0, a))
    e = ex - 1                                    # a = 2^e * (1 + mant)
    q = np.rint((np.ldexp(np.where(sub, 1.0, a), -e) - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    normal_code = ((e + 7) << 3) | q
    code = np.where(sub, code, normal_code)
    code = np.where((a >= 448.0) | (code > 0x7E), 0x7E, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def pin_known_codes(dec, enc, quant):
    t = dec(np.arange(256))
    known = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0x01: 2.0 ** -9,
             0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in known.items():
        assert t[c] == v, (hex(c), t[c], v)
    assert np.signbit(t[0x80]) and t[0x80] == 0.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(np.delete(t, [0x7F, 0xFF])).all()


def pin_table_shape(dec, enc, quant):
    pos = dec(np.arange(0x7F))
    assert (np.diff(pos) > 0).all()
    assert pos[1] == 2.0 ** -9 and pos[-1] == 448.0
    assert np.array_equal(dec(np.arange(0x80, 0xFF)), -pos)


def pin_round_trip(dec, enc, quant):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(enc(dec(codes)), codes.astype(np.uint8))


def pin_ties_to_even(dec, enc, quant):
    pos = dec(np.arange(0x7F))
    mid = (pos[:-1] + pos[1:]) / 2          # exact in fp64
    c = np.arange(0x7E)
    even = np.where(c % 2 == 0, c, c + 1)
    assert np.array_equal(enc(mid), even.astype(np.uint8))
    assert np.array_equal(enc(-mid), (even | 0x80).astype(np.uint8))
    gap = pos[1:] - pos[:-1]
    assert np.array_equal(enc(mid - gap / 64), c.astype(np.uint8))
    assert np.array_equal(enc(mid + gap / 64), (c + 1).astype(np.uint8))


def pin_independent_rounding(dec, enc, quant):
    rng = np.random.default_rng(7)
    a = np.exp2(rng.uniform(-13.0, 9.5, 200_000)) * rng.choice([-1.0, 1.0], 200_000)
    assert np.array_equal(enc(a), independent_encode(a))


def pin_saturation(dec, enc, quant):
    big = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1e6, 1e300, np.inf])
    assert (enc(big) == 0x7E).all()
    assert (enc(-big) == 0xFE).all()


def pin_quantizer_divides(dec, enc, quant):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    for s in (0.0123, 3.5, 1.0):
        vals = (dec(codes) * np.float32(s)).astype(np.float32)
        assert np.array_equal(quant(vals, s), codes.astype(np.uint8)), s


ALL_PINS = [pin_known_codes, pin_table_shape, pin_round_trip, pin_ties_to_even,
            pin_independent_rounding, pin_saturation, pin_quantizer_divides]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_fp8_pin(pin):
    pin(oracle.fp8_e4m3_decode, oracle.fp8_e4m3_encode, oracle.fp8_quantize)


# ---------------------------------------------------------------------------- mutants

MUTATIONS = {
    "exponent_bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "subnormal_exponent": ("(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),
    "nan_on_whole_top_binade": ("(e == 15) & (m == 7)", "(e == 15)"),
    "ties_away_from_zero": ("np.where(lo % 2 == 0, lo, hi)", "hi"),
    "overflow_to_nan": ("pick = np.where(a >= _E4M3_TABLE[-1], len(_E4M3_TABLE) - 1, pick)",
                        "pick = np.where(a > _E4M3_TABLE[-1], len(_E4M3_TABLE), pick)"),
    "sign_dropped": ("np.where(np.signbit(x.ravel()), 0x80, 0)",
                     "np.where(np.signbit(x.ravel()), 0, 0)"),
    "quantizer_multiplies": ("np.asarray(x, dtype=np.float32) / np.float32(scale)",
                             "np.asarray(x, dtype=np.float32) * np.float32(scale)"),
}


def _fp8_section():
    src = inspect.getsource(oracle)
    start = src.index("def fp8_e4m3_decode")
    return src[start:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_fp8_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    sec = _fp8_section()
    assert sec.count(old) == 1, "mutation target not found: " + old
    ns = {"np": np}
    exec(compile(sec.replace(old, new), "<mutant %s>" % name, "exec"), ns)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(ns["fp8_e4m3_decode"], ns["fp8_e4m3_encode"], ns["fp8_quantize"])
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake " + name
