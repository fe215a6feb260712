"""Pins for the oracle's static INT8 quantizer (CPU only).

The quantizer is the one the 8-bit SSD inputs use (Quamba2 rebuttal, "impact of
SSD quantization": x, B, C quantized; SSDi8 Table 10: per-head scale for x,
per-group for B and C): code = saturate_127(round_half_even(fp32(v) / s)),
with the fp32 quotient correctly rounded.  The pins below do not re-run that
formula: they derive codes from exact rational arithmetic, from hand-worked
ties, and from invariants that any correct implementation must satisfy.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

ALL_F16 = np.arange(65536, dtype=np.uint16).view(np.float16)


def _round_to_f32(t: Fraction) -> Fraction | float:
    """Correct rounding (nearest, ties to even) of an exact rational to binary32,
    done with integers only."""
    if t == 0:
        return Fraction(0)
    sign = -1 if t < 0 else 1
    a = abs(t)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum_exp = max(e, -126) - 23
    m = a / Fraction(2) ** quantum_exp
    m_int = round(m)  # Fraction.__round__ rounds half to even
    val = m_int * Fraction(2) ** quantum_exp
    if val >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * val


def _exact_code(v: float, s: float) -> int:
    if np.isnan(v):
        return 0
    if np.isinf(v):
        return 127 if v > 0 else -127
    q = _round_to_f32(Fraction(float(v)) / Fraction(float(s)))
    if isinstance(q, float):  # overflowed to +-inf
        return 127 if q > 0 else -127
    r = round(q)  # half to even
    return int(max(-127, min(127, r)))


@pytest.mark.parametrize("scale", [np.float32(0.3), np.float32(1.0) / np.float32(127.0)])
def test_every_f16_against_exact_rationals(scale):
    # 0.3 is a scale where v * (1/s) and v / s round to different codes for 12 inputs,
    # so this catches a reciprocal-multiply shortcut as well as a wrong rounding rule.
    codes = oracle.quantize_values(ALL_F16, float(scale))
    vals = ALL_F16.astype(np.float64)
    expect = np.array([_exact_code(v, float(scale)) for v in vals], dtype=np.int8)
    bad = np.nonzero(codes != expect)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first at {vals[bad[:5]]}: {codes[bad[:5]]} vs {expect[bad[:5]]}"


# (value, scale, code): hand-derived from the rounding rule and the saturation bound.
HAND_CASES = [
    (2.5, 1.0, 2),        # tie -> even
    (3.5, 1.0, 4),        # tie -> even
    (-2.5, 1.0, -2),      # tie -> even, symmetric
    (0.5, 1.0, 0),        # tie -> even (0)
    (1.5, 1.0, 2),
    (126.5, 1.0, 126),    # tie -> even inside the range
    (127.5, 1.0, 127),    # rounds to 128, saturates
    (-127.5, 1.0, -127),  # rounds to -128, saturates: -128 is never produced
    (-200.0, 1.0, -127),
    (10000.0, 1.0, 127),
    (1.25, 0.5, 2),       # 1.25 / 0.5 = 2.5 exactly -> 2
    (7.5, 3.0, 2),        # 7.5 / 3 = 2.5 exactly -> 2
    (4.5, 3.0, 2),        # 1.5 -> 2
    (0.0, 0.25, 0),
    (-0.0, 0.25, 0),
    (0.1, 0.25, 0),       # 0.39990234375 -> 0
    (float("inf"), 1.0, 127),
    (float("-inf"), 1.0, -127),
    (float("nan"), 1.0, 0),
    (65504.0, 2.0 ** -20, 127),   # fp16 max over a tiny scale saturates
    (2.0 ** -24, 2.0 ** -20, 0),  # smallest subnormal: 1/16 -> 0
]


@pytest.mark.parametrize("v,s,code", HAND_CASES)
def test_hand_cases(v, s, code):
    got = oracle.quantize_values(np.array([v], dtype=np.float16), s)
    assert int(got[0]) == code


@pytest.mark.parametrize("scale", [1.0, 0.5, 1.0 / 127.0, 3.0, 0.0123, 2.0 ** -20])
def test_invariants_all_f16(scale):
    q = oracle.quantize_values(ALL_F16, scale).astype(np.int32)
    v = ALL_F16.astype(np.float64)
    fin = np.isfinite(v)
    # range: never -128
    assert q.min() >= -127 and q.max() <= 127
    # odd symmetry: q(-v) = -q(v)  (the sign bit is bit 15)
    neg = (np.arange(65536, dtype=np.uint32) ^ 0x8000).astype(np.int64)
    assert np.array_equal(q[neg], -q)
    # monotone non-decreasing in v over the finite values
    order = np.argsort(v[fin], kind="stable")
    assert np.all(np.diff(q[fin][order]) >= 0)
    # unsaturated codes are within half a step of v / s
    inside = fin & (np.abs(q) < 127)
    assert np.all(np.abs(q[inside] - v[inside] / np.float32(scale)) <= 0.5 + 1e-6)


def test_tensor_layout_uses_per_head_scale():
    # x viewed as (rows, heads, headdim): head k must use scale[k]
    x = np.full((3, 4, 5), 10.0, dtype=np.float16)
    s = np.array([1.0, 2.0, 4.0, 0.5], dtype=np.float32)
    q = oracle.quantize(x, s)
    assert np.array_equal(q[0, :, 0], np.array([10, 5, 2, 20], dtype=np.int8))  # 2.5 -> 2
    assert np.all(q == q[0:1])
