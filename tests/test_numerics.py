"""Host checks of numerical claims that the GPU parity tests lean on (no GPU needed).

The 8-bit cached decode state re-scales every state row by s = m / 127 (m the row's largest
magnitude).  The kernel forms that quotient without a division instruction: with
y = binary32(1/127), q0 = RN(m y), r = fma(-q0, 127, m) (exact: the residual of a quotient within
an ulp) and s = fma(r, y, q0).  The GPU test of the 8-bit state bounds the scale's difference
from the oracle's on the assumption that this sequence is the correctly rounded binary32(m / 127)
for every normal m.  Here that assumption is checked for every binary32 significand: the
sequence commutes with scaling m by a power of two as long as every intermediate stays normal,
so one binade of m, [1, 2), covers every normal m whose scale is normal.  All arithmetic below is
exact integer arithmetic on significands."""
import numpy as np

I64 = np.int64


def _bitlen(v: np.ndarray) -> np.ndarray:
    """Bit length of positive int64 values (exact)."""
    e = np.frexp(v.astype(np.float64))[1].astype(I64)     # within one of the true length
    e = np.where(v >= (I64(1) << np.minimum(e, 62)), e + 1, e)
    e = np.where(v < (I64(1) << np.maximum(e - 1, 0)), e - 1, e)
    return e


def _round_sig24(v: np.ndarray, sticky: np.ndarray):
    """Round positive integers v (plus a sticky bit below them) to 24 significant bits, ties to
    even: returns (significand in [2^23, 2^24], shift) with the value significand * 2^shift."""
    n = _bitlen(v)
    sh = np.maximum(n - 24, 0)
    q = v >> sh
    rem = v - (q << sh)
    half = np.where(sh > 0, I64(1) << np.maximum(sh - 1, 0), 0)
    up = (sh > 0) & ((rem > half) | ((rem == half) & (sticky | ((q & 1) == 1))))
    q = q + up.astype(I64)
    return q, sh


def _as_pair(sig, sh, base_exp):
    """Normalize (sig * 2^(sh + base_exp)) to a 24-bit significand and exponent."""
    over = sig >= (I64(1) << 24)
    sig = np.where(over, sig >> 1, sig)
    return sig, sh + base_exp + over.astype(I64)


def test_row_scale_division_sequence_is_correctly_rounded():
    M = np.arange(1 << 23, 1 << 24, dtype=I64)                # m = M 2^-23 in [1, 2)
    zero = np.zeros(M.shape, bool)
    # y = binary32(1/127): 2^30 / 127 rounded to 24 bits
    Y, ysh = _round_sig24(np.array([I64(1) << 40]) // 127, np.array([(I64(1) << 40) % 127 != 0]))
    Y, ey = int(Y[0]), int(ysh[0]) - 40                      # y = Y 2^ey
    assert abs(Y * 2.0 ** ey - 1 / 127) <= 2.0 ** (ey - 1)
    # q0 = RN(m y): exact product M Y 2^(ey - 23)
    q0s, q0sh = _round_sig24(M * I64(Y), zero)
    q0s, q0e = _as_pair(q0s, q0sh, ey - 23)                   # q0 = q0s 2^q0e
    # r = m - 127 q0, exact in units of 2^q0e (m = M 2^-23 with -23 >= q0e)
    R = (M << (-23 - q0e)) - 127 * q0s
    assert np.all(np.abs(R) < (I64(1) << 24))                # representable: the fma result is exact
    # s = RN(q0 + r y), exact sum in units of 2^(q0e + ey): q0s 2^-ey + R Y
    S = (q0s << (-ey)) + R * I64(Y)
    assert np.all(S > 0)
    ss, ssh = _round_sig24(S, zero)
    ss, se = _as_pair(ss, ssh, q0e + ey)
    # the correctly rounded binary32(m / 127): M 2^10 / 127 with its remainder as a sticky bit
    num = M << 10
    ts, tsh = _round_sig24(num // 127, num % 127 != 0)
    ts, te = _as_pair(ts, tsh, -33)
    # equal as numbers (both normalized to 24-bit significands)
    assert np.array_equal(ss, ts) and np.array_equal(se, te)


def test_exact_integer_rounding_helper():
    """The helper itself against binary32 conversions of exactly representable float64 values."""
    rng = np.random.default_rng(5)
    v = rng.integers(1, 1 << 52, size=200_000, dtype=I64)
    sig, sh = _round_sig24(v, np.zeros(v.shape, bool))
    got = sig.astype(np.float64) * np.exp2(sh.astype(np.float64))
    want = v.astype(np.float64).astype(np.float32).astype(np.float64)   # v exact in float64
    assert np.array_equal(got, want)
