"""The quantize kernel's divide-free arithmetic, checked on the host.

The kernel takes s = range / d (d = 15 or 7 for INT4, 255 or 127 for W8) as
q1 = fma(fma(-q0, d, a), y, q0) with y = RN(1/d) and q0 = RN(a * y), and
claims q1 equals the IEEE quotient RN(a / d) for every fp32 a. A scale by a
power of two scales every step exactly (for normal values), so one binade of
significands covers every normal a; two binades are run here. numpy has no
fp32 fma, so each fma is taken exactly in fp64 and rounded once to fp32:
* the residual a - q0 d is exact in fp64 (at most 33 significant bits) and
  fits fp32 (checked), so the inner fma returns it unrounded;
* q0 + r y is exact in fp64 up to one rounding of the sum; a fp64 sum that
  lands exactly on a fp32 half-way point could round twice the wrong way,
  so those cases are redone in exact rational arithmetic.
"""

from fractions import Fraction

import numpy as np
import pytest

F32, F64 = np.float32, np.float64


def _fma32_exact(a, b, c):
    """RN32(a * b + c) for one fp32 triple, in exact rationals."""
    return F32(_round_to_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))))


def _round_to_f32(x):
    """Round a Fraction to the nearest fp32 value, ties to even."""
    lo = F32(float(x))                      # within one unit of x
    cands = [np.nextafter(lo, F32(-np.inf)), lo, np.nextafter(lo, F32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x),
                                     int(np.array(c, F32).view(np.uint32)) & 1))
    return best


def _div_const(a, d):
    """The kernel's q1 over an array of fp32 a (see the module docstring)."""
    y = F32(1) / F32(d)
    q0 = a * y                                            # RN32 product
    r64 = a.astype(F64) - q0.astype(F64) * F64(d)         # exact residual
    r = r64.astype(F32)
    assert np.array_equal(r.astype(F64), r64), "residual not representable in fp32"
    s64 = q0.astype(F64) + r.astype(F64) * F64(y)         # r*y exact; one fp64 rounding
    q1 = s64.astype(F32)
    # fp64 sums sitting exactly on a fp32 half-way point: redo exactly
    bits = s64.view(np.uint64)
    mid = (bits & np.uint64((1 << 29) - 1)) == np.uint64(1 << 28)
    for i in np.nonzero(mid)[0]:
        q1[i] = _fma32_exact(r[i], y, q0[i])
    return q1


@pytest.mark.parametrize("d", [7, 15, 127, 255])
@pytest.mark.parametrize("exponent", [127, 140])
def test_div_const_equals_ieee_quotient(d, exponent):
    sig = np.arange(1 << 23, dtype=np.uint32)
    a = ((np.uint32(exponent) << np.uint32(23)) | sig).view(F32)
    got = _div_const(a, d)
    want = a / F32(d)                                     # IEEE fp32 divide
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"d={d}: {bad.size} significands differ, first a={a[bad[0]]!r}"


def test_plain_product_is_not_enough():
    """The correction is needed: the bare product misses many quotients (so
    the check above can fail)."""
    sig = np.arange(1 << 23, dtype=np.uint32)
    a = ((np.uint32(127) << np.uint32(23)) | sig).view(F32)
    assert np.count_nonzero(a * (F32(1) / F32(15)) != a / F32(15)) > 1_000_000


def test_magic_rounding_is_rint_plus_base():
    """t = RN(x + 1.5 * 2^23 + z) puts rint(x) + z in the low bits of t for
    |x| well inside 2^22, away from half-way points (the kernel sends values
    near those to the exact divide): the kernel's code read."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200_000) * 40).astype(F32)
    x = x[np.abs(np.abs(x - np.rint(x)) - F32(0.5)) > F32(1e-3)]
    for z in (0, 8, 15, 128):
        base = F32(12582912.0 + z)
        t = (x.astype(F64) + F64(base)).astype(F32)       # the fma's one rounding (x * 1 exact)
        got = t.view(np.int32).astype(np.int64) - np.int64(0x4B400000)
        want = np.rint(x.astype(F64)).astype(np.int64) + z
        assert np.array_equal(got, want)
