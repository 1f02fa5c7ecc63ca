"""Host check of the exact centroid-sum arithmetic of the clustering kernels.

Each input x of a head is scaled by 2^S (S = B - E, with |x| < 2^E over the head
and B = min(51, 62 - ceil(log2(N + 1)))) and split into the nearest integer a
and the remainder r = x 2^S - a; both a and r 2^B become 64-bit integers through
the fp64 magic-number add.  The kernel's fp64 steps are emulated here in exact
rational arithmetic (each step rounded once to the nearest fp64, as IEEE fma and
add do), so the test checks the numerical argument itself: for every N the
library accepts, the images are integers below 2^51, their sums over N rows stay
below 2^62, and the value (a + r_img 2^-B) 2^-S reproduces x exactly whenever
its unit in the last place is at least 2^(E - 2B) -- the documented floor
(include/svgear.h, "Input values").  Values below the floor are the ones the
library reports as out of range.
"""
from fractions import Fraction

import numpy as np
import pytest

MAGIC = 1.5 * 2.0 ** 52


def fl(q: Fraction) -> float:
    """Round an exact rational to the nearest fp64 (ties to even)."""
    return float(q)   # int / int true division in CPython is correctly rounded


def fma(a, b, c) -> float:
    return fl(Fraction(a) * Fraction(b) + Fraction(c))


def fix_base(N: int) -> int:
    lg = 0
    while lg < 31 and (1 << lg) <= N:
        lg += 1
    return min(62 - lg, 51)


def fix_exp(max_abs: float) -> int:
    """Smallest E with max_abs < 2^E (max_abs a finite non-negative fp32 value)."""
    if max_abs == 0.0:
        return 0
    m, e = np.frexp(np.float32(max_abs))   # max_abs = m 2^e, 0.5 <= m < 1
    return int(e)


def images(x: float, S: int, B: int):
    s, t = 2.0 ** S, 2.0 ** B
    a = fma(x, s, MAGIC)                 # magic + nearest integer of x 2^S
    r = fma(x, s, MAGIC - a)             # remainder, exact
    lo = fma(r, t, MAGIC)
    return int(Fraction(a) - Fraction(MAGIC)), int(Fraction(lo) - Fraction(MAGIC)), Fraction(r)


def bf16_values(rng, n, scale):
    x = (rng.standard_t(3.0, n) * scale).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def ulp_exp(x: np.float32, prec: int) -> int:
    """Exponent of the unit in the last place of a non-zero value with prec bits."""
    m, e = np.frexp(np.float32(abs(x)))
    return max(int(e) - 1, -126) - (prec - 1)


@pytest.mark.parametrize("N", [1, 8, 100, 611, 1024, 75600, 118800, 1 << 20])
def test_split_is_exact_above_the_floor(N):
    rng = np.random.default_rng(N)
    B = fix_base(N)
    for scale in (1e-3, 1.0, 150.0, 2000.0):
        x = bf16_values(rng, 64, scale)
        x[0] = np.float32(scale * 37.0)          # the head's largest magnitude
        E = fix_exp(float(np.abs(x).max()))
        S = B - E
        for v in x:
            hi, lo, _ = images(float(v), S, B)
            assert abs(hi) <= 2 ** 51 and abs(lo) < 2 ** 51
            if v != 0 and ulp_exp(v, 8) >= E - 2 * B:
                # exact: the value is recovered from the two images
                assert Fraction(hi) + Fraction(lo, 2 ** B) == Fraction(float(v)) * 2 ** S
        # sums of N rows of the largest image stay inside 62 bits
        assert N * 2 ** (E + S) <= 2 ** 62
        assert N * 2 ** (B - 1) < 2 ** 62


@pytest.mark.parametrize("N,x", [(611, 150.0), (100, 20.0), (1, 1.0), (16, 1.0), (1, 255.0)])
def test_small_n_values_the_old_fixed_shift_rounded(N, x):
    """The fixed shift S = 54 - lg of the previous library rounded these; the
    per-head scale captures them exactly."""
    B = fix_base(N)
    E = fix_exp(x)
    hi, lo, _ = images(x, B - E, B)
    assert Fraction(hi) + Fraction(lo, 2 ** B) == Fraction(x) * 2 ** (B - E)


def test_values_below_the_floor_are_not_exact():
    """A non-zero bf16 value whose ulp lies below 2^(E - 2B) is rounded when
    its last mantissa bit is set: the library must report such a head (its
    check, on the smallest non-zero magnitude, is conservative: it also reports
    values below the floor whose low mantissa bits happen to be zero)."""
    N = 75600
    B = fix_base(N)
    E = 9                                   # largest magnitude in [256, 512)
    tiny = np.float32((1 + 127 / 128) * 2.0 ** (E + 7 - 2 * B - 2))   # below the floor, all mantissa bits set
    assert ulp_exp(tiny, 8) < E - 2 * B
    hi, lo, _ = images(float(tiny), B - E, B)
    assert Fraction(hi) + Fraction(lo, 2 ** B) != Fraction(float(tiny)) * 2 ** (B - E)
    ok = np.float32(2.0 ** (E + 7 - 2 * B))                # exactly at the floor
    hi, lo, _ = images(float(ok), B - E, B)
    assert Fraction(hi) + Fraction(lo, 2 ** B) == Fraction(float(ok)) * 2 ** (B - E)
