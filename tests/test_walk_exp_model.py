"""A host model of the walk kernel's two table-driven float64 exps.

The kernel computes exp(y), y <= 0, as 2^k * tab[j] * exp(r) with
n = round(256 y / ln2) = 256 k + j taken from the low word of
y * 256 / ln2 + 1.5 * 2^52, r = y - n ln2 / 256 (ln2 / 256 in two parts) and
exp(r) by its degree-4 Taylor polynomial.  The general form clamps y at -746
and scales with ldexp; the fast form (batches whose entries all lie within
700 of the running max) skips the clamp and adds k to the exponent field of a
second table whose entries carry j << 12 less in their high word.  Modelled
here in float64 with exact fused multiply-adds (through fractions): the fast
form gives the same bits as the general one on [-700, 0], and both stay
within 2 ulp of exp.  The model writes the formulas out independently of the
kernel source; the GPU parity tests then check the walk's decisions.
"""
import math
import random
import struct
from fractions import Fraction

K_INV = 369.3299304675746            # 256 / ln2
SHIFT = 6755399441055744.0           # 1.5 * 2^52
LN2_HI = 6.93147180369123816490e-01 / 256
LN2_LO = 1.90821492927058770002e-10 / 256
TAB = [2.0 ** (j / 256) for j in range(256)]


def _fma(a, b, c):
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def _words(x):
    u = struct.unpack("<Q", struct.pack("<d", x))[0]
    return u >> 32, u & 0xFFFFFFFF


def _from_words(hi, lo):
    return struct.unpack("<d", struct.pack("<Q", ((hi & 0xFFFFFFFF) << 32) | lo))[0]


def _signed32(u):
    return u - (1 << 32) if u & 0x80000000 else u


TAB2 = [_from_words(_words(t)[0] - (j << 12), _words(t)[1]) for j, t in enumerate(TAB)]


def _reduce(y):
    t = _fma(y, K_INV, SHIFT)
    n = t - SHIFT
    ni = _signed32(_words(t)[1])
    r = _fma(-n, LN2_HI, y)
    r = _fma(-n, LN2_LO, r)
    p = 1.0 / 24.0
    for c in (1.0 / 6.0, 0.5, 1.0, 1.0):
        p = _fma(p, r, c)
    return ni, p


def exp_general(y):
    yc = max(y, -746.0)
    ni, p = _reduce(yc)
    return math.ldexp(TAB[ni & 255] * p, ni >> 8)


def exp_fast(y):
    ni, p = _reduce(y)
    hi, lo = _words(TAB2[ni & 255])
    return p * _from_words(hi + ((ni << 12) & 0xFFFFFFFF), lo)


def _ulps(a, b):
    return abs(a - b) / math.ulp(b)


def test_fast_exp_matches_general_bitwise_and_within_2ulp():
    rng = random.Random(20251203)
    ys = [0.0, -0.0, -1e-300, -1e-17, -700.0, -699.9999999999, -math.log(2) / 512,
          -math.log(2) / 256, -745.0 + 45.0]
    ys += [-rng.random() * 700.0 for _ in range(6000)]
    ys += [-rng.random() * 8.0 for _ in range(3000)]
    ys += [-rng.random() * 1e-3 for _ in range(1000)]
    worst = 0.0
    for y in ys:
        g = exp_general(y)
        f = exp_fast(y)
        assert struct.pack("<d", g) == struct.pack("<d", f), (y, g, f)
        worst = max(worst, _ulps(g, math.exp(y)))
    # math.exp itself is within about half an ulp
    assert worst <= 2.5, worst


def test_general_exp_underflows_to_zero_and_handles_minus_inf():
    assert exp_general(-746.0) == 0.0
    assert exp_general(-1e30) == 0.0
    assert exp_general(-math.inf) == 0.0
    assert exp_general(-700.0) > 0.0
