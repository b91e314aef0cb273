"""The float64 exp of the acceptance and draft-tree kernels (csrc/rowstream.h: Tang's table
method, a 2^(j/256) table with a degree-4 polynomial or a 2^(j/64) table with degree 5),
replayed step by step on the host with every float64 operation rounded as the device
rounds it (an FMA rounded once), against exp in 60 digits.  The constants are read from
the source, so a wrong digit there fails here."""
import math
import random
import re
from decimal import Decimal, getcontext
from pathlib import Path

import pytest

getcontext().prec = 60
SRC = (Path(__file__).resolve().parents[1] / "tree_attention_verification_ev_amd" / "csrc"
       / "rowstream.h").read_text()
LN2 = Decimal("0.693147180559945309417232121458176568075500134360255254120680009")
SHIFT = float(re.search(r"constexpr double kShifter = ([0-9.e+-]+);", SRC).group(1))


def consts(bits):
    body = re.search(r"struct ExpReduction<%d> \{(.*?)\};" % bits, SRC, re.S).group(1)
    get = lambda n: float(re.search(r"%s = ([0-9.e+-]+);" % n, body).group(1))
    return get("kInvLn2xN"), get("kLn2dNHi"), get("kLn2dNLo")


def fma(a, b, c):
    return float(Decimal(a) * Decimal(b) + Decimal(c))


def make_exp(bits):
    n = 1 << bits
    inv, hi, lo = consts(bits)
    tab = [float(Decimal(2) ** (Decimal(j) / n)) for j in range(n)]

    def dev_exp(x):
        x = max(x, -745.0)
        t = fma(x, inv, SHIFT)
        kf = t - SHIFT
        k = int(kf)
        r = fma(-kf, hi, x)
        r = fma(-kf, lo, r)
        if bits >= 8:
            p = fma(r, 1.0 / 24.0, 1.0 / 6.0)
        else:
            p = fma(r, 1.0 / 120.0, 1.0 / 24.0)
            p = fma(r, p, 1.0 / 6.0)
        p = fma(r, p, 0.5)
        p = fma(r, p, 1.0)
        p = p * r
        tj = tab[k & (n - 1)]
        return math.ldexp(fma(tj, p, tj), k >> bits)
    return dev_exp


@pytest.mark.parametrize("bits", [8, 6])
def test_constants(bits):
    n = 1 << bits
    inv, hi, lo = consts(bits)
    assert inv == float(Decimal(n) / LN2)
    assert hi == float(LN2 / n) and abs(Decimal(hi) + Decimal(lo) - LN2 / n) < Decimal(1e-35)
    assert SHIFT == 1.5 * 2.0 ** 52


@pytest.mark.parametrize("bits", [8, 6])
def test_within_two_ulp_over_the_range(bits):
    dev_exp = make_exp(bits)
    rng = random.Random(7)
    xs = [-rng.uniform(0, 40) for _ in range(2000)] + [-rng.uniform(40, 700) for _ in range(300)]
    xs += [0.0, -1e-300, -math.log(2) / (2 << bits), -math.log(2) / (1 << bits), -1.0, -708.0]
    worst = 0.0
    for x in xs:
        want = Decimal(x).exp()
        got = dev_exp(x)
        worst = max(worst, abs(Decimal(got) - want) / Decimal(math.ulp(float(want))))
    assert worst <= 2, worst


@pytest.mark.parametrize("bits", [8, 6])
def test_below_the_clamp(bits):
    dev_exp = make_exp(bits)
    assert dev_exp(-745.0) <= 5e-324 and dev_exp(-1e300) <= 5e-324 and dev_exp(-800.0) <= 5e-324
