"""Pins for the oracle's fixed-order reduction (CPU only).

The reduction is out[j] = bf16_rne(((f32(x0) + f32(x1)) + ...) + f32(x_{N-1}))
with binary32 round-to-nearest-even additions in rank order.  It is pinned by

* an exact rational emulation of every binary32 addition (Python
  ``fractions.Fraction``, written here from the IEEE 754 rounding rule and
  sharing nothing with the C code) on special-value cross products;
* numpy float32 element-wise additions in rank order on random payloads
  (an independent implementation of the same additions), rounded to bf16 by
  torch;
* hand-derived closed-form cases in ``tests/golden/reduce_cases.txt``;
* the classic error bound of recursive summation against the exact sum.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import GOLDEN

# ------------------------------------------------ exact binary32 emulation --

_MIN_EXP = -126          # smallest normal exponent
_MANT_BITS = 23
_TINY_Q = Fraction(1, 2 ** 149)            # quantum of subnormals
_OVERFLOW = Fraction(2 ** 128) - Fraction(2 ** 103)  # rounds to Inf at/above


def _f32_decode(u):
    """binary32 bits -> ('nan',) | ('inf', sign) | ('num', Fraction, sign)."""
    sign = -1 if (u >> 31) & 1 else 1
    e = (u >> 23) & 0xFF
    m = u & 0x7FFFFF
    if e == 0xFF:
        return ("nan",) if m else ("inf", sign)
    if e == 0:
        val = Fraction(m, 2 ** 149)
    else:
        val = Fraction((1 << 23) | m, 1) * Fraction(2) ** (e - 127 - 23)
    return ("num", sign * val, sign)


def _round_f32(x: Fraction):
    """Round an exact rational to binary32, nearest even; returns a decoded tuple."""
    if x == 0:
        return ("num", Fraction(0), 1)
    sign = -1 if x < 0 else 1
    a = abs(x)
    if a >= _OVERFLOW:
        return ("inf", sign)
    # exponent of the leading bit
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, _MIN_EXP) - _MANT_BITS)
    n = a / q
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    val = lo * q
    if val >= Fraction(2 ** 128):
        return ("inf", sign)
    return ("num", sign * val, sign)


def _add_exact(a, b):
    """IEEE binary32 addition, round to nearest even, on decoded tuples."""
    if a[0] == "nan" or b[0] == "nan":
        return ("nan",)
    if a[0] == "inf" and b[0] == "inf":
        return a if a[1] == b[1] else ("nan",)
    if a[0] == "inf":
        return a
    if b[0] == "inf":
        return b
    s = a[1] + b[1]
    if s == 0:
        # exact zero sum: -0 only when both operands are -0 (round to nearest)
        neg = a[1] == 0 and b[1] == 0 and a[2] < 0 and b[2] < 0
        return ("num", Fraction(0), -1 if neg else 1)
    return _round_f32(s)


def _to_bf16(d):
    """Decoded binary32 -> bf16 bits, nearest even, NaN -> 0x7FC0 (exact)."""
    if d[0] == "nan":
        return 0x7FC0
    if d[0] == "inf":
        return 0x7F80 if d[1] > 0 else 0xFF80
    val, sign = d[1], d[2]
    if val == 0:
        return 0x8000 if sign < 0 else 0x0000
    s = 0x8000 if val < 0 else 0
    a = abs(val)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, _MIN_EXP) - 7)
    n = a / q
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    v = lo * q
    if v >= Fraction(2 ** 128):
        return s | 0x7F80
    if v < Fraction(2) ** _MIN_EXP:            # subnormal bf16
        return s | int(v / Fraction(2) ** (_MIN_EXP - 7))
    e2 = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e2 > v:
        e2 -= 1
    mant = int(v / Fraction(2) ** (e2 - 7)) - 128
    return s | ((e2 + 127) << 7) | mant


def _exact_reduce(rows):
    """Rank-order reduction of bf16 columns, every step exact-then-rounded."""
    out = []
    for col in zip(*rows):
        acc = _f32_decode(col[0] << 16)
        for b in col[1:]:
            acc = _add_exact(acc, _f32_decode(b << 16))
        out.append(_to_bf16(acc))
    return out


def test_exact_emulation_self_consistency():
    """Sanity of the emulator on values whose binary32 sum is obvious."""
    one = _f32_decode(0x3F800000)
    assert _to_bf16(_add_exact(one, one)) == 0x4000
    assert _to_bf16(_f32_decode(0x3F808000)) == 0x3F80   # tie even
    assert _to_bf16(_f32_decode(0x3F818000)) == 0x3F82   # tie odd


SPECIALS = [
    0x0000, 0x8000,            # +-0
    0x0001, 0x8001,            # +-min subnormal
    0x007F, 0x807F,            # +-max subnormal
    0x0080, 0x8080,            # +-min normal
    0x3F80, 0xBF80,            # +-1
    0x3F81, 0x3B80, 0x3400,    # rounding probes
    0x4B80, 0xCB80,            # +-2^24
    0x7F7F, 0xFF7F,            # +-max finite
    0x7F80, 0xFF80,            # +-Inf
    0x7FC0, 0xFFC0, 0xFFFF, 0x7F81,  # NaNs (quiet, negative, sentinel, signalling)
]


def test_reduce_n2_special_pairs_vs_exact():
    rows = [[a for a, _ in itertools.product(SPECIALS, SPECIALS)],
            [b for _, b in itertools.product(SPECIALS, SPECIALS)]]
    x = np.array(rows, dtype=np.uint16)
    ours = oracle.reduce(x).tolist()
    assert ours == _exact_reduce(rows)


def test_reduce_n3_special_triples_vs_exact():
    trip = list(itertools.product(SPECIALS, repeat=3))
    rows = [[t[k] for t in trip] for k in range(3)]
    x = np.array(rows, dtype=np.uint16)
    assert oracle.reduce(x).tolist() == _exact_reduce(rows)


@pytest.mark.parametrize("n,count,seed", [(1, 121, 1), (2, 97, 2), (3, 64, 3), (4, 121, 4)])
def test_reduce_random_wide_exponent_vs_exact(n, count, seed):
    """Random bf16 bit patterns over the whole exponent range (ragged counts)."""
    rng = np.random.default_rng(seed)
    x = rng.integers(0, 1 << 16, size=(n, count), dtype=np.uint32).astype(np.uint16)
    assert oracle.reduce(x).tolist() == _exact_reduce(x.tolist())


@pytest.mark.parametrize("n,count,dist,seed", [
    (4, 4096, "normal", 11), (8, 4096, "normal", 12), (16, 32768, "normal", 13),
    (8, 20000, "uniform", 14), (2, 1, "normal", 15), (5, 999, "uniform", 16),
])
def test_reduce_random_vs_numpy_float32(n, count, dist, seed):
    """Rank-order numpy float32 additions, bf16 rounding by torch."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        f = rng.standard_normal((n, count), dtype=np.float32)
    else:
        f = 2 * rng.random((n, count), dtype=np.float32) - 1
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wide = (x.astype(np.uint32) << 16).view(np.float32)
    acc = wide[0].copy()
    for r in range(1, n):
        acc = (acc + wide[r]).astype(np.float32)
    ref = torch.from_numpy(acc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.reduce(x), ref)


def _golden_reduce_cases():
    cases = []
    with open(os.path.join(GOLDEN, "reduce_cases.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line.startswith("case:"):
                continue
            lhs, rhs = line[len("case:"):].split("->")
            rows = [[int(t, 16) for t in part.split()] for part in lhs.split("|")]
            cases.append((rows, [int(t, 16) for t in rhs.split()]))
    return cases


@pytest.mark.parametrize("rows,expected", _golden_reduce_cases())
def test_reduce_golden_cases(rows, expected):
    x = np.array(rows, dtype=np.uint16)
    assert oracle.reduce(x).tolist() == expected
    # the same case through the full encode/validate/decode path, every protocol
    for proto in ("ll", "ll128", "sentinel", "barrier"):
        st, out = oracle.allreduce(x, proto, seq=9)
        assert st == oracle.READY
        assert out.tolist() == expected, proto


def test_reduce_within_recursive_summation_bound():
    """|result - exact| <= (n-1) u32 sum|x| + half a bf16 unit of the result."""
    rng = np.random.default_rng(21)
    n, count = 16, 2048
    f = rng.standard_normal((n, count), dtype=np.float32) * np.float32(3.0)
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out = oracle.reduce(x)
    wide = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    exact = wide.sum(axis=0)           # float64 holds these sums exactly enough
    absum = np.abs(wide).sum(axis=0)
    got = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    half_bf16 = np.abs(got) * 2.0 ** -8 + 2.0 ** -133
    bound = (n - 1) * 2.0 ** -24 * absum + half_bf16
    assert np.all(np.abs(got - exact) <= bound)
