"""Pins for the oracle's producer epilogue y = bf16_rne(f32(x) * s) (CPU).

* hand-derived cases (tests/golden/scale_cases.txt): ties, halfway points,
  signed zeros, Inf * 0, overflow, subnormal results;
* an exact rational emulation of the binary32 multiply (Fraction, written
  from the IEEE 754 rounding rule) on every bf16 value against a set of
  scales;
* numpy's float32 multiply followed by torch's RNE bfloat16 conversion (an
  independent implementation) on random payloads and scales;
* closed forms: s = 1 leaves every non-NaN value unchanged; s = 2^k with an
  in-range result adds k to the exponent exactly.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import GOLDEN
from test_oracle_sum import _f32_decode, _round_f32, _to_bf16


def _f32_bits(f):
    return struct.unpack("<I", struct.pack("<f", f))[0]


def _f32_from_bits(u):
    return struct.unpack("<f", struct.pack("<I", u))[0]


def _mul_exact(a, b):
    """IEEE binary32 multiplication, round to nearest even, decoded tuples."""
    if a[0] == "nan" or b[0] == "nan":
        return ("nan",)
    sa = a[1] if a[0] == "inf" else a[2]
    sb = b[1] if b[0] == "inf" else b[2]
    sign = sa * sb
    if a[0] == "inf" or b[0] == "inf":
        other = b if a[0] == "inf" else a
        if other[0] == "num" and other[1] == 0:
            return ("nan",)
        return ("inf", sign)
    p = a[1] * b[1]
    if p == 0:
        return ("num", Fraction(0), sign)
    return _round_f32(p)


def _scale_exact(x_bits, s_bits):
    return _to_bf16(_mul_exact(_f32_decode(x_bits << 16), _f32_decode(s_bits)))


def test_scale_golden_cases():
    n = 0
    with open(GOLDEN + "/scale_cases.txt") as fh:
        for line in fh:
            if not line.startswith("case:"):
                continue
            lhs, rhs = line[5:].split("->")
            xb, sb = (int(t, 16) for t in lhs.split())
            want = int(rhs.strip(), 16)
            got = int(oracle.scale(np.array([xb], dtype=np.uint16), _f32_from_bits(sb))[0])
            assert got == want, (hex(xb), hex(sb), hex(got), hex(want))
            assert _scale_exact(xb, sb) == want                 # the emulation agrees
            n += 1
    assert n == 15


SCALES = [1.0, -1.0, 0.5, 3.0, 1.0078125, 0.1, -7.25, 1e-30, 1e30, 2.0 ** -130]


@pytest.mark.parametrize("s", SCALES)
def test_scale_all_bf16_vs_exact(s):
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.scale(x, s)
    sb = _f32_bits(s)
    step = 7 if s not in (1.0, 0.5) else 1         # every value for two scales
    for xb in range(0, 1 << 16, step):
        assert int(got[xb]) == _scale_exact(xb, sb), (hex(xb), s)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_scale_random_vs_numpy(seed):
    rng = np.random.default_rng(seed)
    x = rng.integers(0, 1 << 16, 200_000, dtype=np.uint16)
    for s in rng.standard_normal(8).astype(np.float32) * np.float32(10.0) ** rng.integers(-20, 20, 8):
        s = np.float32(s)
        f = (x.astype(np.uint32) << 16).view(np.float32)
        with np.errstate(all="ignore"):
            p = f * s                                   # binary32 multiply, RNE
        want = torch.from_numpy(p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        want = np.where(np.isnan(p), np.uint16(0x7FC0), want)
        assert np.array_equal(oracle.scale(x, float(s)), want)


def test_scale_closed_forms():
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(f)
    one = oracle.scale(x, 1.0)
    assert np.array_equal(one[~nan], x[~nan]) and np.all(one[nan] == 0x7FC0)
    # normal values whose exponent stays in range: s = 2^k adds k to it
    for k in (-5, 1, 7):
        y = oracle.scale(x, 2.0 ** k)
        e = (x.astype(np.int32) >> 7) & 0xFF
        ok = (e >= 1) & (e <= 254) & (e + k >= 1) & (e + k <= 254)
        want = (x.astype(np.int32) + k * 128).astype(np.uint16)
        assert np.array_equal(y[ok], want[ok])
