"""Pins for the oracle's bf16 conversions (CPU only).

The oracle's binary32 -> bf16 rounding is pinned to an independent library
routine (torch's CPU float -> bfloat16 conversion, round to nearest even)
over every one of the 2^32 binary32 bit patterns.  torch's CPU conversion
maps NaN to 0xFFFF, so NaN inputs are pinned separately: numpy decides which
inputs are NaN, and the oracle must return the canonical 0x7FC0 for exactly
those (the reading for NaN results).  The sentinel canonicalization is pinned
exhaustively over all 2^16 bf16 patterns against numpy's own NaN and sign
tests on the widened value.
"""
import numpy as np
import pytest
import torch

import oracle


def _bits_to_f32(u32):
    return np.asarray(u32, dtype=np.uint32).view(np.float32)


@pytest.mark.parametrize("val,expected", [
    (1.0, 0x3F80),
    (-1.0, 0xBF80),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
    (float("nan"), 0x7FC0),
])
def test_bf16_rne_simple_values(val, expected):
    assert oracle.bf16_rne_scalar(val) == expected


@pytest.mark.parametrize("u32,expected", [
    (0x3F808000, 0x3F80),  # tie, kept part even -> stays
    (0x3F818000, 0x3F82),  # tie, kept part odd -> rounds up
    (0x3F808001, 0x3F81),  # just above the tie
    (0x3F807FFF, 0x3F80),  # just below the tie
    (0x7F7FFFFF, 0x7F80),  # largest binary32 rounds to +Inf in bf16
    (0x7F7F7FFF, 0x7F7F),  # stays the largest finite bf16
    (0x00000001, 0x0000),  # tiny denormal rounds to +0
    (0x00008000, 0x0000),  # tie at zero, even -> +0
    (0x00018000, 0x0002),  # tie, odd -> up
    (0x807FFFFF, 0x8080),  # largest negative denormal rounds to -min normal
    (0xFFC00001, 0x7FC0),  # negative quiet NaN -> canonical
    (0x7F800001, 0x7FC0),  # signalling NaN -> canonical
])
def test_bf16_rne_edge_patterns(u32, expected):
    f = _bits_to_f32([u32])
    assert int(oracle.bf16_rne(f)[0]) == expected


def test_bf16_rne_exhaustive_against_torch():
    """All 2^32 binary32 patterns: non-NaN equals torch's RNE, NaN -> 0x7FC0."""
    chunk = 1 << 24
    for start in range(0, 1 << 32, chunk):
        u = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        f = u.view(np.float32)
        ours = oracle.bf16_rne(f)
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        ok = ~nan
        if not np.array_equal(ours[ok], ref[ok]):
            bad = np.nonzero(ours[ok] != ref[ok])[0][0]
            pytest.fail(f"bf16_rne mismatch at 0x{u[ok][bad]:08x}: "
                        f"oracle 0x{ours[ok][bad]:04x} torch 0x{ref[ok][bad]:04x}")
        assert np.all(ours[nan] == 0x7FC0)


def test_bf16_roundtrip_is_identity_on_non_nan():
    """Every non-NaN bf16 widened to binary32 and rounded back is itself."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    back = oracle.bf16_rne(f)
    nan = np.isnan(f)
    assert np.array_equal(back[~nan], b[~nan])
    assert np.all(back[nan] == 0x7FC0)
    # the C widening agrees with the bit-level definition on a few values
    for v in (0x3F80, 0x0001, 0x8000, 0x7F80):
        assert oracle._load().o_bf16_to_f32(v) == float(_bits_to_f32([v << 16])[0])


def test_canon_in_exhaustive():
    """Exactly the 127 negative-NaN patterns change, and they become 0x7FC0."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    widened = (b.astype(np.uint32) << 16).view(np.float32)
    neg_nan = np.isnan(widened) & np.signbit(widened)
    out = oracle.canon_in(b)
    assert int(neg_nan.sum()) == 127
    assert np.all(out[neg_nan] == 0x7FC0)
    assert np.array_equal(out[~neg_nan], b[~neg_nan])
    # the sentinel itself is a negative NaN and is never sent
    assert oracle.canon_in_scalar(0xFFFF) == 0x7FC0
    assert not np.any(out == 0xFFFF)
    # positive NaNs, -Inf and -0 are values, not sentinels
    for v in (0x7FC0, 0x7FFF, 0xFF80, 0x8000):
        assert oracle.canon_in_scalar(v) == v
