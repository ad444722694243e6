"""Pins for the oracle's row-parallel linear producer and its chain (CPU).

The producer (a reading; the pages name the pattern of "SiFAR" abstract --
the all-reduce result feeding the next layer -- not a layer) is one decode
token's row-parallel linear shard: rank r's partial output
y[j] = bf16_rne(S(0, kr)), S the pairwise (recursive halving) binary32 sum
of the products f32(v[k]) * f32(w[j][k]) over rank r's input slice.  Pinned by

* hand-derived cases (tests/golden/linear_cases.txt): sums whose value
  depends on the tree (pairwise against left-to-right and right-to-left),
  overflow to Inf, Inf - Inf, 0 * Inf, signed zeros, subnormals;
* an exact rational emulation (Fraction, the IEEE 754 rounding rule) of
  every multiply and add of the recursion, on special values and random
  bf16 patterns, for lengths that are and are not powers of two;
* numpy float32 arithmetic in a bottom-up tree (add adjacent pairs, halve,
  repeat), an independent implementation of the same sum for powers of two;
* the error bound of pairwise summation against the exact dot product;
* closed forms of the chain: identity weights keep the input, a cyclic
  shift matrix rotates it by one element per op (a transposed weight layout
  would rotate the other way), doubled identity weights double it, layers
  are taken in turn, and each rank reads only its own slice of its row.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import GOLDEN
from test_oracle_scale import _mul_exact
from test_oracle_sum import _add_exact, _f32_decode, _to_bf16


def _f32_bits(f):
    return struct.unpack("<I", struct.pack("<f", f))[0]


def _exact_pairwise(v, w, a, b):
    if b - a == 1:
        return _mul_exact(_f32_decode(int(v[a]) << 16), _f32_decode(int(w[a]) << 16))
    m = a + (b - a) // 2
    return _add_exact(_exact_pairwise(v, w, a, m), _exact_pairwise(v, w, m, b))


def _decoded_matches(d, f):
    """Exact-emulation tuple d against the oracle's binary32 result f."""
    if d[0] == "nan":
        return math.isnan(f)
    if d[0] == "inf":
        return math.isinf(f) and (f > 0) == (d[1] > 0)
    if d[1] == 0:
        return f == 0 and (math.copysign(1.0, f) < 0) == (d[2] < 0)
    return Fraction(f) == d[1]


def _golden():
    cases = []
    with open(GOLDEN + "/linear_cases.txt") as fh:
        for line in fh:
            if not line.startswith("case:"):
                continue
            lhs, rhs = line[5:].split("->")
            v, w = lhs.split("|")
            cases.append((np.array([int(t, 16) for t in v.split(",")], dtype=np.uint16),
                          np.array([int(t, 16) for t in w.split(",")], dtype=np.uint16),
                          int(rhs.strip(), 16)))
    return cases


def test_linear_golden_cases():
    cases = _golden()
    assert len(cases) == 12
    for v, w, want in cases:
        got = int(oracle.linear_shard(v, w[None, :])[0])
        assert got == want, (v, w, hex(got), hex(want))
        assert _to_bf16(_exact_pairwise(v, w, 0, v.size)) == want   # the emulation agrees


SPECIALS = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x3F81,
            0x4B80, 0xCB80, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0x3380, 0x1C80]


@pytest.mark.parametrize("kr", [1, 2, 3, 4, 5, 7, 8, 13, 16, 64])
def test_linear_dot_vs_exact_emulation(kr):
    rng = np.random.default_rng(7000 + kr)
    trials = 0
    for t in range(60):
        if t % 3 == 0:      # special values
            v = rng.choice(SPECIALS, kr).astype(np.uint16)
            w = rng.choice(SPECIALS, kr).astype(np.uint16)
        elif t % 3 == 1:    # random patterns of every exponent (NaNs included)
            v = rng.integers(0, 1 << 16, kr, dtype=np.uint32).astype(np.uint16)
            w = rng.integers(0, 1 << 16, kr, dtype=np.uint32).astype(np.uint16)
        else:               # ordinary magnitudes with cancellation
            v = oracle.bf16_rne(rng.standard_normal(kr).astype(np.float32))
            w = oracle.bf16_rne((rng.standard_normal(kr) * 2.0 ** rng.integers(-30, 30, kr))
                                .astype(np.float32))
        d = _exact_pairwise(v, w, 0, kr)
        f = oracle.linear_dot(v, w)
        assert _decoded_matches(d, f), (kr, v, w, d, f)
        assert int(oracle.linear_shard(v, w[None, :])[0]) == _to_bf16(d)
        trials += 1
    assert trials == 60


def _numpy_tree(v, wt):
    """Pairwise sum for a power-of-two length by adding adjacent pairs of
    float32 partial sums level by level (numpy arithmetic), then bf16."""
    p = v.astype(np.uint32)[None, :] << 16
    q = wt.astype(np.uint32) << 16
    s = p.view(np.float32) * q.view(np.float32)
    while s.shape[1] > 1:
        s = s[:, 0::2] + s[:, 1::2]
    import torch
    return torch.from_numpy(s[:, 0].copy()).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


@pytest.mark.parametrize("kr", [64, 256, 512, 1024, 2048])
def test_linear_shard_vs_numpy_tree(kr):
    rng = np.random.default_rng(7100 + kr)
    count = 96
    v = oracle.bf16_rne(rng.standard_normal(kr).astype(np.float32))
    wt = oracle.bf16_rne((rng.standard_normal((count, kr)) / math.sqrt(kr)).astype(np.float32))
    want = _numpy_tree(v, wt)
    got = oracle.linear_shard(v, wt)
    # NaN is canonical in both (no NaN arises here)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kr", [128, 512, 2048])
def test_linear_error_bound(kr):
    rng = np.random.default_rng(7200 + kr)
    count = 64
    v = oracle.bf16_rne(rng.standard_normal(kr).astype(np.float32))
    wt = oracle.bf16_rne(rng.standard_normal((count, kr)).astype(np.float32))
    vf = (v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (wt.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    u = 2.0 ** -24
    depth = math.ceil(math.log2(kr))
    for j in range(count):
        prods = vf * wf[j]                  # bf16 * bf16 is exact in binary64
        exact = math.fsum(prods)
        bound = depth * u / (1 - depth * u) * float(np.abs(prods).sum())
        f = oracle.linear_dot(v, wt[j])
        assert abs(f - exact) <= bound, (j, f, exact, bound)
        # and the bf16 output is within half a bf16 ulp of the binary32 sum
        y = int(oracle.linear_shard(v, wt[j:j + 1])[0])
        yf = struct.unpack("<f", struct.pack("<I", y << 16))[0]
        assert abs(yf - f) <= 2.0 ** (math.frexp(f)[1] - 9)


# ------------------------------------------------------------ chain forms --

def _normal_row(rng, count):
    x = oracle.bf16_rne(rng.standard_normal(count).astype(np.float32))
    x[x == 0] = 0x3F80
    return x


def _identity(n, count, value=0x3F80, shift=0):
    """weights [n, count, kr]: rank r's row j holds `value` at the k with
    j == (r*kr + k + shift) mod count, zero elsewhere."""
    kr = count // n
    w = np.zeros((n, count, kr), dtype=np.uint16)
    for r in range(n):
        for k in range(kr):
            w[r, (r * kr + k + shift) % count, k] = value
    return w


@pytest.mark.parametrize("proto", ["ll", "ll128", "sentinel"])
def test_chain_identity_weights_keep_the_input(proto):
    n, count = 4, 256
    x = _normal_row(np.random.default_rng(7300), count)
    w = _identity(n, count)[None]
    out = oracle.linear_chain_ops(np.stack([x] * n), w, 5, proto)
    for i in range(5):
        assert np.array_equal(out[i], x), i


def test_chain_shift_matrix_rotates_by_one_per_op():
    n, count = 4, 128
    x = _normal_row(np.random.default_rng(7301), count)
    w = _identity(n, count, shift=1)[None]
    out = oracle.linear_chain_ops(np.stack([x] * n), w, 4, "ll")
    for i in range(4):
        assert np.array_equal(out[i], np.roll(x, i + 1)), i


def test_chain_doubled_identity_doubles_each_op():
    n, count = 2, 128
    x = _normal_row(np.random.default_rng(7302), count)
    w = _identity(n, count, value=0x4000)[None]        # 2.0
    out = oracle.linear_chain_ops(np.stack([x] * n), w, 6, "sentinel")
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    for i in range(6):
        want = oracle.bf16_rne((xf * np.float32(2.0 ** (i + 1))).astype(np.float32))
        assert np.array_equal(out[i], want), i


def test_chain_takes_layers_in_turn():
    n, count = 4, 256
    x = _normal_row(np.random.default_rng(7303), count)
    w = np.stack([_identity(n, count), _identity(n, count, shift=1)])
    out = oracle.linear_chain_ops(np.stack([x] * n), w, 5, "ll128")
    shifts = [0, 1, 1, 2, 2]
    for i in range(5):
        assert np.array_equal(out[i], np.roll(x, shifts[i])), i


def test_chain_rank_reads_only_its_slice_of_its_row():
    n, count = 4, 256
    kr = count // n
    rng = np.random.default_rng(7304)
    want = _normal_row(rng, count)
    x0 = np.full((n, count), 0x7FC0, dtype=np.uint16)   # NaN everywhere else
    for r in range(n):
        x0[r, r * kr:(r + 1) * kr] = want[r * kr:(r + 1) * kr]
    out = oracle.linear_chain_ops(x0, _identity(n, count)[None], 2, "sentinel")
    assert np.array_equal(out[0], want)
    assert np.array_equal(out[1], want)


def test_chain_equals_shards_then_allreduce():
    """Random weights: op i's result is the rank-order all-reduce of the
    per-rank linear_shard outputs of op i-1's result (composition check
    with the separately pinned allreduce)."""
    n, count, nops = 3, 192, 3
    kr = count // n
    rng = np.random.default_rng(7305)
    x = _normal_row(rng, count)
    w = oracle.bf16_rne((rng.standard_normal((2, n, count, kr)) / math.sqrt(kr))
                        .astype(np.float32))
    out = oracle.linear_chain_ops(np.stack([x] * n), w, nops, "ll")
    z = x
    for i in range(nops):
        y = np.stack([oracle.linear_shard(z[r * kr:(r + 1) * kr], w[i % 2, r])
                      for r in range(n)])
        z = oracle.reduce(y)
        assert np.array_equal(out[i], z), i


def test_chain_shapes_are_checked():
    x = np.zeros((4, 256), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.linear_chain_ops(x, np.zeros((1, 4, 256, 32), dtype=np.uint16), 1)
    with pytest.raises(ValueError):
        oracle.linear_chain_ops(x, np.zeros((1, 3, 256, 64), dtype=np.uint16), 1)
    with pytest.raises(ValueError):
        oracle.linear_shard(np.zeros(8, dtype=np.uint16), np.zeros((4, 7), dtype=np.uint16))
