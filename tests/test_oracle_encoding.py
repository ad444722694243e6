"""Pins for the oracle's readiness encodings and invariants (CPU only).

* Hand-written golden byte vectors (``tests/golden/*.txt``) fix the LL,
  LL128, sentinel and barrier layouts.  The pages print no layout, so parity
  with the pages themselves is unpinned; these vectors pin the stated reading.
* Invariants from the pages: decode(encode(x)) is the identity up to the
  sentinel canonicalization; the sentinel never appears in sentinel-encoded
  data; a partially delivered, stale or never-written slot is not ready; an
  impossible flag is corrupt; the result does not depend on arrival order;
  all protocols deliver identical bits.
"""
import numpy as np
import pytest

import oracle
from conftest import hex_bytes, hex_u16, read_golden

PROTOS = ("ll", "ll128", "sentinel", "barrier")


@pytest.mark.parametrize("name", [
    "ll_count3_seq1.txt", "ll128_count61_seq7.txt",
    "sentinel_count5.txt", "barrier_count3.txt",
])
def test_golden_encoding(name):
    g = read_golden(name)
    x = hex_u16(g["x"])
    count, seq = int(g["count"]), int(g["seq"])
    assert x.size == count
    want = hex_bytes(g["bytes"])
    got = oracle.encode(g["proto"], x, seq)
    assert got.tobytes().hex(" ") == want.tobytes().hex(" ")
    st, y = oracle.decode(g["proto"], want, count, seq)
    assert st == oracle.READY
    expect = hex_u16(g["decoded"]) if "decoded" in g else x
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("proto,count,E", [
    ("ll", 4096, 16384), ("ll", 3, 16), ("ll", 4, 16), ("ll", 5, 32), ("ll", 0, 0),
    ("ll128", 8192, 17536), ("ll128", 32768, 70016), ("ll128", 131072, 279680),
    ("ll128", 60, 128), ("ll128", 61, 256), ("ll128", 1, 128),
    ("sentinel", 4096, 8192), ("sentinel", 32768, 65536), ("sentinel", 9, 32),
    ("barrier", 1024, 2048), ("barrier", 1, 16),
])
def test_encoded_sizes(proto, count, E):
    """E per slot: LL 16*ceil(n/4), LL128 128*ceil(n/60), others 16*ceil(n/8)."""
    assert oracle.encoded_bytes(proto, count) == E


def _rand_payload(rng, count, specials=False):
    x = rng.integers(0, 1 << 16, size=count, dtype=np.uint32).astype(np.uint16)
    if specials and count:
        idx = rng.choice(count, size=max(1, count // 8), replace=False)
        x[idx] = rng.choice(np.array([0xFFFF, 0xFFC0, 0xFF81, 0x7FC0, 0x8000, 0xFF80],
                                     dtype=np.uint16), size=idx.size)
    return x


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("count", [0, 1, 2, 3, 7, 8, 59, 60, 61, 127, 4096, 4099])
def test_pack_unpack_identity(proto, count):
    rng = np.random.default_rng(1000 + count)
    x = _rand_payload(rng, count, specials=True)
    seq = int(rng.integers(1, 1 << 32))
    wire = oracle.encode(proto, x, seq)
    st, y = oracle.decode(proto, wire, count, seq)
    assert st == oracle.READY
    want = oracle.canon_in(x) if proto == "sentinel" else x
    assert np.array_equal(y, want)


def test_sentinel_never_transmitted():
    rng = np.random.default_rng(5)
    x = _rand_payload(rng, 5000, specials=True)
    x[::7] = 0xFFFF
    wire = oracle.encode("sentinel", x, 1)
    assert not np.any(wire.view(np.uint16) == 0xFFFF)


@pytest.mark.parametrize("proto", ["ll", "ll128"])
def test_flag_classification(proto):
    rng = np.random.default_rng(7)
    count = 300
    x = _rand_payload(rng, count)
    seq = 1000
    stale = oracle.epoch_prev(oracle.epoch_prev(seq))
    wire = oracle.encode(proto, x, seq)
    # never written (all zero)
    assert oracle.decode(proto, np.zeros_like(wire), count, seq)[0] == oracle.NOT_READY
    # whole slot from two ops ago
    assert oracle.decode(proto, oracle.encode(proto, x, stale), count, seq)[0] == oracle.NOT_READY
    # the current epoch is ready; the previous epoch's flag is impossible here
    assert oracle.decode(proto, wire, count, seq)[0] == oracle.READY
    prev = oracle.encode(proto, x, oracle.epoch_prev(seq))
    assert oracle.decode(proto, prev, count, seq)[0] == oracle.CORRUPT
    # one unit (word / line) still stale -> not ready
    unit = 8 if proto == "ll" else 128
    old = oracle.encode(proto, x, stale)
    part = wire.copy()
    k = int(rng.integers(0, wire.size // unit))
    part[k * unit:(k + 1) * unit] = old[k * unit:(k + 1) * unit]
    assert oracle.decode(proto, part, count, seq)[0] == oracle.NOT_READY
    # one unit with a garbage flag -> corrupt (even if another unit is stale)
    bad = part.copy()
    j = (k + 1) % (wire.size // unit)
    flag_off = j * unit + (4 if proto == "ll" else 120)
    bad[flag_off] ^= 0x5A
    assert oracle.decode(proto, bad, count, seq)[0] == oracle.CORRUPT


def test_sentinel_partial_delivery_not_ready():
    rng = np.random.default_rng(8)
    count = 333
    x = _rand_payload(rng, count, specials=True)
    wire = oracle.encode("sentinel", x, 4)
    armed = np.full_like(wire, 0xFF)
    assert oracle.decode("sentinel", armed, count, 4)[0] == oracle.NOT_READY
    for k in (0, count // 2, count - 1):
        part = wire.copy()
        part[2 * k:2 * k + 2] = 0xFF
        assert oracle.decode("sentinel", part, count, 4)[0] == oracle.NOT_READY


def test_epoch_wrap():
    assert oracle.epoch_next(1) == 2
    assert oracle.epoch_next(0xFFFFFFFF) == 1
    assert oracle.epoch_prev(1) == 0xFFFFFFFF
    for s in (1, 2, 3, 0xFFFFFFFE, 0xFFFFFFFF):
        assert oracle.epoch_prev(oracle.epoch_next(s)) == s
        assert oracle.epoch_next(s) != 0


@pytest.mark.parametrize("proto", PROTOS)
def test_arrival_order_independence(proto):
    rng = np.random.default_rng(9)
    n, count = 16, 1000
    x = rng.standard_normal((n, count)).astype(np.float32)
    xb = oracle.bf16_rne(x)
    st0, ref = oracle.allreduce(xb, proto, seq=3)
    assert st0 == oracle.READY
    for _ in range(5):
        perm = rng.permutation(n).astype(np.int32)
        st, out = oracle.allreduce(xb, proto, seq=3, perm=perm)
        assert st == oracle.READY
        assert np.array_equal(out, ref)


def test_protocols_deliver_identical_bits():
    rng = np.random.default_rng(10)
    n, count = 8, 2053
    x = np.stack([_rand_payload(rng, count, specials=True) for _ in range(n)])
    outs = [oracle.allreduce(x, p, seq=77)[1] for p in PROTOS]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    # and equal to the bare fixed-order reduction of the canonicalized input
    assert np.array_equal(outs[0], oracle.reduce(oracle.canon_in(x)))


def test_allreduce_rejects_bad_permutation():
    x = np.zeros((3, 4), dtype=np.uint16)
    st, _ = oracle.allreduce(x, "ll", 1, perm=np.array([0, 0, 1], dtype=np.int32))
    assert st == oracle.CORRUPT
