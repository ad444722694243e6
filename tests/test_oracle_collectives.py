"""Pins for the oracle's all-gather and two-shot all-reduce (CPU only).

* share bounds: hand-computed cases (tests/golden/shard_bounds.txt) and the
  partition invariants (disjoint, in order, covering, 16-byte aligned starts);
* all-gather: a hand-derived sentinel case, the pack/unpack identity per
  row for every protocol (canon_in for the sentinel), arrival-order
  independence;
* two-shot: a hand-derived 3-rank case whose columns pin the rank order,
  ties-to-even and NaN/Inf/-0/subnormal handling across a ragged last share,
  and equality with the pinned one-shot oracle (the same definition reached
  through a different data path) over shapes with empty shares;
* both reject what the one-shot oracle rejects (a repeated rank in the
  arrival order).
"""
import numpy as np
import pytest

import oracle
from conftest import hex_u16, read_golden


def _cases(name):
    with open(__import__("os").path.join(__import__("conftest").GOLDEN, name)) as fh:
        for line in fh:
            if line.startswith("case:"):
                yield line[5:].strip()


def test_shard_bounds_golden():
    n_cases = 0
    for c in _cases("shard_bounds.txt"):
        lhs, rhs = c.split("->")
        count, n = (int(t) for t in lhs.split())
        want = [tuple(int(v) for v in t.split(",")) for t in rhs.split()]
        assert len(want) == n
        assert [oracle.shard_bounds(count, n, k) for k in range(n)] == want, c
        n_cases += 1
    assert n_cases == 7


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 13, 16])
def test_shard_partition_invariants(n):
    for count in [0, 1, 2, 7, 8, 9, 15, 16, 17, 61, 100, 1000, 4095, 4096, 4097, 32768, 131072]:
        b = [oracle.shard_bounds(count, n, k) for k in range(n)]
        assert b[0][0] == 0 and b[-1][1] == count
        for (lo, hi), (lo2, _) in zip(b, b[1:]):
            assert lo <= hi == lo2
        assert all(lo % 8 == 0 or lo == count for lo, _ in b)
        widths = [hi - lo for lo, hi in b]
        full = max(widths)
        assert full % 8 == 0 or full == count
        # every share but the last non-empty one has the full width
        nz = [w for w in widths if w]
        assert all(w == full for w in nz[:-1])


def test_allgather_sentinel_golden():
    g = read_golden("allgather_sentinel_n2_count3.txt")
    x = np.stack([hex_u16(g["rank0"]), hex_u16(g["rank1"])])
    st, got = oracle.allgather(x, "sentinel", 1)
    assert st == oracle.READY
    assert np.array_equal(got[0], hex_u16(g["row0"]))
    assert np.array_equal(got[1], hex_u16(g["row1"]))
    # the other encodings deliver the bits unchanged, negative NaNs included
    for p in ("ll", "ll128", "barrier"):
        st, got = oracle.allgather(x, p, 1)
        assert st == oracle.READY and np.array_equal(got, x)


@pytest.mark.parametrize("proto", ["ll", "ll128", "sentinel", "barrier"])
@pytest.mark.parametrize("n,count", [(1, 5), (2, 1), (3, 61), (4, 1000), (8, 4099), (16, 33)])
def test_allgather_identity_and_order(proto, n, count):
    rng = np.random.default_rng(n * 1000 + count)
    x = rng.integers(0, 1 << 16, (n, count), dtype=np.uint16)
    x[:, ::7] = 0xFFFF                      # the sentinel itself as input
    want = oracle.canon_in(x) if proto == "sentinel" else x
    st, got = oracle.allgather(x, proto, 77)
    assert st == oracle.READY and np.array_equal(got, want)
    perm = rng.permutation(n).astype(np.int32)
    st, got2 = oracle.allgather(x, proto, 77, perm)
    assert st == oracle.READY and np.array_equal(got2, want)
    if proto == "sentinel":
        assert not np.any(got == 0xFFFF)


def test_allgather_rejects_repeated_rank():
    x = np.zeros((3, 8), dtype=np.uint16)
    st, _ = oracle.allgather(x, "ll", 1, np.array([0, 0, 2], dtype=np.int32))
    assert st == oracle.CORRUPT


def test_twoshot_golden():
    g = read_golden("twoshot_n3_count20.txt")
    x = np.stack([hex_u16(g[f"rank{r}"]) for r in range(3)])
    want = hex_u16(g["out"])
    assert x.shape == (3, 20)
    for p in ("ll", "ll128", "sentinel", "barrier"):
        st, got = oracle.twoshot(x, p, 5)
        assert st == oracle.READY
        assert np.array_equal(got, want), p


@pytest.mark.parametrize("proto", ["ll", "ll128", "sentinel", "barrier"])
@pytest.mark.parametrize("n,count", [(1, 7), (2, 0), (2, 9), (3, 20), (4, 5), (5, 61),
                                     (8, 4096), (8, 4099), (16, 33), (16, 1000)])
def test_twoshot_equals_oneshot(proto, n, count):
    rng = np.random.default_rng(7 * n + count)
    x = oracle.bf16_rne(rng.standard_normal((n, count), dtype=np.float32))
    specials = np.array([0xFFFF, 0xFFC0, 0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001,
                         0x8001, 0x7F7F], dtype=np.uint16)
    if count:
        idx = rng.integers(0, x.size, max(1, x.size // 16))
        x.reshape(-1)[idx] = rng.choice(specials, idx.size)
    st1, one = oracle.allreduce(x, proto, 9)
    st2, two = oracle.twoshot(x, proto, 9)
    assert st1 == st2 == oracle.READY
    assert np.array_equal(one, two)


def test_twoshot_ops_match_allreduce_ops():
    rng = np.random.default_rng(5)
    x = oracle.bf16_rne(rng.standard_normal((4, 8, 300), dtype=np.float32))
    assert np.array_equal(oracle.twoshot_ops(x, "sentinel", 3),
                          oracle.allreduce_ops(x, "sentinel", 3))
    got = oracle.allgather_ops(x, "ll", 3)
    assert np.array_equal(got, x)
