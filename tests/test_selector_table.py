"""Host tests of the protocol selector's fit and table (CPU only).

The fit is checked on synthetic exact data, and the library's argmin
(ar_select_protocol) is checked against a plain Python argmin over the same
table.  When the committed cost table (measured on an MI355X) is present, its
structure and recorded regret are checked too.
"""
import os

import numpy as np
import pytest

from collective_synchronization_amd import abi, selector


def test_fit_recovers_exact_line():
    sizes = [2 ** k for k in range(11, 23)]
    alpha, beta = 2.5, 3e-4
    times = [alpha + beta * s for s in sizes]
    a, b = selector.fit_alpha_beta(sizes, times)
    assert abs(a - alpha) < 1e-9 and abs(b - beta) < 1e-12


def test_fit_flat_data_is_constant():
    sizes = [2048, 4096, 8192]
    a, b = selector.fit_alpha_beta(sizes, [3.0, 3.0, 3.0])
    assert b == pytest.approx(0.0, abs=1e-15) and a == pytest.approx(3.0)


def test_fit_table_and_regret_on_synthetic_points():
    pts = []
    model = {"ll": (2.0, 2e-4), "ll128": (3.0, 1.1e-4), "sentinel": (2.2, 1.5e-4),
             "barrier": (5.0, 1.2e-4)}
    for n in (4, 8):
        for s in selector.SIZES:
            for p, (a, b) in model.items():
                pts.append({"nranks": n, "proto": p, "bytes": s, "us": a + b * s})
    lsq = selector.fit_table(pts, method="lsq")
    assert [e["nranks"] for e in lsq] == [4, 8]
    interp = selector.fit_table(pts)
    assert [e["nranks"] for e in interp] == [4] * 11 + [8] * 11
    for entries in (lsq, interp):
        reg = selector.regret(pts, entries)
        assert all(r["regret"] == pytest.approx(1.0) for r in reg)


def test_interpolating_table_by_hand():
    """Three measured sizes, two protocols: the table holds the line through
    each pair of neighbouring points, so it reproduces the measurements,
    interpolates between them and extends the end lines beyond them."""
    pts = [{"nranks": 8, "proto": "ll", "bytes": 1000, "us": 1.0},
           {"nranks": 8, "proto": "ll", "bytes": 2000, "us": 1.2},
           {"nranks": 8, "proto": "ll", "bytes": 4000, "us": 3.2},
           {"nranks": 8, "proto": "sentinel", "bytes": 1000, "us": 1.5},
           {"nranks": 8, "proto": "sentinel", "bytes": 2000, "us": 1.6},
           {"nranks": 8, "proto": "sentinel", "bytes": 4000, "us": 1.8}]
    e = selector.fit_table(pts)
    assert [x["max_bytes"] for x in e] == [2000, 0]
    # first interval: LL 1.0 + 2e-4 (S - 1000); sentinel 1.5 + 1e-4 (S - 1000)
    assert e[0]["beta_us_per_byte"][0] == pytest.approx(2e-4)
    assert e[0]["alpha_us"][0] == pytest.approx(0.8)
    assert e[0]["alpha_us"][1] is None and e[0]["alpha_us"][3] is None
    # second interval: LL 1.2 + 1e-3 (S - 2000) -> alpha -0.8 (a valid line)
    assert e[1]["beta_us_per_byte"][0] == pytest.approx(1e-3)
    assert e[1]["alpha_us"][0] == pytest.approx(-0.8)
    t = abi.cost_table(e)
    for s, want in ((1000, 1.0), (2000, 1.2), (4000, 1.8), (1500, 1.1), (500, 0.9)):
        assert abi.ar_select_protocol(t, s, 8)[1] == pytest.approx(want), s
    # LL 1.2 + 1e-3 * 300 = 1.5 against the sentinel's 1.6 + 1e-4 * 300 = 1.63
    assert abi.ar_select_protocol(t, 2300, 8)[0] == abi.AR_LL
    # LL 2.2 against 1.7 at 3000: the sentinel
    assert abi.ar_select_protocol(t, 3000, 8)[0] == abi.AR_SENTINEL
    assert abi.ar_select_protocol(t, 8000, 8)[0] == abi.AR_SENTINEL


def test_library_argmin_matches_python():
    rng = np.random.default_rng(3)
    entries = [{"nranks": n, "alpha_us": list(rng.uniform(1, 6, 4)),
                "beta_us_per_byte": list(rng.uniform(5e-5, 3e-4, 4))} for n in (4, 8, 16)]
    table = abi.cost_table(entries)
    for n in (4, 8, 16):
        e = [x for x in entries if x["nranks"] == n][0]
        for s in [2 ** k for k in range(8, 24)]:
            pick, pred = abi.ar_select_protocol(table, s, n)
            ref, tref = selector.argmin_py(e, s)
            assert pick == ref and pred == pytest.approx(tref)


@pytest.mark.skipif(not os.path.exists(selector.TABLE_PATH), reason="no measured table")
def test_committed_table():
    t = selector.load_table()
    assert t["protocols"] == list(selector.PROTOS)
    assert {e["nranks"] for e in t["entries"]} >= {4, 8}
    for e in t["entries"]:
        assert len(e["alpha_us"]) == 4 and len(e["beta_us_per_byte"]) == 4
    # the library's choice on every measured point is within the recorded regret
    recomputed = selector.regret(t["points"], t["entries"])
    worst = max(r["regret"] for r in recomputed if r["regret"])
    assert worst == pytest.approx(t["max_regret"])
    assert worst < 1.5
    # out of sample: sizes between the fitted ones, never used by the fit
    if "heldout_points" in t:
        fitted = {p["bytes"] for p in t["points"]}
        assert not fitted & {p["bytes"] for p in t["heldout_points"]}
        held = selector.regret(t["heldout_points"], t["entries"])
        hworst = max(r["regret"] for r in held if r["regret"])
        assert hworst == pytest.approx(t["heldout_max_regret"])
        assert hworst <= 1.10


def test_library_ranges_match_python():
    """Piecewise tables: the library picks the nearest rank count, then the
    size range holding the payload, then the argmin, as select_py states."""
    rng = np.random.default_rng(11)
    entries = []
    for n in (4, 8, 16):
        cuts = sorted(rng.choice([2 ** k for k in range(10, 22)], size=2, replace=False))
        for hi in list(cuts) + [0]:
            entries.append({"nranks": n, "max_bytes": int(hi),
                            "alpha_us": list(rng.uniform(1, 6, 4)),
                            "beta_us_per_byte": list(rng.uniform(5e-5, 3e-4, 4))})
    rng.shuffle(entries)
    table = abi.cost_table(entries)
    for n in (1, 4, 6, 8, 12, 16):
        for s in [0] + [2 ** k for k in range(8, 24)] + [3000, 70000]:
            pick, pred = abi.ar_select_protocol(table, s, n)
            ref, tref = selector.select_py(entries, s, n)
            assert pick == ref and pred == pytest.approx(tref), (n, s)


def test_library_closed_ranges_fall_back_to_last():
    e = [{"nranks": 8, "max_bytes": 4096, "alpha_us": [1, 2, 3, 4],
          "beta_us_per_byte": [0, 0, 0, 0]},
         {"nranks": 8, "max_bytes": 65536, "alpha_us": [4, 3, 2, 1],
          "beta_us_per_byte": [0, 0, 0, 0]}]
    t = abi.cost_table(e)
    assert abi.ar_select_protocol(t, 4096, 8)[0] == abi.AR_LL
    assert abi.ar_select_protocol(t, 4097, 8)[0] == abi.AR_BARRIER
    assert abi.ar_select_protocol(t, 1 << 30, 8)[0] == abi.AR_BARRIER


def test_fit_finds_regime_change():
    """Two regimes (a cheap latency line that turns steep past 16 KiB for
    LL): one line per protocol cannot rank the protocols right on both
    sides; the two-range fit splits at 16 KiB and has no regret."""
    pts = []
    for s in selector.SIZES:
        ll = 1.5 + 2e-5 * s if s <= 16384 else 1.0 + 2e-4 * s
        sent = 2.0 + 1e-5 * s
        for proto, us in (("ll", ll), ("ll128", sent + 1.0), ("sentinel", sent),
                          ("barrier", 4.0 + 4e-4 * s)):
            pts.append({"nranks": 8, "proto": proto, "bytes": s, "us": us})
    one = selector.fit_table(pts, max_ranges=1, method="lsq")
    two = selector.fit_table(pts, max_ranges=2, method="lsq")
    assert len(one) == 1 and len(two) == 2
    assert sorted(e["max_bytes"] for e in two) == [0, 16384]
    assert max(r["regret"] for r in selector.regret(pts, one)) > 1.05
    assert max(r["regret"] for r in selector.regret(pts, two)) == pytest.approx(1.0)


def _random_entries(rng, colls=("allreduce", "twoshot", "allgather")):
    entries = []
    for coll in colls:
        for n in (4, 8, 16):
            cuts = sorted(rng.choice([2 ** k for k in range(10, 22)], size=1, replace=False))
            for hi in list(cuts) + [0]:
                a = list(rng.uniform(1, 6, 4))
                if coll != "allreduce":
                    a[3] = None                      # no barrier form
                entries.append({"nranks": n, "collective": coll, "max_bytes": int(hi),
                                "alpha_us": a,
                                "beta_us_per_byte": list(rng.uniform(5e-5, 3e-4, 4))})
    rng.shuffle(entries)
    return entries


def test_library_collective_and_algorithm_choice_match_python():
    rng = np.random.default_rng(21)
    entries = _random_entries(rng)
    table = abi.cost_table(entries)
    for n in (1, 4, 6, 8, 12, 16):
        for s in [0, 3000, 70000] + [2 ** k for k in range(8, 24)]:
            for coll in ("allreduce", "twoshot", "allgather"):
                pick, pred = abi.ar_select_collective(table, coll, s, n)
                ref, tref = selector.select_py(entries, s, n, coll)
                assert pick == ref and pred == pytest.approx(tref), (coll, n, s)
            cid, pick, pred = abi.ar_select_allreduce(table, s, n)
            rc, rp, rt = selector.select_allreduce_py(entries, s, n)
            assert (selector.COLLECTIVES[cid], pick) == (rc, rp) and pred == pytest.approx(rt)
    # one-shot entries only drive ar_select_protocol
    for n in (4, 8):
        for s in (2048, 1 << 20):
            assert abi.ar_select_protocol(table, s, n)[0] == selector.select_py(entries, s, n)[0]


def test_selection_without_entries_for_a_collective():
    rng = np.random.default_rng(22)
    one = _random_entries(rng, colls=("allreduce",))
    table = abi.cost_table(one)
    with pytest.raises(abi.ArError):
        abi.ar_select_collective(table, "twoshot", 4096, 8)
    cid, pick, _ = abi.ar_select_allreduce(table, 4096, 8)      # no two-shot: one-shot
    assert cid == abi.AR_ALLREDUCE
    only_two = _random_entries(rng, colls=("twoshot",))
    with pytest.raises(abi.ArError):                             # needs one-shot entries
        abi.ar_select_allreduce(abi.cost_table(only_two), 4096, 8)


def test_fit_chooses_two_shot_past_the_crossover():
    """One-shot: low latency, steep per-byte cost; two-shot: one more
    exchange, N/2 times fewer bytes.  The fitted table picks one-shot below
    the crossover and two-shot above it, with no regret."""
    pts = []
    for s in selector.SIZES:
        for proto, k in (("ll", 1.0), ("ll128", 1.3), ("sentinel", 1.1)):
            pts.append({"collective": "allreduce", "nranks": 16, "proto": proto,
                        "bytes": s, "us": k * (2.0 + 8e-4 * s)})
            pts.append({"collective": "twoshot", "nranks": 16, "proto": proto,
                        "bytes": s, "us": k * (4.0 + 1e-4 * s)})
        pts.append({"collective": "allreduce", "nranks": 16, "proto": "barrier",
                    "bytes": s, "us": 9.0 + 9e-4 * s})
    entries = selector.fit_table(pts)
    reg = selector.regret(pts, entries)
    assert {r["kind"] for r in reg} == {"protocol", "allreduce"}
    assert max(r["regret"] for r in reg) == pytest.approx(1.0)
    table = abi.cost_table(entries)
    assert abi.ar_select_allreduce(table, 2048, 16)[:2] == (abi.AR_ALLREDUCE, abi.AR_LL)
    assert abi.ar_select_allreduce(table, 1 << 20, 16)[:2] == (abi.AR_TWOSHOT, abi.AR_LL)


def _kinked_sweep(rng, n=8):
    """One-shot: flat latency that turns steep past a random size; two-shot:
    a higher floor with a gentler slope; LL, LL128 and sentinel scaled
    copies with noise.  Random shapes, one rank count."""
    pts = []
    kink = 2 ** int(rng.integers(12, 18))
    a1, b1, b1k = rng.uniform(1.0, 1.6), rng.uniform(1e-6, 5e-6), rng.uniform(2e-5, 8e-5)
    a2, b2 = rng.uniform(2.5, 4.0), rng.uniform(5e-6, 1.2e-5)
    for s in selector.SIZES:
        one = a1 + b1 * s + (b1k * (s - kink) if s > kink else 0.0)
        two = a2 + b2 * s
        for proto, k in (("ll", rng.uniform(0.9, 1.2)), ("ll128", 1.4), ("sentinel", 1.0)):
            pts.append({"collective": "allreduce", "nranks": n, "proto": proto, "bytes": s,
                        "us": one * k * rng.uniform(0.97, 1.03)})
            pts.append({"collective": "twoshot", "nranks": n, "proto": proto, "bytes": s,
                        "us": two * k * rng.uniform(0.97, 1.03)})
        pts.append({"collective": "allreduce", "nranks": n, "proto": "barrier", "bytes": s,
                    "us": 3 * one})
    return pts


def test_joint_split_never_worse_than_separate_splits():
    """The one-shot and two-shot size splits of a rank count are chosen
    together: the worst regret over the protocol and algorithm choices is
    never above that of splits chosen for each collective alone, and on some
    sweeps it is strictly lower."""
    rng = np.random.default_rng(31)
    better = 0
    for _ in range(12):
        pts = _kinked_sweep(rng)
        joint = selector.fit_table(pts, method="lsq")
        sep = []
        for coll in ("allreduce", "twoshot"):
            _, cands = selector._candidates(pts, coll, 8, 2)
            sep += min(cands, key=lambda t: (round(t[0], 9), t[1], t[2]))[3]
        wj = max(r["regret"] for r in selector.regret(pts, joint))
        ws = max(r["regret"] for r in selector.regret(pts, sep))
        assert wj <= ws + 1e-12
        better += wj < ws - 1e-9
    assert better >= 1


def test_regime_sizes_bisect_both_sides(monkeypatch):
    """The sweep's extra sizes: both sides of each regime change between two
    measured sizes (multiples of 16 bytes), none of the avoided sizes, and
    no search past a size the simulator cannot run."""
    def key(abi_, coll, n, proto, nbytes):
        if nbytes > 100000:
            return None
        return (nbytes >= 5008, nbytes >= 40000)
    monkeypatch.setattr(selector, "geometry_key", key)
    sizes = [2048, 4096, 8192, 16384, 32768, 65536, 131072]
    assert selector.regime_sizes(None, "allreduce", 8, "ll", sizes) == {4992, 5008, 39984,
                                                                         40000}
    got = selector.regime_sizes(None, "allreduce", 8, "ll", sizes, avoid={5008})
    assert got == {4992, 39984, 40000}

    def two(abi_, coll, n, proto, nbytes):             # two changes in one interval
        return (nbytes >= 9000, nbytes >= 12000)
    monkeypatch.setattr(selector, "geometry_key", two)
    assert selector.regime_sizes(None, "allreduce", 8, "ll", [8192, 16384]) == {
        8992, 9008, 11984, 12000}


def test_last_range_extends_a_wide_interval():
    """Past the last measured size the table extends the line from the
    largest size at most 4/5 of it, not the line across a 16-byte interval."""
    pts = [{"nranks": 8, "proto": "ll", "bytes": b, "us": u}
           for b, u in ((1000, 1.0), (2000, 2.0), (2016, 10.0))]
    pts += [{"nranks": 8, "proto": "sentinel", "bytes": b, "us": u}
            for b, u in ((1000, 3.0), (2000, 3.5), (2016, 3.6))]
    e = selector.fit_interp(pts)
    last = [x for x in e if x["max_bytes"] == 0][0]
    assert last["beta_us_per_byte"][0] == pytest.approx((10.0 - 1.0) / 1016)
    assert last["alpha_us"][0] + last["beta_us_per_byte"][0] * 2016 == pytest.approx(10.0)
    mid = [x for x in e if x["max_bytes"] == 2000][0]
    assert mid["beta_us_per_byte"][0] == pytest.approx(1.0 / 1000)


def test_fit_sizes_keep_the_heldout_sizes_out():
    """The fit measures the powers of two and, from 64 KiB on, 5/4 and 7/4 of
    each; none of them is a held-out size, and all are 16-byte multiples
    (whole encoded chunks for every protocol's row alignment)."""
    assert set(selector.SIZES) <= set(selector.FIT_SIZES)
    assert not set(selector.FIT_SIZES) & set(selector.HELDOUT_SIZES)
    assert list(selector.FIT_SIZES) == sorted(set(selector.FIT_SIZES))
    assert all(s % 16 == 0 for s in selector.FIT_SIZES)
    q = [s for s in selector.FIT_SIZES if s not in selector.SIZES]
    assert min(q) == 80 << 10 and max(q) == 3584 << 10 and len(q) == 12
