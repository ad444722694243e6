"""Cost-guided selector: measurement sweep, fit and table.

"flash-comm: Self-Synchronizing Collective Communication for LLM Decoding",
abstract: the readiness encoding is chosen by message size and the number of
GPUs, trading synchronization overhead against the extra bytes an encoding
moves.  "Why Microseconds Matter in AI Infrastructure", sections "What I
learned from it" and "Where I think this is heading": the choice is made from
measurements of the kernels, with a performance model as the next step.
"SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM Inference",
abstract: one-shot scales poorly with the number of GPUs and two-shot does
better at higher degrees -- so the same model also chooses the all-reduce
algorithm.

Model per collective (one-shot all-reduce, two-shot all-reduce, all-gather),
protocol p, rank count N and size range: T_p(S) = alpha_p + beta_p * S, with
S the payload bytes per rank.  alpha and beta are fitted to per-op times
measured with the persistent simulator on this GPU (system mode, every rank
running the full program), minimising relative error so that the
latency-bound small sizes count as much as the large ones.  The simulator
changes kernel and geometry with size (a workgroup per peer at the smallest
sizes, a wave per tile beyond), so each (collective, rank count) may get two
ranges, split where that lowers the worst-case protocol regret on the
measured points.  The argmin itself runs in the library
(``ar_select_protocol``, ``ar_select_collective``, ``ar_select_allreduce``);
this module measures, fits, stores and loads the table.

    python -m collective_synchronization_amd.selector --out cost_table.json

runs the sweep on cuda:0 and writes the table next to this file.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE_PATH = os.path.join(HERE, "cost_table.json")
PROTOS = ("ll", "ll128", "sentinel", "barrier")
COLLECTIVES = ("allreduce", "allgather", "twoshot")     # ids 0, 1, 2 of ar.h
SIZES = tuple(2 ** k for k in range(11, 23))          # 2 KiB .. 4 MiB per rank
# sizes between those of the fit, measured only to score the table on
# payloads it was not fitted to
HELDOUT_SIZES = (3 << 10, 12 << 10, 48 << 10, 96 << 10, 192 << 10, 384 << 10, 768 << 10,
                 3 << 19, 3 << 20)
GATHER_MAX = 1 << 20                                  # all-gather sweep: up to 1 MiB
# from 64 KiB on, per-op times bend between the powers of two without a
# change of kernel, tile class or launch (the working set of an op outgrows
# a cache level): the fit also measures 5/4 and 7/4 of each power there
QUARTER_SIZES = tuple(m * 2 ** k // 4 for k in range(16, 22) for m in (5, 7))
FIT_SIZES = tuple(sorted(SIZES + QUARTER_SIZES))


def _coll(p) -> str:
    return p.get("collective", "allreduce")


def fit_alpha_beta(sizes, times):
    """Relative least squares for T = alpha + beta * S (alpha, beta >= 0)."""
    S = np.asarray(sizes, dtype=np.float64)
    T = np.asarray(times, dtype=np.float64)
    A = np.stack([1.0 / T, S / T], axis=1)
    coef, *_ = np.linalg.lstsq(A, np.ones_like(T), rcond=None)
    alpha, beta = float(coef[0]), float(coef[1])
    if beta < 0.0:                       # flat data: constant model
        beta = 0.0
        alpha = float(len(T) / np.sum(1.0 / T))
    if alpha < 0.0:
        alpha = 0.0
        beta = float(np.sum(S / T) / np.sum((S / T) ** 2))
    return alpha, beta


def _pts(points, coll, n):
    return [p for p in points if _coll(p) == coll and p["nranks"] == n]


def _fit_range(pts, sizes):
    alpha = [None] * 4                   # None: protocol not measured here
    beta = [None] * 4
    for pi, proto in enumerate(PROTOS):
        q = [p for p in pts if p["proto"] == proto and p["bytes"] in sizes]
        if len(q) >= 2:
            alpha[pi], beta[pi] = fit_alpha_beta([p["bytes"] for p in q],
                                                 [p["us"] for p in q])
    return alpha, beta


def _fit_ranges(pts, coll, n, cuts):
    """One entry per size range; cuts are the inclusive upper ends of all
    ranges but the last (which has no upper end)."""
    sizes = sorted({p["bytes"] for p in pts})
    entries, lo = [], -1
    for hi in list(cuts) + [None]:
        rng = {s for s in sizes if s > lo and (hi is None or s <= hi)}
        alpha, beta = _fit_range(pts, rng)
        entries.append({"nranks": n, "collective": coll,
                        "max_bytes": 0 if hi is None else int(hi),
                        "alpha_us": alpha, "beta_us_per_byte": beta})
        lo = hi if hi is not None else lo
    return entries


def _score(pts, entries):
    """(max protocol regret, sum of squared relative model errors) on the
    measured points of one collective and rank count."""
    worst, sq = 1.0, 0.0
    for s in sorted({p["bytes"] for p in pts}):
        meas = {p["proto"]: p["us"] for p in pts if p["bytes"] == s}
        e = _range_entry(entries, s)
        pick, _ = argmin_py(e, s)
        if pick >= 0 and PROTOS[pick] in meas:
            worst = max(worst, meas[PROTOS[pick]] / min(meas.values()))
        for pi, proto in enumerate(PROTOS):
            if proto in meas and _available(e, pi):
                t = e["alpha_us"][pi] + e["beta_us_per_byte"][pi] * s
                sq += ((t - meas[proto]) / meas[proto]) ** 2
    return worst, sq


def _candidates(points, coll, n, max_ranges):
    """Every admissible split of one (collective, rank count): a list of
    (worst protocol regret, number of cuts, squared error, entries)."""
    pts = _pts(points, coll, n)
    sizes = sorted({p["bytes"] for p in pts})
    cands = [()]
    if max_ranges >= 2:
        cands += [(c,) for c in sizes[1:-2]]
    out = []
    for cuts in cands:
        ent = _fit_ranges(pts, coll, n, cuts)
        worst, sq = _score(pts, ent)
        out.append((worst, len(cuts), sq, ent))
    return pts, out


def _algorithm_regret(pts_one, pts_two, ent_one, ent_two):
    """Worst measured regret of the one-shot / two-shot choice (the rule of
    select_allreduce_py) over the sizes measured for both."""
    worst = 1.0
    sizes = sorted({p["bytes"] for p in pts_one} & {p["bytes"] for p in pts_two})
    for s in sizes:
        meas = {("allreduce", p["proto"]): p["us"] for p in pts_one if p["bytes"] == s}
        meas.update({("twoshot", p["proto"]): p["us"] for p in pts_two if p["bytes"] == s})
        p1, t1 = argmin_py(_range_entry(ent_one, s), s)
        p2, t2 = argmin_py(_range_entry(ent_two, s), s)
        key = ("twoshot", PROTOS[p2]) if (p2 >= 0 and t2 < t1) else ("allreduce", PROTOS[p1])
        if key in meas:
            worst = max(worst, meas[key] / min(meas.values()))
    return worst


def fit_interp(points):
    """Piecewise-linear table through the measured points: per collective and
    rank count, one range per interval between consecutive measured sizes
    (s_lo, s_hi], holding for each protocol the line through its two
    measurements there (alpha = T(s_lo) - beta * s_lo, beta = (T(s_hi) -
    T(s_lo)) / (s_hi - s_lo); None where a protocol lacks either point).  The
    first range also covers sizes below the first measurement and the last
    one, with no upper end, those above the last: the end lines extended
    (the last one drawn from the largest size at most 4/5 of the last, so
    that a narrow interval does not set its slope).
    The table reproduces every measured time, so the in-sample regret is 1,
    and between two measured sizes it predicts by linear interpolation."""
    entries = []
    for coll in COLLECTIVES:
        for n in sorted({p["nranks"] for p in points if _coll(p) == coll}):
            pts = _pts(points, coll, n)
            meas = {(p["proto"], p["bytes"]): p["us"] for p in pts}
            sizes = sorted({p["bytes"] for p in pts})
            if len(sizes) < 2:
                continue
            for i in range(1, len(sizes)):
                lo, hi = sizes[i - 1], sizes[i]
                if i == len(sizes) - 1:
                    # the line extended past the last size: through a size at
                    # most 4/5 of it, not across a narrow interval between
                    # two sides of a regime change
                    lo = max([x for x in sizes[:-1] if x * 5 <= hi * 4], default=lo)
                alpha, beta = [None] * 4, [None] * 4
                for pi, proto in enumerate(PROTOS):
                    if (proto, lo) in meas and (proto, hi) in meas:
                        b = (meas[(proto, hi)] - meas[(proto, lo)]) / (hi - lo)
                        alpha[pi] = meas[(proto, lo)] - b * lo
                        beta[pi] = b
                entries.append({"nranks": n, "collective": coll,
                                "max_bytes": 0 if i == len(sizes) - 1 else int(hi),
                                "alpha_us": alpha, "beta_us_per_byte": beta})
    return entries


def fit_table(points, max_ranges=2, method="interp"):
    """points: list of {collective?, nranks, proto, bytes, us} (collective
    defaults to the one-shot all-reduce).  Returns table entries.

    method "interp" (the committed table): fit_interp.  method "lsq": the
    least-squares alternative below, kept to compare with (its worst regret
    on held-out sizes was 1.145, against 1.081 for the interpolation).

    Per collective and rank count, one alpha-beta line per protocol over the
    whole sweep, or, with max_ranges=2, two lines split at a measured size
    (each range holds at least two measured sizes).  The split is the one
    with the lowest worst-case regret on the measured points (ties: one
    range, then the smaller squared relative error).  Where a rank count has
    both one-shot and two-shot points, their two splits are chosen together,
    and the regret also counts the choice between the two algorithms."""
    if method == "interp":
        return fit_interp(points)

    def ranks(coll):
        return sorted({p["nranks"] for p in points if _coll(p) == coll})

    entries = []
    for coll in COLLECTIVES:
        for n in ranks(coll):
            joint = n in ranks("allreduce") and n in ranks("twoshot")
            if coll == "twoshot" and joint:
                continue                         # chosen with the one-shot
            if coll == "allreduce" and joint:
                p_one, c_one = _candidates(points, "allreduce", n, max_ranges)
                p_two, c_two = _candidates(points, "twoshot", n, max_ranges)
                best = None
                for w1, k1, q1, e1 in c_one:
                    for w2, k2, q2, e2 in c_two:
                        worst = max(w1, w2, _algorithm_regret(p_one, p_two, e1, e2))
                        key = (round(worst, 9), k1 + k2, q1 + q2)
                        if best is None or key < best[0]:
                            best = (key, e1 + e2)
                entries.extend(best[1])
            else:
                _, c = _candidates(points, coll, n, max_ranges)
                entries.extend(min(c, key=lambda t: (round(t[0], 9), t[1], t[2]))[3])
    return entries


def _range_entry(entries, nbytes):
    """The entry of one (collective, rank count) whose size range holds
    nbytes (the same rule as the library)."""
    def upper(e):
        m = e.get("max_bytes", 0)
        return m if m > 0 else float("inf")
    fit = [e for e in entries if upper(e) >= nbytes]
    if fit:
        return min(fit, key=upper)
    return max(entries, key=upper)


def _available(entry, p):
    """A protocol is unavailable in an entry when a coefficient is None or not
    a finite number (the library's rule, NaN in the C table)."""
    a, b = entry["alpha_us"][p], entry["beta_us_per_byte"][p]
    return a is not None and b is not None and math.isfinite(a) and math.isfinite(b)


def argmin_py(entry, nbytes):
    best, tbest = -1, 0.0
    for p in range(4):
        a, b = entry["alpha_us"][p], entry["beta_us_per_byte"][p]
        if not _available(entry, p):
            continue
        t = a + b * nbytes
        if best < 0 or t < tbest:
            best, tbest = p, t
    return best, tbest


def select_py(entries, nbytes, nranks, collective="allreduce"):
    """Plain-Python statement of the library's choice within one collective:
    nearest rank count (ties: smaller), then the size range, then the
    argmin.  Returns (-1, 0.0) when the collective has no entries."""
    mine = [e for e in entries if _coll(e) == collective]
    if not mine:
        return -1, 0.0
    ns = sorted({e["nranks"] for e in mine})
    n_use = min(ns, key=lambda n: (abs(n - nranks), n))
    return argmin_py(_range_entry([e for e in mine if e["nranks"] == n_use], nbytes),
                     nbytes)


def select_allreduce_py(entries, nbytes, nranks):
    """(collective, protocol id, predicted us): the one-shot choice unless the
    two-shot one predicts strictly less."""
    p1, t1 = select_py(entries, nbytes, nranks, "allreduce")
    p2, t2 = select_py(entries, nbytes, nranks, "twoshot")
    if p2 >= 0 and t2 < t1:
        return "twoshot", p2, t2
    return "allreduce", p1, t1


def regret(points, entries):
    """Measured time of the library's choice over the best measured time.

    kind "protocol": the protocol choice within each collective;
    kind "allreduce": the algorithm-and-protocol choice of the all-reduce,
    over the best one-shot or two-shot measurement at that point."""
    from . import abi
    table = abi.cost_table(entries)
    out = []
    for coll in COLLECTIVES:
        if not any(_coll(e) == coll for e in entries):
            continue
        for n in sorted({p["nranks"] for p in points if _coll(p) == coll}):
            for s in sorted({p["bytes"] for p in points if _coll(p) == coll and
                             p["nranks"] == n}):
                meas = {p["proto"]: p["us"] for p in points
                        if _coll(p) == coll and p["nranks"] == n and p["bytes"] == s}
                if len(meas) < 2:
                    continue
                pick, _ = abi.ar_select_collective(table, coll, s, n)
                chosen = meas.get(PROTOS[pick])
                out.append({"kind": "protocol", "collective": coll, "nranks": n,
                            "bytes": s, "pick": PROTOS[pick],
                            "best": min(meas, key=meas.get),
                            "regret": (chosen / min(meas.values())) if chosen else None})
    if any(_coll(e) == "twoshot" for e in entries):
        for n in sorted({p["nranks"] for p in points if _coll(p) == "twoshot"}):
            for s in sorted({p["bytes"] for p in points if _coll(p) == "twoshot" and
                             p["nranks"] == n}):
                meas = {(_coll(p), p["proto"]): p["us"] for p in points
                        if _coll(p) in ("allreduce", "twoshot") and p["nranks"] == n and
                        p["bytes"] == s}
                if not any(k[0] == "allreduce" for k in meas):
                    continue
                cid, pick, _ = abi.ar_select_allreduce(table, s, n)
                key = (COLLECTIVES[cid], PROTOS[pick])
                chosen = meas.get(key)
                best = min(meas, key=meas.get)
                out.append({"kind": "allreduce", "nranks": n, "bytes": s,
                            "pick": "/".join(key), "best": "/".join(best),
                            "regret": (chosen / meas[best]) if chosen else None})
    return out


def load_table(path: str = TABLE_PATH):
    with open(path) as fh:
        return json.load(fh)


def select(nbytes: int, nranks: int, path: str = TABLE_PATH):
    """One-shot protocol chosen by the library for a payload of nbytes per rank."""
    from . import abi
    t = load_table(path)
    pick, pred = abi.ar_select_protocol(abi.cost_table(t["entries"]), nbytes, nranks)
    return PROTOS[pick], pred


def select_allreduce(nbytes: int, nranks: int, path: str = TABLE_PATH):
    """(algorithm, protocol, predicted us) chosen by the library."""
    from . import abi
    t = load_table(path)
    cid, pick, pred = abi.ar_select_allreduce(abi.cost_table(t["entries"]), nbytes, nranks)
    return COLLECTIVES[cid], PROTOS[pick], pred


# ------------------------------------------------------------------ sweep --

def measure_point(torch, abi, buffers, inputs, proto, nranks, nbytes, nops, reps,
                  seed=1004, collective="allreduce"):
    count = nbytes // 2
    x = inputs.payload(seed + nbytes, (nops, nranks, count), "uniform")
    ws = buffers.Workspace(nranks, count, proto, nranks, collective=collective)
    xd, stride = buffers.rows_to_device(x)
    ostride = ws.gather_stride() if collective == "allgather" else stride
    outd = torch.zeros((nops * nranks, ostride), dtype=torch.int16, device="cuda")
    for _ in range(2):
        ws.sim(nops, xd, stride, outd, ostride, timeout_ns=2_000_000_000)
    torch.cuda.synchronize()
    if ws.status() != 0:
        raise RuntimeError(f"{collective} {proto} N={nranks} S={nbytes}: "
                           f"{abi.status_string(ws.status())}")
    st = torch.cuda.current_stream()
    ms = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        if proto == "barrier":
            ws.reset_ctrl()
        p = ws.sim_params(nops, xd, stride, outd, ostride, timeout_ns=2_000_000_000)
        a.record(st)
        abi.ar_sim_run(p, st)
        b.record(st)
        ws.flip(nops)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    if ws.status() != 0:
        raise RuntimeError(f"{collective} {proto} N={nranks} S={nbytes}: "
                           f"{abi.status_string(ws.status())}")
    return statistics.median(ms) * 1e3 / nops


# a device address for geometry queries, which check alignment and read nothing
_GEO_ADDR = 1 << 20


def _nops_of(nbytes: int) -> int:
    # launches long enough for the library's cooperative-launch choice (at
    # least 32 ops), as in a decode step
    return 64 if nbytes <= (256 << 10) else 32


def geometry_key(abi, coll, n, proto, nbytes):
    """Kernel, whether a wave or workgroup walks one tile or several, and
    launch the simulator takes at this size (None where it cannot run):
    where one of them changes, the per-op time can jump.  (The number of
    tiles beyond the first grows with the size and adds time smoothly.)"""
    count = nbytes // 2
    rs = (count + 7) // 8 * 8
    d = abi.make_desc(n, count, proto, n, coll)
    p = abi.sim_params(d, _nops_of(nbytes), _GEO_ADDR, rs, _GEO_ADDR,
                       n * rs if coll == "allgather" else rs, _GEO_ADDR, _GEO_ADDR,
                       abi.ar_epoch_init())
    try:
        g = abi.ar_sim_geometry(p)
    except abi.ArError:
        return None
    return (g["kernel"], g["tiles_per_wave"] > 1, g["launch"])


def regime_sizes(abi, coll, n, proto, sizes, avoid=()):
    """The sizes on both sides of every regime change (geometry_key) between
    consecutive `sizes`, found by bisection on multiples of 16 bytes: the
    last size of one regime and the first of the next.  Measuring there keeps
    the interpolation from drawing a line across a jump."""
    out = set()
    for lo, hi in zip(sizes, sizes[1:]):
        k_hi = geometry_key(abi, coll, n, proto, hi)
        a, k_a = lo, geometry_key(abi, coll, n, proto, lo)
        for _ in range(8):                         # a few changes at most
            if k_a == k_hi or k_a is None or k_hi is None:
                break
            b = hi                                 # key(a) = k_a, key(b) != k_a
            while b - a > 16:
                mid = max(a + 16, (a + b) // 32 * 16)
                if geometry_key(abi, coll, n, proto, mid) == k_a:
                    a = mid
                else:
                    b = mid
            out.update(x for x in (a, b) if x not in avoid)
            a, k_a = b, geometry_key(abi, coll, n, proto, b)
    return out


def sweep(ranks=(4, 8, 16), sizes=FIT_SIZES, protos=PROTOS, reps=7, collectives=COLLECTIVES,
          tag="", regimes=False):
    """Per-op times of every protocol at every size; with `regimes`, also at
    the sizes on both sides of each regime change of any protocol between
    two of `sizes` (never one of HELDOUT_SIZES)."""
    import torch
    from . import abi, buffers, inputs
    torch.cuda.set_device(0)
    points = []
    for coll in collectives:
        for n in ranks:
            grid = set(sizes)
            if regimes:
                for proto in protos:
                    if coll != "allreduce" and proto == "barrier":
                        continue
                    top = [x for x in sorted(sizes)
                           if not (coll == "allgather" and x > GATHER_MAX)]
                    grid |= regime_sizes(abi, coll, n, proto, top, avoid=HELDOUT_SIZES)
                print(tag + json.dumps({"collective": coll, "nranks": n,
                                        "regime_sizes": sorted(grid - set(sizes))}),
                      flush=True)
            for s in sorted(grid):
                if coll == "allgather" and s > GATHER_MAX:
                    continue
                # system-mode receive buffers must stay below 4 GiB in total
                E_max = 2 * s
                if n * 2 * n * E_max >= (1 << 32):
                    continue
                nops = _nops_of(s)
                for proto in protos:
                    if coll != "allreduce" and proto == "barrier":
                        continue
                    us = measure_point(torch, abi, buffers, inputs, proto, n, s, nops, reps,
                                       collective=coll)
                    points.append({"collective": coll, "nranks": n, "proto": proto,
                                   "bytes": s, "us": round(us, 4)})
                    print(tag + json.dumps(points[-1]), flush=True)
    return points


def _worst(reg):
    worst = max((r["regret"] for r in reg if r["regret"]), default=1.0)
    by = {}
    for r in reg:
        k = r["kind"] if r["kind"] == "allreduce" else f"protocol/{r['collective']}"
        if r["regret"]:
            by[k] = max(by.get(k, 1.0), r["regret"])
    return worst, by


def main() -> int:
    ap = argparse.ArgumentParser(description="measure, fit and write the cost table")
    ap.add_argument("--out", default=TABLE_PATH)
    ap.add_argument("--ranks", default="4,8,16")
    ap.add_argument("--reps", type=int, default=7)
    ap.add_argument("--refit", metavar="TABLE",
                    help="refit the points stored in an existing table instead of measuring")
    ap.add_argument("--no-regimes", action="store_true",
                    help="measure only the powers of two, not also the sizes on both "
                         "sides of each kernel-regime change between them")
    ap.add_argument("--no-heldout", action="store_true",
                    help="skip the held-out sizes (measured between the fitted ones to "
                         "score the table out of sample)")
    args = ap.parse_args()
    t0 = time.time()
    old = None
    ranks = tuple(int(r) for r in args.ranks.split(","))
    if args.refit:
        old = load_table(args.refit)
        points = old["points"]
        heldout = old.get("heldout_points", [])
        measured_with = old["measured_with"]
    else:
        points = sweep(ranks, reps=args.reps, regimes=not args.no_regimes)
        heldout = [] if args.no_heldout else sweep(ranks, sizes=HELDOUT_SIZES,
                                                   reps=args.reps, tag="heldout ")
        measured_with = ("python -m collective_synchronization_amd.selector "
                         f"--ranks {args.ranks} --reps {args.reps}"
                         f"{' --no-regimes' if args.no_regimes else ''} (one MI355X, "
                         "system mode, persistent simulator, median per-op time)")
    entries = fit_table(points)
    reg = regret(points, entries)
    worst, worst_by = _worst(reg)
    table = {
        "model": "T_p(S) = alpha_us[p] + beta_us_per_byte[p] * S for S <= max_bytes "
                 "(0: no upper end), per collective and rank count; "
                 "S = payload bytes per rank; one range per interval between "
                 "measured sizes, each line through the two measurements "
                 "(null: protocol not measured there)",
        "protocols": list(PROTOS),
        "collectives": list(COLLECTIVES),
        "measured_with": measured_with,
        "entries": entries,
        "points": points,
        "regret": reg,
        "max_regret": worst,
        "max_regret_by_kind": worst_by,
        "sweep_seconds": (old.get("sweep_seconds") if old
                          else round(time.time() - t0, 1)),
    }
    if heldout:
        # out of sample: the same choices scored on sizes the fit never saw
        hreg = regret(heldout, entries)
        hworst, hby = _worst(hreg)
        lsq = fit_table(points, method="lsq")
        table.update({"heldout_sizes": sorted({p["bytes"] for p in heldout}),
                      "heldout_points": heldout, "heldout_regret": hreg,
                      "heldout_max_regret": hworst, "heldout_max_regret_by_kind": hby,
                      "lsq_two_range_fit": {
                          "max_regret": _worst(regret(points, lsq))[0],
                          "heldout_max_regret": _worst(regret(heldout, lsq))[0]}})
    with open(args.out, "w") as fh:
        json.dump(table, fh, indent=1)
    print(json.dumps({"max_regret": worst, "by_kind": worst_by,
                      "heldout_max_regret": table.get("heldout_max_regret"),
                      "heldout_by_kind": table.get("heldout_max_regret_by_kind")}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
