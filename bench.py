#!/usr/bin/env python3
"""Benchmark of the self-synchronizing one-shot bf16 all-reduce on one MI355X.

One step = one decode token's worth of all-reduces for the workload: `nops`
back-to-back one-shot all-reduces (2 per layer) run by one persistent launch
of the simulator -- encode, poll + validate, fixed-order reduce, sentinel
re-arm and epoch flip for every op.  The N simulated ranks are wave groups
placed on different XCDs; by default (system mode) every rank runs the full
per-rank program, consume(op) -> produce(op+1), into its own receive buffer,
so each op carries the real cross-rank dependency.  Share mode (one receive
buffer, rank 0's share of the traffic) is reported beside it.  Inputs are
resident in HBM before the timed region.

`--collective allgather|twoshot` times the standalone all-gather or the
two-shot all-reduce (system mode) on the same transfers instead.

Prints ONE JSON line: value = microseconds per all-reduce (lower is better),
with the roofline of the simulator kernel (algorithmic HBM bytes per launch /
HIP-event duration of the launch), the measured one-chip floor, and the CPU
oracle timed on the host as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("µs per all-reduce and achieved HBM GB/s vs roofline, "
          "N simulated ranks, 1 MI355X")
HBM_PEAK_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def _env(name, cast, fallback):
    """An environment override (unset or empty: the fallback)."""
    v = os.environ.get(name, "")
    return fallback if v == "" else cast(v)


# environment overrides: AR_TIMEOUT_US (poll deadline), AR_PROTO (default
# protocol), AR_WG_PER_RANK (tile groups per rank; 0 = the library's choice)
MAX_TIMEOUT_US = 60e6          # the library's bound (AR_MAX_TIMEOUT_NS, 60 s)


def _timeout_ns():
    """AR_TIMEOUT_US as nanoseconds: (None, message) unless 0 < value <= 60 s."""
    try:
        us = _env("AR_TIMEOUT_US", float, 2e6)
    except ValueError:
        return None, f"AR_TIMEOUT_US={os.environ.get('AR_TIMEOUT_US')!r} is not a number"
    if not (0.0 < us <= MAX_TIMEOUT_US) or int(us * 1e3) < 1:
        return None, (f"AR_TIMEOUT_US={us:g} must be a poll deadline above 0 and at most "
                      f"{MAX_TIMEOUT_US:g} us")
    return int(us * 1e3), ""


TIMEOUT_NS, TIMEOUT_ERROR = _timeout_ns()
KERNEL_SOURCES = [
    os.path.join(ROOT, "collective_synchronization_amd", "csrc", n)
    for n in ("ar_kernels.hip", "ar_protocols.h", "ar_device.h")
]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(proto: str, nranks: int, count: int, nconsumers: int,
                      collective: str = "allreduce") -> int:
    """HBM bytes one op must move (re-polls not counted).

    allreduce: every rank reads its payload (N*S); every consumer receives E
    from each of the N-1 other ranks (written once, read once) and writes S
    of output; sentinel slots are re-armed after reading (another (N-1)*E
    per consumer).  A rank's own contribution stays in registers.
    allgather: the same exchange, but every consumer writes N*S of output.
    twoshot: every rank reads its payload (N*S); each share k's encoding E_k
    is received by its owner from the N-1 others (reduce-scatter) and the
    reduced share is received by the N-1 others (all-gather), each written
    once and read once; every rank writes S of output; sentinel slots of
    both exchanges are re-armed."""
    from collective_synchronization_amd import abi
    S = 2 * count
    if collective == "twoshot":
        sumE = 0
        for k in range(nranks):
            lo, hi = abi.ar_shard_bounds(count, nranks, k)
            sumE += abi.ar_encoded_bytes(proto, hi - lo)
        recv = 2 * (nranks - 1) * sumE
        b = nranks * S + 2 * recv + nranks * S
        if proto == "sentinel":
            b += recv
        return b
    E = abi.ar_encoded_bytes(proto, count)
    recv = nconsumers * (nranks - 1) * E
    out = nconsumers * S * (nranks if collective == "allgather" else 1)
    b = nranks * S + 2 * recv + out
    if proto == "sentinel":
        b += recv
    return b


def measure_floor(torch, abi, iters=2000):
    """One-chip floor in the form 2*L_load + L_oneway (cross-XCD)."""
    hz = abi.ar_wallclock_hz()
    work = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    res = torch.zeros(8, dtype=torch.int64, device="cuda")
    oneway = []
    for xb in range(1, 8):
        work.zero_()
        res.zero_()
        abi.ar_probe_pingpong(work, iters, 0, xb, res)
        torch.cuda.synchronize()
        r = res.cpu().tolist()
        if r[4] == 0 and r[1] == iters:
            oneway.append(r[0] / iters / hz / 2 * 1e6)
    chain_bytes = 16 << 20
    cw = torch.zeros(chain_bytes, dtype=torch.uint8, device="cuda")
    res.zero_()
    abi.ar_probe_loadchain(cw, chain_bytes, iters, res)
    torch.cuda.synchronize()
    r = res.cpu().tolist()
    load_us = r[0] / r[1] / hz * 1e6
    ow = statistics.median(oneway) if oneway else float("nan")
    return {"oneway_us": round(ow, 4), "load_us": round(load_us, 4),
            "sol_us": round(2 * load_us + ow, 4),
            "pingpong_pairs": len(oneway)}


def measure_launch_and_copy(torch, abi, launches=200, copy_bytes=256 << 20, copies=5):
    """Empty-kernel launch time (HIP events around a burst of launches, per
    launch) and the streaming-copy ceiling (bytes read + written per second,
    best of `copies` copies of copy_bytes)."""
    stream = torch.cuda.current_stream()
    for _ in range(10):
        abi.ar_probe_empty(stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(launches):
        abi.ar_probe_empty(stream)
    b.record(stream)
    torch.cuda.synchronize()
    empty_us = a.elapsed_time(b) * 1e3 / launches
    src = torch.ones(copy_bytes // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    abi.ar_probe_copy(src, dst, copy_bytes, stream)
    best = float("inf")
    for _ in range(copies):
        a.record(stream)
        abi.ar_probe_copy(src, dst, copy_bytes, stream)
        b.record(stream)
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e-3)
    ok = bool(torch.equal(src, dst))
    del src, dst
    return {"empty_kernel_us": round(empty_us, 3),
            "copy_gbs": round(2 * copy_bytes / best / 1e9, 1) if ok else None,
            "copy_bytes": copy_bytes}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(x, proto, seconds, collective="allreduce"):
    import oracle
    us, ops = oracle.time_collective(x, proto, collective, seconds=seconds)
    return us, ops


def load_traffic(kernel_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    try:
        with open(PROFILE_TRAFFIC) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = t.get(kernel_name)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def measure(torch, abi, buffers, x, proto, nranks, count, nops, mode, steps, warmup,
            waves_per_rank=0, flags=0, collective="allreduce"):
    """Time `steps` launches of the simulator (one step = nops ops).

    Returns per-launch HIP-event durations (ms, on the launch stream), the
    wall-clock duration of the timed region (s), geometry and status."""
    nconsumers = nranks if mode == "system" else 1
    xd, stride = buffers.rows_to_device(x)
    ws = buffers.Workspace(nranks, count, proto, nconsumers, collective=collective)
    ostride = ws.gather_stride() if collective == "allgather" else stride
    outd = torch.zeros((nops * nconsumers, ostride), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    kw = dict(timeout_ns=TIMEOUT_NS, waves_per_rank=waves_per_rank, flags=flags)
    for _ in range(warmup):
        ws.sim(nops, xd, stride, outd, ostride, **kw)
    torch.cuda.synchronize()
    if ws.status() != 0:
        raise RuntimeError(f"device status {abi.status_string(ws.status())}")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    params = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        if proto == "barrier":
            ws.reset_ctrl()
        p = ws.sim_params(nops, xd, stride, outd, ostride, **kw)
        params.append(p)
        starts[k].record(stream)
        abi.ar_sim_run(p, stream)
        ends[k].record(stream)
        ws.flip(nops)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if ws.status() != 0:
        raise RuntimeError(f"device status {abi.status_string(ws.status())}")
    launch_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    geo = abi.ar_sim_geometry(params[0])
    return dict(launch_ms=launch_ms, wall=wall, geo=geo, nconsumers=nconsumers)


def measure_placement(torch, abi, blocks, threads):
    """Where the workgroups of the timed grid ran: the XCC_ID of each,
    against round-robin dispatch (workgroup b on XCD (s + b) mod 8, s the
    XCD of workgroup 0), which the simulators' placement relies on."""
    import numpy as np
    work = torch.zeros(256, dtype=torch.uint8, device="cuda")
    res = torch.full((blocks,), -2, dtype=torch.int32, device="cuda")
    abi.ar_probe_placement(blocks, threads, work, res)
    torch.cuda.synchronize()
    x = res.cpu().numpy()
    props = torch.cuda.get_device_properties(0)
    return {"blocks": blocks, "threads": threads,
            "round_robin_start": int(x[0]),
            "on_expected_xcd": round(float(np.mean(x == (x[0] + np.arange(blocks)) % 8)), 4),
            "xcds_seen": int(len(set(x[x >= 0].tolist()))),
            "cus": int(props.multi_processor_count),
            "device": props.name, "arch": getattr(props, "gcnArchName", ""),
            # one device spanning all eight XCDs (256 CUs) is the SPX partition
            "partition": "SPX" if len(set(x[x >= 0].tolist())) == 8 else "other"}


def measure_skew(torch, abi, buffers, inputs, x, proto, nranks, count, nops, steps,
                 warmup, skew_us, seed, collective):
    """Ops with a seeded producer delay U[0, skew_us) per (op, producer) and
    the wall-clock trace: per-op time and the post-arrival latency (op done
    at the last consumer minus the last producer's last store).  The trace
    makes every sender wait for its stores before its timestamp, so these
    runs are slower than the untraced ones."""
    import numpy as np
    xd, stride = buffers.rows_to_device(x)
    ws = buffers.Workspace(nranks, count, proto, nranks, collective=collective)
    ostride = ws.gather_stride() if collective == "allgather" else stride
    outd = torch.zeros((nops * nranks, ostride), dtype=torch.int16, device="cuda")
    hz = abi.ar_wallclock_hz()
    d_us = inputs.delays_us(seed + 1, nops, nranks, skew_us)
    ticks = torch.from_numpy(np.round(d_us * hz * 1e-6).astype(np.int32)).to("cuda")
    trace = torch.zeros(nops * 2 * nranks + 1, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    post, per_op = [], []
    for k in range(warmup + steps):
        trace.zero_()
        trace[-1] = -1
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        ws.sim(nops, xd, stride, outd, ostride, timeout_ns=TIMEOUT_NS,
               delay_ticks=ticks, trace=trace)
        b.record(stream)
        torch.cuda.synchronize()
        if ws.status() != 0:
            raise RuntimeError(f"device status {abi.status_string(ws.status())}")
        if k < warmup:
            continue
        t = trace.cpu().numpy()[:-1].reshape(nops, 2, nranks).astype(np.float64)
        post.extend(((t[:, 1, :].max(axis=1) - t[:, 0, :].max(axis=1)) / hz * 1e6).tolist())
        per_op.append(a.elapsed_time(b) * 1e3 / nops)
    return {"skew_us": skew_us, "mean_delay_us": round(float(d_us.mean()), 3),
            "us_per_op": round(statistics.median(per_op), 3),
            "post_arrival_us_median": round(float(np.median(post)), 3),
            "post_arrival_us_p90": round(float(np.percentile(post, 90)), 3)}


def measure_epilogue(torch, abi, buffers, x, proto, nranks, count, steps, warmup):
    """Stream-ordered ops whose producer is a per-rank scale, two ways:
    fused (ar_scale_pack sends from the producer's epilogue) and unfused
    (ar_scale_rows writes the result, ar_pack_* encodes it).  Both end with
    ar_reduce_validate (system mode).  HIP events around the producer part
    and around the whole op, median over `steps` ops."""
    stride = buffers.row_stride(count)
    xd, _ = buffers.rows_to_device(x)
    scales = torch.linspace(0.5, 1.5, nranks, dtype=torch.float32, device="cuda")
    yd = torch.zeros((nranks, stride), dtype=torch.int16, device="cuda")
    outd = torch.zeros((nranks, stride), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    out = {}
    for mode in ("fused", "unfused"):
        ws = buffers.Workspace(nranks, count, proto, nranks)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for k in range(warmup + steps):
            e = ev[k - warmup] if k >= warmup else None
            if e:
                e[0].record(stream)
            if mode == "fused":
                abi.ar_scale_pack(ws.desc, xd, stride, scales, ws.scratch, ws.epoch, stream)
            else:
                abi.ar_scale_rows(nranks, count, xd, stride, scales, yd, stride, stream)
                ws.pack(yd, stride, stream)
            if e:
                e[1].record(stream)
            ws.reduce(outd, stride, timeout_ns=TIMEOUT_NS, stream=stream)
            if e:
                e[2].record(stream)
            ws.flip()
        torch.cuda.synchronize()
        if ws.status() != 0:
            raise RuntimeError(f"device status {abi.status_string(ws.status())}")
        out[mode] = {
            "producer_us": round(statistics.median(a.elapsed_time(b) for a, b, _ in ev) * 1e3, 3),
            "op_us": round(statistics.median(a.elapsed_time(c) for a, _, c in ev) * 1e3, 3),
        }
    return out


def measure_chain(torch, abi, buffers, x0, proto, nranks, count, nops, steps, warmup,
                  seed=7):
    """The chained simulator (ar_sim_chain_run): op i+1's payload of rank r
    is op i's result times a per-rank factor s[i+1][r] ~ U[0.5, 1.5)/nranks,
    in one persistent launch.  HIP events per launch, median over `steps`
    launches, plus the wall clock of the timed launches."""
    import numpy as np
    ws = buffers.Workspace(nranks, count, proto, nranks)
    xd, stride = buffers.rows_to_device(x0)
    rng = np.random.default_rng(seed)
    s = (rng.uniform(0.5, 1.5, size=(nops, nranks)) / nranks).astype(np.float32)
    sd = torch.from_numpy(s).to("cuda")
    outd = torch.zeros((nops * nranks, stride), dtype=torch.int16, device="cuda")
    geo = abi.ar_sim_chain_geometry(ws.sim_params(nops, xd, stride, outd, stride))
    kw = dict(timeout_ns=TIMEOUT_NS)
    for _ in range(warmup):
        ws.sim_chain(nops, xd, stride, outd, stride, sd, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        ws.sim_chain(nops, xd, stride, outd, stride, sd, **kw)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if ws.status() != 0:
        raise RuntimeError(f"device status {abi.status_string(ws.status())}")
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return {
        "us_per_op": round(wall * 1e6 / (steps * nops), 4),
        "kernel_us_per_op": round(statistics.median(ms) * 1e3 / nops, 4),
        "kernel_us_per_op_p10_p90": [round(float(np.percentile(ms, 10)) * 1e3 / nops, 4),
                                     round(float(np.percentile(ms, 90)) * 1e3 / nops, 4)],
        "launch": geo["launch"], "blocks": geo["blocks"],
        "producer": "per-rank scale bf16_rne(f32(x)*s), s ~ U[0.5,1.5)/nranks",
    }


def summarize(res, proto, nranks, count, nops, steps, collective="allreduce"):
    import numpy as np
    launch_ms = res["launch_ms"]
    b_op = algorithmic_bytes(proto, nranks, count, res["nconsumers"], collective)
    avg = statistics.mean(launch_ms)
    return dict(
        us_per_op=res["wall"] * 1e6 / (steps * nops),
        ms_per_step=res["wall"] * 1e3 / steps,
        kernel_us_per_op=statistics.median(launch_ms) * 1e3 / nops,
        p10=float(np.percentile(launch_ms, 10)) * 1e3 / nops,
        p90=float(np.percentile(launch_ms, 90)) * 1e3 / nops,
        avg_launch_us=avg * 1e3,
        bytes_op=b_op, bytes_launch=b_op * nops,
        gbs=b_op * nops / (avg * 1e-3) / 1e9,
    )


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--proto", default=_env("AR_PROTO", str, "sentinel"),
                    choices=["ll", "ll128", "sentinel", "barrier", "auto"],
                    help="auto: the protocol the committed cost table chooses")
    ap.add_argument("--mode", default="system", choices=["share", "system"])
    ap.add_argument("--collective", default="allreduce",
                    choices=["allreduce", "allgather", "twoshot", "auto"],
                    help="one-shot all-reduce (default), standalone all-gather or "
                         "two-shot all-reduce (the last two: system mode)")
    ap.add_argument("--nranks", type=int, default=8)
    ap.add_argument("--rows", type=int, default=1)
    ap.add_argument("--hidden", type=int, default=4096)
    ap.add_argument("--nops", type=int, default=64)
    ap.add_argument("--waves-per-rank", type=int, default=_env("AR_WG_PER_RANK", int, 0))
    ap.add_argument("--launch", default="auto", choices=["auto", "cooperative", "ordinary"],
                    help="simulator launch: the library's choice, or forced")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-floor", action="store_true")
    ap.add_argument("--no-share", action="store_true")
    ap.add_argument("--seed", type=int, default=None,
                    help="input seed (default: that of the 8-rank [1,4096] workload)")
    ap.add_argument("--skew-us", type=float, default=0.0,
                    help="also run with a seeded producer delay U[0, D) us per (op, "
                         "producer) and report the post-arrival latency")
    ap.add_argument("--epilogue", action="store_true",
                    help="also time stream-ordered ops whose producer (a per-rank "
                         "scale) sends from its epilogue, against a separate pack")
    ap.add_argument("--chain", action="store_true",
                    help="also time the chained simulator: each op's result, scaled "
                         "per rank, is the next op's payload, in one launch")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="also run ar_probe_copy over BYTES, 3 times (reference "
                         "dispatches for hardware byte counters)")
    args = ap.parse_args()
    if TIMEOUT_NS is None:
        print(f"bench.py: {TIMEOUT_ERROR}", file=sys.stderr)
        return 2
    protos = ("ll", "ll128", "sentinel", "barrier", "auto")
    if args.proto not in protos:          # an AR_PROTO default is not checked by argparse
        print(f"bench.py: protocol {args.proto!r} (AR_PROTO?) is not one of {protos}",
              file=sys.stderr)
        return 2

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the benchmark measures "
              "N simulated ranks on ONE GPU; there is no multi-GPU path.",
              file=sys.stderr)
        return 2

    import torch

    from collective_synchronization_amd import abi, buffers, inputs
    from collective_synchronization_amd.configs import BENCH_CONFIG, CONFIGS

    torch.cuda.set_device(0)
    cfg = CONFIGS[BENCH_CONFIG]
    nranks, count, nops, proto = args.nranks, args.rows * args.hidden, args.nops, args.proto
    coll = args.collective
    selected = None
    if proto == "auto" or coll == "auto":
        # the library's choice from the committed cost table
        from collective_synchronization_amd import selector
        table = abi.cost_table(selector.load_table()["entries"])
        if coll == "auto":
            cid, pid, pred = abi.ar_select_allreduce(table, 2 * count, nranks)
            coll = selector.COLLECTIVES[cid]
            if proto == "auto":
                proto = selector.PROTOS[pid]
            else:
                pid, pred = abi.ar_select_collective(table, coll, 2 * count, nranks)
        else:
            pid, pred = abi.ar_select_collective(table, coll, 2 * count, nranks)
            proto = selector.PROTOS[pid]
        selected = {"collective": coll, "protocol": proto, "predicted_us": round(pred, 3)}
    if coll != "allreduce" and (args.mode != "system" or proto == "barrier"):
        print("bench.py: --collective allgather/twoshot run in system mode with "
              "ll, ll128 or sentinel", file=sys.stderr)
        return 2
    default_workload = (nranks, args.rows, args.hidden, nops, proto, args.mode, coll,
                        args.seed in (None, cfg["seed"])) == \
        (cfg["nranks"], 1, cfg["hidden"], cfg["nops"], "sentinel", "system", "allreduce", True)
    workload = cfg["name"] if default_workload else \
        f"n{nranks}_{proto}_{args.rows}x{args.hidden}_{nops}ops_{args.mode}" + \
        ("" if coll == "allreduce" else f"_{coll}")
    flags = {"auto": 0, "cooperative": abi.AR_SIM_COOPERATIVE,
             "ordinary": abi.AR_SIM_ORDINARY}[args.launch]

    seed = cfg["seed"] if args.seed is None else args.seed
    x = inputs.payload(seed, (nops, nranks, count), "normal")
    if args.calibrate_copy > 0:
        n = args.calibrate_copy // 16 * 16
        src = torch.ones(n // 2, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            abi.ar_probe_copy(src, dst, n)
        torch.cuda.synchronize()
        del src, dst
    try:
        res = measure(torch, abi, buffers, x, proto, nranks, count, nops, args.mode,
                      args.steps, args.warmup, args.waves_per_rank, flags, coll)
    except RuntimeError as e:
        print(f"bench.py: {e}", file=sys.stderr)
        return 1
    m = summarize(res, proto, nranks, count, nops, args.steps, coll)
    if coll == "allreduce":
        kname = ("k_sim_wide" if res["geo"]["kernel"] == "wide" else "k_sim") + \
            f"<{abi.proto_id(proto)}>"
    else:
        kname = ("k_sim_gather" if coll == "allgather" else "k_sim_twoshot") + \
            f"<{abi.proto_id(proto)}>"
    unit = "us per all-gather" if coll == "allgather" else "us per all-reduce"

    line = {
        "metric": METRIC,
        "value": round(m["us_per_op"], 4),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload, "nranks": nranks, "shape": [args.rows, args.hidden],
            "protocol": proto, "collective": coll, "ops_per_step": nops, "mode": args.mode,
            "nconsumers": res["nconsumers"], "values": "N(0,1) seed %d" % seed,
            "tile_groups_per_rank": res["geo"]["waves_per_rank"],
            "blocks": res["geo"]["blocks"], "kernel": res["geo"]["kernel"],
            "launch": res["geo"]["launch"],
            "input_sha256": inputs.sha256(x)[:16],
            "selected_by_cost_table": selected,
        },
        "kernel_us_per_op": round(m["kernel_us_per_op"], 4),
        "kernel_us_per_op_p10_p90": [round(m["p10"], 4), round(m["p90"], 4)],
        "roofline": {
            "bound": "hbm", "achieved": round(m["gbs"], 3), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(m["gbs"] / HBM_PEAK_GBS, 6),
            "traffic": load_traffic(kname),
            "kernel": kname, "avg_launch_us": round(m["avg_launch_us"], 3),
            "algorithmic_bytes_per_launch": m["bytes_launch"],
            "algorithmic_bytes_per_op": m["bytes_op"],
        },
    }

    if not args.no_share and args.mode == "system" and coll == "allreduce":
        try:
            rs = measure(torch, abi, buffers, x, proto, nranks, count, nops, "share",
                         args.steps, args.warmup, args.waves_per_rank, flags)
            ms = summarize(rs, proto, nranks, count, nops, args.steps)
            line["share_mode"] = {
                "us_per_op": round(ms["us_per_op"], 4),
                "kernel_us_per_op": round(ms["kernel_us_per_op"], 4),
                "achieved_gbs": round(ms["gbs"], 3),
                "frac": round(ms["gbs"] / HBM_PEAK_GBS, 6),
                "algorithmic_bytes_per_op": ms["bytes_op"],
            }
        except RuntimeError as e:
            line["share_mode"] = {"error": str(e)}

    if args.skew_us > 0 and args.mode == "system":
        try:
            line["skew"] = measure_skew(torch, abi, buffers, inputs, x, proto, nranks, count,
                                        nops, min(args.steps, 10), 2, args.skew_us,
                                        seed, coll)
        except RuntimeError as e:
            line["skew"] = {"error": str(e)}

    if args.epilogue:
        try:
            line["epilogue"] = measure_epilogue(torch, abi, buffers, x[0], proto, nranks,
                                                count, args.steps, args.warmup)
        except RuntimeError as e:
            line["epilogue"] = {"error": str(e)}

    if args.chain and args.mode == "system" and coll == "allreduce" and proto != "barrier":
        try:
            line["chain"] = measure_chain(torch, abi, buffers, x[0], proto, nranks, count,
                                          nops, args.steps, args.warmup)
        except RuntimeError as e:
            line["chain"] = {"error": str(e)}

    if not args.no_floor:
        threads = 64 * nranks if res["geo"]["kernel"] == "wide" else 64
        line["placement"] = measure_placement(torch, abi, res["geo"]["blocks"], threads)
        fl = measure_floor(torch, abi)
        fl["frac_of_op"] = round(fl["sol_us"] / m["kernel_us_per_op"], 4)
        fl.update(measure_launch_and_copy(torch, abi))
        if fl["copy_gbs"]:
            line["roofline"]["frac_of_copy"] = round(m["gbs"] / fl["copy_gbs"], 6)
        line["floor"] = fl
        if coll == "allreduce":
            # the same workload one op per launch: what a stream-ordered
            # caller that launches each op pays
            try:
                r1 = measure(torch, abi, buffers, x[:1], proto, nranks, count, 1, args.mode,
                             min(args.steps, 50), 3, 0, flags, coll)
                line["single_op_launch"] = {
                    "kernel_us": round(statistics.median(r1["launch_ms"]) * 1e3, 3),
                    "empty_kernel_us": fl["empty_kernel_us"]}
            except RuntimeError as e:
                line["single_op_launch"] = {"error": str(e)}

    if not args.no_cpu_baseline:
        us, ops = cpu_baseline(x, proto, args.cpu_seconds, coll)
        what = {"allreduce": "encode N + validate/decode N + fixed-order reduce",
                "allgather": "encode N + validate/decode N",
                "twoshot": "per share: encode N + validate/decode N + fixed-order "
                           "reduce + encode/decode of the reduced share"}[coll]
        line["cpu_baseline"] = {
            "value": round(us, 3), "unit": unit, "cores": 1,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": (f"{ops} ops of the same workload (N={nranks}, [{args.rows},"
                       f"{args.hidden}], {proto}: {what} for one receiving rank, "
                       f"single thread, ~{args.cpu_seconds:g} s)"),
        }

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
