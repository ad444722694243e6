#!/usr/bin/env python3
"""Benchmark of the self-synchronizing bf16 all-reduce on one MI355X.

One step = `nops` back-to-back all-reduces run by one persistent launch of
the simulator -- encode, poll + validate, fixed-order reduce, sentinel
re-arm and epoch flip for every op.  The N simulated ranks are wave groups
placed on different XCDs; in system mode every rank runs the full per-rank
program, consume(op) -> produce(op+1), into its own receive buffer, so each
op carries the real cross-rank dependency.  Inputs are resident in HBM
before the timed region.

Headline (no arguments): the largest single-GPU workload, the top size of
the 8-rank 2 KiB-4 MiB sweep -- 8 simulated ranks, 4 MiB bf16 payloads per
rank drawn from U[-1,1), one-shot all-reduce in system mode with the
protocol the committed cost table picks (ar_select_protocol), 64 ops per
step.  Beside it, under "workloads", the other workloads at their own sizes
(8 ranks [1,4096] with the sentinel and with the table's pick, 4 ranks
[1,4096] LL one op per launch, 4 ranks [16,8192] LL128 over 160 ops,
16 ranks [8,4096] with and without producer skew, and the two-shot pick at
4 MiB), each with its fraction of the measured one-chip floor.

Options select another workload for the headline line (--nranks, --rows,
--hidden, --bytes, --proto, --collective, ...); `--collective
allgather|twoshot` times the standalone all-gather or the two-shot
all-reduce (system mode) on the same transfers.

Prints ONE JSON line: value = microseconds per all-reduce (lower is better),
with the roofline of the simulator kernel (algorithmic HBM bytes per launch /
HIP-event duration of the launch), the measured one-chip floor, and the CPU
oracle timed on the host as a baseline, whose results on the timed step's
inputs are also compared with the GPU's outputs.
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
    os.path.join(ROOT, "collective_synchronization_amd", "csrc", "ar_kernels.hip"),
    os.path.join(ROOT, "collective_synchronization_amd", "csrc", "ar_collectives.hip"),
    os.path.join(ROOT, "collective_synchronization_amd", "csrc", "ar_linear.hip"),
    os.path.join(ROOT, "include", "ar_protocols.h"),
    os.path.join(ROOT, "include", "ar_device.h"),
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


def cpu_baseline_checked(torch, x, proto, collective, outd, nconsumers, seconds):
    """The oracle on the timed step's inputs, one op at a time, single
    thread: every op once, compared with every consumer's GPU output of that
    op (not timed), then the ops again in order until about `seconds` of
    oracle time.  Returns (microseconds per op, ops timed, ops compared,
    consumer outputs that differ)."""
    import numpy as np
    import oracle
    K, n, count = x.shape
    run = oracle.twoshot if collective == "twoshot" else oracle.allreduce
    spent, ops, bad, i = 0.0, 0, 0, 0
    while True:
        t0 = time.perf_counter()
        st, want = run(x[i % K], proto, 1)
        spent += time.perf_counter() - t0
        ops += 1
        if st != oracle.READY:
            raise RuntimeError(f"oracle op {i % K} not ready: status {st}")
        if i < K:
            w = torch.from_numpy(want.view(np.int16)).to(outd.device)
            got = outd[i * nconsumers:(i + 1) * nconsumers, :count]
            bad += int((got != w[None, :]).any(dim=1).sum().item())
        i += 1
        if i >= K and spent >= seconds:
            break
    return spent * 1e6 / ops, ops, min(K, i), bad


def kernel_label(proto, nranks, geo, mode, collective):
    """Name of the simulator kernel variant a launch ran (the key of its
    counter summary in profiles/traffic.json)."""
    from collective_synchronization_amd import abi
    pid = abi.proto_id(proto)
    nmax = 4 if nranks <= 4 else (8 if nranks <= 8 else 16)
    if collective == "allgather":
        return f"k_sim_gather<{pid},{nmax}>"
    if collective == "twoshot":
        return ("k_sim_twoshot" if geo["kernel"] == "wide" else "k_sim_twoshot_narrow") + \
            f"<{pid},{nmax}>"
    one = geo["tiles_per_wave"] <= 1 and (geo["kernel"] == "wide" or proto != "barrier")
    if geo["kernel"] == "wide":
        return f"k_sim_wide<{pid},{nmax},{mode},{1 if one else 2}>"
    return f"k_sim<{pid},{nmax},{mode},{'one' if one else 'many'}>"


def load_traffic(kernel_name: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel (None: the one kernel summarized for the workload) on this
    workload, if it was taken on the current kernel source."""
    try:
        with open(PROFILE_TRAFFIC) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if kernel_name is None:        # whichever kernel that workload ran
        ents = [v for k, v in t.items() if k.endswith("@" + workload)]
        ent = ents[0] if len(ents) == 1 else None
    else:
        ent = t.get(f"{kernel_name}@{workload}")
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def measure(torch, abi, buffers, x, proto, nranks, count, nops, mode, steps, warmup,
            waves_per_rank=0, flags=0, collective="allreduce", keep=False):
    """Time `steps` launches of the simulator (one step = nops ops).

    Returns per-launch HIP-event durations (ms, on the launch stream), the
    wall-clock duration of the timed region (s), geometry and status; with
    `keep`, also the output buffer, which then holds the last timed step."""
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
    del xd, ws
    return dict(launch_ms=launch_ms, wall=wall, geo=geo, nconsumers=nconsumers,
                out=outd if keep else None)


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
    """Ops with a seeded producer delay U[0, skew_us) per (op, producer)
    (none when skew_us is 0) and the wall-clock trace: per-op time, the
    post-arrival latency (op done at the last consumer minus the last
    producer's last store), and the first op's timeline from the first wave's
    start.  The trace makes every sender wait for its stores before its
    timestamp, so these runs are slower than the untraced ones."""
    import numpy as np
    xd, stride = buffers.rows_to_device(x)
    ws = buffers.Workspace(nranks, count, proto, nranks, collective=collective)
    ostride = ws.gather_stride() if collective == "allgather" else stride
    outd = torch.zeros((nops * nranks, ostride), dtype=torch.int16, device="cuda")
    hz = abi.ar_wallclock_hz()
    ticks = None
    d_us = np.zeros((nops, nranks))
    if skew_us > 0:
        d_us = inputs.delays_us(seed + 1, nops, nranks, skew_us)
        ticks = torch.from_numpy(np.round(d_us * hz * 1e-6).astype(np.int32)).to("cuda")
    trace = torch.zeros(nops * 2 * nranks + 1, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    post, per_op, first_store, first_done, last_done = [], [], [], [], []
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
        raw = trace.cpu().numpy()
        start = float(raw[-1])
        t = raw[:-1].reshape(nops, 2, nranks).astype(np.float64)
        post.extend(((t[:, 1, :].max(axis=1) - t[:, 0, :].max(axis=1)) / hz * 1e6).tolist())
        first_store.append((t[0, 0, :].max() - start) / hz * 1e6)
        first_done.append((t[0, 1, :].max() - start) / hz * 1e6)
        last_done.append((t[-1, 1, :].max() - start) / hz * 1e6)
        per_op.append(a.elapsed_time(b) * 1e3 / nops)
    return {"skew_us": skew_us, "mean_delay_us": round(float(d_us.mean()), 3),
            "us_per_op": round(statistics.median(per_op), 3),
            "post_arrival_us_median": round(float(np.median(post)), 3),
            "post_arrival_us_p90": round(float(np.percentile(post, 90)), 3),
            "timeline_us": {"first_op_last_store": round(float(np.median(first_store)), 3),
                            "first_op_done": round(float(np.median(first_done)), 3),
                            "last_op_done": round(float(np.median(last_done)), 3)}}


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


def measure_graph(torch, abi, buffers, x, proto, nranks, count, steps):
    """Calls captured in a HIP graph against the same calls issued eagerly.
    Two sequences of K = x.shape[0] ops (system mode): K one-op persistent
    launches (ar_sim_run), and K stream-ordered pack + reduce pairs; each
    sequence starts with ar_state_reset, which makes its replays sound (a
    replay repeats the captured epochs).  Eagerly, the arguments of every
    call are built before the timed region, and the sequence starts from the
    same reset.  Microseconds per op: HIP events around a replay, or around
    the eager sequence, on the launch stream; median over `steps`.  proto:
    LL, LL128 or SENTINEL (the barrier baseline's launches need a counter
    reset each)."""
    import ctypes
    if proto not in ("ll", "ll128", "sentinel"):
        raise RuntimeError(f"graph replay timing: no {proto} sequence")
    K = x.shape[0]
    xd, stride = buffers.rows_to_device(x)
    stream = torch.cuda.current_stream()
    lib = abi.raw()
    pack = getattr(lib, {"ll": "ar_pack_ll", "ll128": "ar_pack_ll128",
                         "sentinel": "ar_pack_sentinel"}[proto])
    flags = abi.AR_FLAG_REARM if proto == "sentinel" else 0
    out = {"ops": K}
    for kind in ("one_op_launches", "pack_reduce"):
        ws = buffers.Workspace(nranks, count, proto, nranks)
        outd = torch.zeros((K * nranks, stride), dtype=torch.int16, device="cuda")
        rows = [(xd[j * nranks:].data_ptr(), outd[j * nranks:].data_ptr()) for j in range(K)]
        calls = []
        for j in range(K):
            if kind == "one_op_launches":
                p = ws.sim_params(1, rows[j][0], stride, rows[j][1], stride,
                                  timeout_ns=TIMEOUT_NS)
                calls.append(lambda sh, p=p: lib.ar_sim_run(ctypes.byref(p), sh))
            else:
                e = abi.ar_epoch(ws.epoch.seq, ws.epoch.parity)
                d = ws.desc
                calls.append(lambda sh, j=j, e=e, d=d: (
                    pack(ctypes.byref(d), rows[j][0], stride, ws.scratch.data_ptr(), e, sh),
                    lib.ar_reduce_validate(ctypes.byref(d), ws.scratch.data_ptr(), rows[j][1],
                                           stride, e, ws.ctrl.data_ptr(), TIMEOUT_NS, flags,
                                           sh)))
            ws.flip()

        def seq():
            # the current stream: under capture, the capturing one
            sh = torch.cuda.current_stream().cuda_stream
            ws.reset_state(sh)
            for c in calls:
                r = c(sh)
                if (r if isinstance(r, int) else min(r)) != abi.AR_OK:
                    raise RuntimeError(f"{kind}: call returned {r}")

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            seq()
        res = {}
        ref = None
        for mode in ("eager", "graph"):
            if mode == "graph":               # the replays must write what eager calls wrote
                ref = outd.clone()
                outd.fill_(-1)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                  for _ in range(steps + 2)]
            for k, (a, b) in enumerate(ev):
                torch.cuda.synchronize()
                a.record(stream)
                if mode == "graph":
                    g.replay()
                else:
                    seq()
                b.record(stream)
            torch.cuda.synchronize()
            if ws.status() != 0:
                raise RuntimeError(f"{kind} {mode}: device status "
                                   f"{abi.status_string(ws.status())}")
            res[mode] = round(statistics.median(a.elapsed_time(b) for a, b in ev[2:])
                              * 1e3 / K, 3)
        if not torch.equal(outd, ref):
            raise RuntimeError(f"{kind}: graph replays wrote other outputs than eager calls")
        out[kind + "_us_per_op"] = res
        del g
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


def linear_bytes(proto: str, nranks: int, count: int) -> int:
    """Algorithmic bytes of one op of the chain whose producer is a
    row-parallel linear shard: every rank's weight rows over its input slice
    (count x count/nranks bf16), its slice of the layer input, and the
    one-shot exchange without the producer's payload read (the payload is
    made in registers)."""
    kr = count // nranks
    return (nranks * count * kr * 2 + nranks * kr * 2 +
            algorithmic_bytes(proto, nranks, count, nranks) - nranks * 2 * count)


def measure_linear(torch, abi, buffers, inputs, proto, nranks, count, nops, layers, steps,
                   warmup, flags=0, seed=5200):
    """The chain whose producer is one decode token's row-parallel linear
    shard (ar_sim_linear_run): op i's payload of rank r is its shard of a
    layer applied to its slice of op i-1's result; `layers` layers of
    N(0, 1/count) weights taken in turn.  HIP events per launch on the
    launch stream, median over `steps` launches, plus the wall clock."""
    import numpy as np
    ws = buffers.Workspace(nranks, count, proto, nranks)
    x0 = inputs.payload(seed, (nranks, count), "normal")
    xd, stride = buffers.rows_to_device(x0)
    w = inputs.weights(seed + 7, layers, nranks, count)
    wd = torch.from_numpy(w.view(np.int16)).to("cuda")
    del w
    outd = torch.zeros((nops * nranks, stride), dtype=torch.int16, device="cuda")
    geo = abi.ar_sim_linear_geometry(ws.sim_params(nops, xd, stride, outd, stride, flags=flags),
                                     wd, layers, ws.linear_work())
    kw = dict(timeout_ns=TIMEOUT_NS, flags=flags)
    for _ in range(warmup):
        ws.sim_linear(nops, xd, stride, outd, stride, wd, layers, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        ws.sim_linear(nops, xd, stride, outd, stride, wd, layers, **kw)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if ws.status() != 0:
        raise RuntimeError(f"device status {abi.status_string(ws.status())}")
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    k_us = statistics.median(ms) * 1e3 / nops
    kr = count // nranks
    nmax = 4 if nranks <= 4 else (8 if nranks <= 8 else 16)
    b_op = linear_bytes(proto, nranks, count)
    kname = f"k_sim_linear<{abi.proto_id(proto)},{nmax},{kr // 64}>"
    wname = f"n{nranks}_linear_{proto}_1x{count}_{nops}ops"
    return {
        "nranks": nranks, "shape": [1, count], "protocol": proto, "ops_per_launch": nops,
        "layers": layers, "weight_bytes_per_layer": nranks * count * kr * 2,
        "us_per_op": round(wall * 1e6 / (steps * nops), 4),
        "kernel_us_per_op": round(k_us, 4),
        "kernel_us_per_op_p10_p90": [round(float(np.percentile(ms, 10)) * 1e3 / nops, 4),
                                     round(float(np.percentile(ms, 90)) * 1e3 / nops, 4)],
        "algorithmic_bytes_per_op": b_op,
        "achieved_gbs": round(b_op / (k_us * 1e-6) / 1e9, 3),
        "frac": round(b_op / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 6),
        "avg_launch_us": round(statistics.mean(ms) * 1e3, 3),
        "launch": geo["launch"], "blocks": geo["blocks"], "gemv_workgroups": geo["workers"],
        "kernel": kname, "workload": wname,
        # counters of the same kernel and workload; rocprofv3 records nothing
        # for cooperative launches here, so the summary is of the ordinary
        # launch (bench.py --linear --launch ordinary)
        "traffic": (load_traffic(kname, wname + "_ordinary")
                    if geo["launch"] == "ordinary" else None),
        "traffic_ordinary_launch": load_traffic(kname, wname + "_ordinary"),
        "producer": ("row-parallel linear shard of a decode token: pairwise binary32 dot "
                     f"products over {kr} inputs per rank, bf16; weights N(0,1/{count}), "
                     f"{layers} layers in turn"),
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


SWEEP_SEED = 1004                 # seed of the 2 KiB-4 MiB sweep: SWEEP_SEED + bytes
HEADLINE = "n8_sweep_4MiB_oneshot_64ops"


def named_workloads():
    """The workloads of the default line: name -> (nranks, rows, hidden, dist,
    seed, nops, proto, collective, mode).  proto "auto": the committed cost
    table's one-shot pick (ar_select_protocol); collective "auto": its
    all-reduce pick (ar_select_allreduce)."""
    from collective_synchronization_amd.configs import CONFIGS
    c1, c2 = CONFIGS["n4_ll_1x4096"], CONFIGS["n8_sentinel_1x4096_64ops"]
    c3, c4 = CONFIGS["n4_ll128_Bx8192_160ops"], CONFIGS["n8_sweep_2KiB_4MiB"]
    c5 = CONFIGS["n16_skew_8x4096_64ops"]
    top = max(c4["sizes"])
    return {
        HEADLINE: (c4["nranks"], 1, top // 2, c4["dist"], c4["seed"] + top, 64, "auto",
                   "allreduce", "system"),
        "n8_sweep_4MiB_pick_64ops": (c4["nranks"], 1, top // 2, c4["dist"], c4["seed"] + top,
                                     64, "auto", "auto", "system"),
        c2["name"]: (c2["nranks"], 1, c2["hidden"], c2["dist"], c2["seed"], c2["nops"],
                     "sentinel", "allreduce", "system"),
        "n8_pick_1x4096_64ops": (c2["nranks"], 1, c2["hidden"], c2["dist"], c2["seed"],
                                 c2["nops"], "auto", "auto", "system"),
        "n4_ll_1x4096_1op_share": (c1["nranks"], 1, c1["hidden"], c1["dist"], c1["seed"], 1,
                                   "ll", "allreduce", "share"),
        "n4_ll128_16x8192_160ops": (c3["nranks"], 16, c3["hidden"], c3["dist"], c3["seed"] + 16,
                                    c3["nops"], "ll128", "allreduce", "system"),
        "n16_8x4096_64ops_oneshot": (c5["nranks"], 8, c5["hidden"], c5["dist"], c5["seed"],
                                     c5["nops"], "auto", "allreduce", "system"),
        "n16_8x4096_64ops_pick": (c5["nranks"], 8, c5["hidden"], c5["dist"], c5["seed"],
                                  c5["nops"], "auto", "auto", "system"),
    }


def workload_name(nranks, proto, rows, hidden, nops, mode, coll, waves_per_rank=0,
                  launch="auto"):
    """Name of a workload given on the command line (the key of its counter
    summary in profiles/traffic.json)."""
    return (f"n{nranks}_{proto}_{rows}x{hidden}_{nops}ops_{mode}" +
            ("" if coll == "allreduce" else f"_{coll}") +
            ("" if waves_per_rank == 0 else f"_wpr{waves_per_rank}") +
            ("" if launch == "auto" else f"_{launch}"))


def resolve(abi, proto, coll, count, nranks):
    """The protocol and collective a workload runs; with "auto", the
    committed cost table's choice.  Returns (proto, coll, selected or None)."""
    if proto != "auto" and coll != "auto":
        return proto, coll, None
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
    return proto, coll, {"collective": coll, "protocol": proto, "predicted_us": round(pred, 3)}


def side_workload(torch, abi, buffers, inputs, name, wl, steps, warmup, floor_us, skew_us=0.0):
    """One extra workload of the default line: per-op time, algorithmic
    GB/s, its fraction of 8 TB/s and of the one-chip floor."""
    nranks, rows, hidden, dist, seed, nops, proto, coll, mode = wl
    count = rows * hidden
    proto, coll, selected = resolve(abi, proto, coll, count, nranks)
    x = inputs.payload(seed, (nops, nranks, count), dist)
    out = {"nranks": nranks, "shape": [rows, hidden], "protocol": proto, "collective": coll,
           "mode": mode, "ops_per_launch": nops}
    if selected:
        out["selected_by_cost_table"] = selected
    if nops == 1:
        # one op per launch: what a stream-ordered caller pays per op
        r = measure(torch, abi, buffers, x, proto, nranks, count, 1, mode, max(steps, 30),
                    warmup, collective=coll)
        us = statistics.median(r["launch_ms"]) * 1e3
        out.update({"kernel_us_per_launch": round(us, 3),
                    "kernel_us_per_launch_p10_p90": [
                        round(float(statistics.quantiles(r["launch_ms"], n=10)[0]) * 1e3, 3),
                        round(float(statistics.quantiles(r["launch_ms"], n=10)[-1]) * 1e3, 3)]})
        return out
    r = measure(torch, abi, buffers, x, proto, nranks, count, nops, mode, steps, warmup,
                collective=coll)
    m = summarize(r, proto, nranks, count, nops, steps, coll)
    kname = kernel_label(proto, nranks, r["geo"], mode, coll)
    out.update({
        "us_per_op": round(m["us_per_op"], 4),
        "kernel_us_per_op": round(m["kernel_us_per_op"], 4),
        "kernel_us_per_op_p10_p90": [round(m["p10"], 4), round(m["p90"], 4)],
        "achieved_gbs": round(m["gbs"], 3), "frac": round(m["gbs"] / HBM_PEAK_GBS, 6),
        "algorithmic_bytes_per_op": m["bytes_op"],
        "floor_frac": round(floor_us / m["kernel_us_per_op"], 4) if floor_us else None,
        "kernel": kname,
        "launch": r["geo"]["launch"],
        # the same workload run on its own: `bench.py --nranks ... --rows ...`
        "traffic": load_traffic(kname, workload_name(nranks, proto, rows, hidden, nops, mode,
                                                     coll)),
    })
    if r["geo"]["launch"] == "cooperative":
        # the profiler records no cooperative launch: the counters of the
        # same workload launched ordinarily (`... --launch ordinary`)
        out["traffic_ordinary_launch"] = load_traffic(
            None, workload_name(nranks, proto, rows, hidden, nops, mode, coll,
                                launch="ordinary"))
    if skew_us > 0:
        out["skew"] = measure_skew(torch, abi, buffers, inputs, x, proto, nranks, count, nops,
                                   min(steps, 10), 2, skew_us, seed, coll)
    return out


def main() -> int:
    if TIMEOUT_NS is None:
        print(f"bench.py: {TIMEOUT_ERROR}", file=sys.stderr)
        return 2
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--proto", default=_env("AR_PROTO", str, "auto"),
                    help="ll, ll128, sentinel, barrier, or auto: the protocol the "
                         "committed cost table chooses")
    ap.add_argument("--mode", default="system", choices=["share", "system"])
    ap.add_argument("--collective", default="allreduce",
                    choices=["allreduce", "allgather", "twoshot", "auto"],
                    help="one-shot all-reduce (default), standalone all-gather or "
                         "two-shot all-reduce (the last two: system mode); auto: the "
                         "cost table's all-reduce choice")
    ap.add_argument("--nranks", type=int, default=8)
    ap.add_argument("--bytes", type=int, default=None,
                    help="payload bytes per rank (a [1, bytes/2] payload), instead of "
                         "--rows x --hidden")
    ap.add_argument("--rows", type=int, default=None)
    ap.add_argument("--hidden", type=int, default=None)
    ap.add_argument("--nops", type=int, default=64)
    ap.add_argument("--dist", default=None, choices=["normal", "uniform"],
                    help="payload values (default: U[-1,1) for --bytes payloads, N(0,1) "
                         "for [rows, hidden] ones)")
    ap.add_argument("--waves-per-rank", type=int, default=_env("AR_WG_PER_RANK", int, 0))
    ap.add_argument("--launch", default="auto", choices=["auto", "cooperative", "ordinary"],
                    help="simulator launch: the library's choice, or forced")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-floor", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline line: no other workloads, share mode or "
                         "single-op launches")
    ap.add_argument("--seed", type=int, default=None,
                    help="input seed (default: that of the workload)")
    ap.add_argument("--skew-us", type=float, default=0.0,
                    help="also run with a seeded producer delay U[0, D) us per (op, "
                         "producer) and report the post-arrival latency")
    ap.add_argument("--timeline", action="store_true",
                    help="also run with the wall-clock trace and no delays: the first "
                         "op's last store and completion after the first wave's start")
    ap.add_argument("--epilogue", action="store_true",
                    help="also time stream-ordered ops whose producer (a per-rank "
                         "scale) sends from its epilogue, against a separate pack")
    ap.add_argument("--chain", action="store_true",
                    help="also time the chained simulator: each op's result, scaled "
                         "per rank, is the next op's payload, in one launch")
    ap.add_argument("--linear", action="store_true",
                    help="also time the chain whose producer is a row-parallel linear "
                         "layer shard (each op's result is the next layer's input), in "
                         "one launch, with the --proto protocol (auto: LL)")
    ap.add_argument("--linear-hidden", type=int, default=4096,
                    help="hidden size of --linear (its own workload: --nranks ranks, one "
                         "decode token, 64 ops)")
    ap.add_argument("--layers", type=int, default=16,
                    help="weight layers of --linear, taken in turn (default 16: 512 MiB "
                         "at 8 ranks and hidden 4096, more than the memory-side cache)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="also run ar_probe_copy over BYTES, 3 times (reference "
                         "dispatches for hardware byte counters)")
    args = ap.parse_args()
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

    torch.cuda.set_device(0)
    named = named_workloads()
    h_nranks, _, h_hidden, h_dist, h_seed, _, _, _, _ = named[HEADLINE]
    shaped = args.rows is not None or args.hidden is not None
    if args.bytes is not None and shaped:
        print("bench.py: give --bytes or --rows/--hidden, not both", file=sys.stderr)
        return 2
    if shaped:
        rows, hidden = args.rows or 1, args.hidden or 4096
        dist = args.dist or "normal"
    else:
        nbytes = args.bytes if args.bytes is not None else 2 * h_hidden
        if nbytes <= 0 or nbytes % 2:
            print("bench.py: --bytes must be a positive even number", file=sys.stderr)
            return 2
        rows, hidden = 1, nbytes // 2
        dist = args.dist or "uniform"
    nranks, count, nops = args.nranks, rows * hidden, args.nops
    proto, coll, selected = resolve(abi, args.proto, args.collective, count, nranks)
    if coll != "allreduce" and (args.mode != "system" or proto == "barrier"):
        print("bench.py: --collective allgather/twoshot run in system mode with "
              "ll, ll128 or sentinel", file=sys.stderr)
        return 2
    default_workload = (nranks, rows, hidden, nops, args.proto, args.mode, args.collective,
                        dist, args.seed in (None, h_seed), args.waves_per_rank,
                        args.launch) == (h_nranks, 1, h_hidden, 64, "auto", "system",
                                         "allreduce", h_dist, True, 0, "auto")
    if default_workload:
        workload = HEADLINE
        seed = h_seed
    else:
        seed = args.seed if args.seed is not None else (
            SWEEP_SEED + 2 * count if not shaped else 1002)
        workload = workload_name(nranks, proto, rows, hidden, nops, args.mode, coll,
                                 args.waves_per_rank, args.launch)
    flags = {"auto": 0, "cooperative": abi.AR_SIM_COOPERATIVE,
             "ordinary": abi.AR_SIM_ORDINARY}[args.launch]

    x = inputs.payload(seed, (nops, nranks, count), dist)
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
                      args.steps, args.warmup, args.waves_per_rank, flags, coll,
                      keep=not args.no_cpu_baseline)
    except RuntimeError as e:
        print(f"bench.py: {e}", file=sys.stderr)
        return 1
    m = summarize(res, proto, nranks, count, nops, args.steps, coll)
    kname = kernel_label(proto, nranks, res["geo"], args.mode, coll)
    unit = "us per all-gather" if coll == "allgather" else "us per all-reduce"
    # the same op counted with every rank's slot in every consumer's
    # buffer, its own included (the kernels keep a rank's own chunk in
    # registers, so `achieved` counts N-1 slots per consumer)
    n2_bytes = None
    if coll == "allreduce":
        E = abi.ar_encoded_bytes(proto, count)
        nc = res["nconsumers"]
        n2_bytes = 2 * nranks * 2 * count + 2 * nc * nranks * E + \
            (nc * nranks * E if proto == "sentinel" else 0) - (nranks - nc) * 2 * count
    avg_s = m["avg_launch_us"] * 1e-6

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
            "workload": workload, "nranks": nranks, "shape": [rows, hidden],
            "payload_bytes_per_rank": 2 * count,
            "protocol": proto, "collective": coll, "ops_per_step": nops, "mode": args.mode,
            "nconsumers": res["nconsumers"],
            "values": ("U[-1,1)" if dist == "uniform" else "N(0,1)") + f" seed {seed}",
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
            "traffic": load_traffic(kname, workload),
            "kernel": kname, "avg_launch_us": round(m["avg_launch_us"], 3),
            "algorithmic_bytes_per_launch": m["bytes_launch"],
            "algorithmic_bytes_per_op": m["bytes_op"],
            "frac_all_slots": (round(n2_bytes * nops / avg_s / 1e9 / HBM_PEAK_GBS, 6)
                                  if n2_bytes else None),
        },
    }

    if selected:
        # the committed table's regret: on its own points and on held-out
        # sizes it was not fitted to
        from collective_synchronization_amd import selector
        t = selector.load_table()
        line["selector"] = {"in_sample_max_regret": round(t["max_regret"], 4),
                            "heldout_max_regret": (round(t["heldout_max_regret"], 4)
                                                   if "heldout_max_regret" in t else None),
                            "heldout_sizes": t.get("heldout_sizes")}

    fl = None
    if not args.no_floor:
        threads = 64 * nranks if res["geo"]["kernel"] == "wide" else 64
        line["placement"] = measure_placement(torch, abi, res["geo"]["blocks"], threads)
        fl = measure_floor(torch, abi)
        fl["frac_of_op"] = round(fl["sol_us"] / m["kernel_us_per_op"], 4)
        fl.update(measure_launch_and_copy(torch, abi))
        if fl["copy_gbs"]:
            line["roofline"]["frac_of_copy"] = round(m["gbs"] / fl["copy_gbs"], 6)
        line["floor"] = fl

    if not args.no_extras and default_workload:
        floor_us = fl["sol_us"] if fl else None
        side = {}
        for name, wl in named.items():
            if name == HEADLINE:
                continue
            try:
                skew = 20.0 if name == "n16_8x4096_64ops_pick" else 0.0
                side[name] = side_workload(torch, abi, buffers, inputs, name, wl,
                                           args.steps, args.warmup, floor_us, skew)
            except RuntimeError as e:
                side[name] = {"error": str(e)}
        # share mode (rank 0's receive side) and one op per launch of the
        # 8-rank [1,4096] sentinel workload
        c2 = named["n8_sentinel_1x4096_64ops"]
        x2 = inputs.payload(c2[4], (c2[5], c2[0], c2[2]), c2[3])
        try:
            rs = measure(torch, abi, buffers, x2, "sentinel", c2[0], c2[2], c2[5], "share",
                         args.steps, args.warmup)
            ms = summarize(rs, "sentinel", c2[0], c2[2], c2[5], args.steps)
            side["n8_sentinel_1x4096_64ops"]["share_mode"] = {
                "kernel_us_per_op": round(ms["kernel_us_per_op"], 4),
                "achieved_gbs": round(ms["gbs"], 3)}
            r1 = measure(torch, abi, buffers, x2[:1], "sentinel", c2[0], c2[2], 1, "system",
                         max(args.steps, 30), 3)
            side["n8_sentinel_1x4096_64ops"]["single_op_launch"] = {
                "kernel_us": round(statistics.median(r1["launch_ms"]) * 1e3, 3),
                "empty_kernel_us": fl["empty_kernel_us"] if fl else None}
        except (RuntimeError, KeyError) as e:
            side["n8_sentinel_1x4096_64ops"]["share_mode"] = {"error": str(e)}
        # the same 64 ops as one-op launches and as stream-ordered pairs,
        # captured in a HIP graph and replayed, against eager calls
        try:
            side["n8_sentinel_1x4096_64ops"]["graph_replay"] = measure_graph(
                torch, abi, buffers, x2, "sentinel", c2[0], c2[2], max(args.steps, 20))
        except (RuntimeError, abi.ArError) as e:
            side["n8_sentinel_1x4096_64ops"]["graph_replay"] = {"error": str(e)}
        # the decode chain whose producer is a row-parallel linear layer (8
        # ranks, hidden 4096, LL, 64 ops over 16 layers of weights)
        try:
            side["n8_linear_ll_1x4096_64ops"] = measure_linear(
                torch, abi, buffers, inputs, "ll", c2[0], c2[2], c2[5], 16, args.steps,
                args.warmup)
        except (RuntimeError, ValueError, abi.ArError) as e:
            side["n8_linear_ll_1x4096_64ops"] = {"error": str(e)}
        line["workloads"] = side

    if args.timeline and args.mode == "system":
        try:
            line["timeline"] = measure_skew(torch, abi, buffers, inputs, x, proto, nranks,
                                            count, nops, min(args.steps, 30), 2, 0.0, seed,
                                            coll)
        except RuntimeError as e:
            line["timeline"] = {"error": str(e)}

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

    if args.linear and args.mode == "system" and (args.proto == "auto" or proto != "barrier"):
        try:
            line["linear"] = measure_linear(torch, abi, buffers, inputs,
                                            "ll" if args.proto == "auto" else proto, nranks,
                                            args.linear_hidden, 64, args.layers,
                                            args.steps, args.warmup, flags)
        except (RuntimeError, ValueError, abi.ArError) as e:
            line["linear"] = {"error": str(e)}

    if not args.no_cpu_baseline:
        if coll == "allgather":
            us, ops = cpu_baseline(x, proto, args.cpu_seconds, coll)
            checked = None
        else:
            us, ops, compared, bad = cpu_baseline_checked(torch, x, proto, coll, res["out"],
                                                          res["nconsumers"], args.cpu_seconds)
            checked = {"ops": compared, "consumers": res["nconsumers"],
                       "mismatched_consumer_ops": bad, "bit_exact": bad == 0}
        what = {"allreduce": "encode N + validate/decode N + fixed-order reduce",
                "allgather": "encode N + validate/decode N",
                "twoshot": "per share: encode N + validate/decode N + fixed-order "
                           "reduce + encode/decode of the reduced share"}[coll]
        line["cpu_baseline"] = {
            "value": round(us, 3), "unit": unit, "cores": 1,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": (f"{ops} ops over the timed step's {nops} inputs (N={nranks}, "
                       f"[{rows},{hidden}], {proto}: {what} for one receiving rank, "
                       f"single thread, ~{args.cpu_seconds:g} s or every op once)"),
        }
        if checked is not None:
            line["verified"] = checked
            if bad:
                print(f"bench.py: {bad} consumer outputs of the timed step differ from "
                      "the oracle", file=sys.stderr)
                print(json.dumps(line), flush=True)
                return 1

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
