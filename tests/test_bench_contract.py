"""bench.py's contract: the one-GPU guard, the algorithmic byte counts its
roofline divides by, and (on a GPU) the fields of its JSON line.

The byte counts are checked against hand-computed figures for the 8-rank
[1,4096] sentinel workload (8 KiB per payload, 8 KiB encoded) and against
encoded sizes taken from the oracle, not from the library."""
import json
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "ONE GPU" in r.stderr
    assert r.stdout == ""


def test_headline_bytes_by_hand():
    # 8 ranks, count 4096: S = 8192, sentinel E = 8192.  Inputs 8*S, every one
    # of 8 consumers receives 7 slots (written once, read once, re-armed once)
    # and writes S of output.
    S = E = 8192
    want = 8 * S + 3 * 8 * 7 * E + 8 * S
    assert want == 1_507_328
    assert bench.algorithmic_bytes("sentinel", 8, 4096, 8) == want
    # share mode: one consumer
    assert bench.algorithmic_bytes("sentinel", 8, 4096, 1) == 8 * S + 3 * 7 * E + S


@pytest.mark.parametrize("proto", ["ll", "ll128", "sentinel", "barrier"])
@pytest.mark.parametrize("nranks,count", [(4, 4096), (8, 1000), (16, 32768)])
def test_allreduce_and_allgather_bytes(proto, nranks, count):
    S = 2 * count
    E = oracle.encoded_bytes(proto, count)
    rearm = 1 if proto == "sentinel" else 0
    recv = nranks * (nranks - 1) * E
    assert bench.algorithmic_bytes(proto, nranks, count, nranks) == \
        nranks * S + (2 + rearm) * recv + nranks * S
    if proto != "barrier":
        assert bench.algorithmic_bytes(proto, nranks, count, nranks, "allgather") == \
            nranks * S + (2 + rearm) * recv + nranks * nranks * S


@pytest.mark.parametrize("proto", ["ll", "ll128", "sentinel"])
@pytest.mark.parametrize("nranks,count", [(4, 4096), (8, 1000), (16, 32768), (16, 20)])
def test_twoshot_bytes(proto, nranks, count):
    S = 2 * count
    sumE = 0
    for k in range(nranks):
        lo, hi = oracle.shard_bounds(count, nranks, k)
        sumE += oracle.encoded_bytes(proto, hi - lo) if hi > lo else 0
    rearm = 2 if proto == "sentinel" else 0
    assert bench.algorithmic_bytes(proto, nranks, count, nranks, "twoshot") == \
        2 * nranks * S + (4 + rearm) * (nranks - 1) * sumE


@pytest.mark.gpu
def test_bench_line_fields():
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "5",
           "--warmup", "1", "--cpu-seconds", "0.5"]
    print("[bench]", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    line = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 5 and line["warmup"] == 1
    assert line["higher_is_better"] is False and line["value"] > 0
    cfg = line["config"]
    assert cfg["workload"] == "n8_sweep_4MiB_oneshot_64ops"
    assert cfg["nranks"] == 8 and cfg["payload_bytes_per_rank"] == 4 << 20
    assert cfg["collective"] == "allreduce" and cfg["mode"] == "system"
    assert cfg["selected_by_cost_table"]["protocol"] == cfg["protocol"]
    roof = line["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["algorithmic_bytes_per_op"] == bench.algorithmic_bytes(
        cfg["protocol"], 8, 2 << 20, 8)
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-5
    # achieved = algorithmic bytes per launch over the average launch
    assert abs(roof["achieved"] - roof["algorithmic_bytes_per_launch"] /
               (roof["avg_launch_us"] * 1e3)) / roof["achieved"] < 1e-3
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] == 1 and cpu["value"] > 0 and cpu["cpu"]
    assert line["verified"]["bit_exact"] and line["verified"]["ops"] >= 1
    fl = line["floor"]
    assert 0 < fl["oneway_us"] < 10 and 0 < fl["load_us"] < 10
    assert fl["empty_kernel_us"] > 0 and fl["copy_gbs"] > 100
    assert line["placement"]["on_expected_xcd"] == 1.0
    assert line["placement"]["device"] and "gfx950" in line["placement"]["arch"]
    wl = line["workloads"]
    for name in ("n8_sentinel_1x4096_64ops", "n8_pick_1x4096_64ops", "n4_ll128_16x8192_160ops",
                 "n16_8x4096_64ops_oneshot", "n16_8x4096_64ops_pick",
                 "n8_sweep_4MiB_pick_64ops"):
        assert wl[name]["kernel_us_per_op"] > 0, name
        assert 0 < wl[name]["floor_frac"] and 0 < wl[name]["frac"] < 1, name
    assert wl["n4_ll_1x4096_1op_share"]["kernel_us_per_launch"] > 0
    assert wl["n8_sentinel_1x4096_64ops"]["algorithmic_bytes_per_op"] == 1_507_328
    assert wl["n8_sentinel_1x4096_64ops"]["single_op_launch"]["kernel_us"] > 0
    assert wl["n16_8x4096_64ops_pick"]["skew"]["us_per_op"] > 0


@pytest.mark.gpu
def test_bench_chain_line():
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "5",
           "--warmup", "1", "--rows", "1", "--hidden", "4096", "--proto", "sentinel",
           "--no-cpu-baseline", "--no-floor", "--chain"]
    print("[bench]", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][0])
    assert line["config"]["workload"] == "n8_sentinel_1x4096_64ops_system"
    assert line["roofline"]["algorithmic_bytes_per_op"] == 1_507_328
    ch = line["chain"]
    assert ch["kernel_us_per_op"] > 0 and ch["launch"] in ("ordinary", "cooperative")


def test_environment_overrides():
    env = dict(os.environ, AR_TIMEOUT_US="5", AR_WG_PER_RANK="16", AR_PROTO="ll")
    r = subprocess.run([sys.executable, "-c",
                        "import bench, sys; sys.argv = ['bench.py']; "
                        "print(bench.TIMEOUT_NS)"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT, env=env)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "5000"
    bad = dict(os.environ, AR_PROTO="bogus")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")],
                       capture_output=True, text=True, timeout=120, cwd=ROOT, env=bad)
    assert r.returncode == 2 and "AR_PROTO" in r.stderr and r.stdout == ""
    # the poll deadline must be positive and within the library's 60 s bound
    for v in ("-5000", "0", "6.01e7", "1e9", "abc"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")],
                           capture_output=True, text=True, timeout=120, cwd=ROOT,
                           env=dict(os.environ, AR_TIMEOUT_US=v))
        assert r.returncode == 2 and "AR_TIMEOUT_US" in r.stderr and r.stdout == "", v
