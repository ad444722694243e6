"""GPU tests of the ordering probes, the floor probes and the launch modes.

The protocols order device-scope coherent (sc1) accesses with a wait for
outstanding memory operations rather than a full cache-flushing fence; the
litmus probe checks the three orderings they rely on between waves on
different XCDs (message passing, LL word atomicity, re-arm before refill).
"""
import numpy as np
import pytest
import torch

import oracle
from collective_synchronization_amd import abi, buffers, inputs

pytestmark = pytest.mark.gpu


def _litmus(kind, xa, xb, iters):
    work = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    res = torch.zeros(8, dtype=torch.int64, device="cuda")
    abi.ar_probe_litmus(work, iters, xa, xb, kind, res)
    torch.cuda.synchronize()
    return res.cpu().tolist()


@pytest.mark.parametrize("kind,iters", [(0, 50000), (1, 50000), (2, 20000)])
@pytest.mark.parametrize("xa,xb", [(0, 1), (2, 6), (7, 4)])
def test_litmus_no_violation(kind, xa, xb, iters):
    print(f"[litmus] kind={kind} xcd {xa}->{xb}", flush=True)
    r = _litmus(kind, xa, xb, iters)
    viol, obs, xcc_a, xcc_b, status, last, second = r[:7]
    print(f"  observations={obs} xcc=({xcc_a},{xcc_b}) 16B-split={second}", flush=True)
    assert status == 0
    assert obs > 0 and last == iters
    assert viol == 0
    assert 0 <= xcc_a < 8 and 0 <= xcc_b < 8


def test_litmus_argument_checks():
    work = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    res = torch.zeros(8, dtype=torch.int64, device="cuda")
    with pytest.raises(abi.ArError):
        abi.ar_probe_litmus(work, 10, 3, 3, 0, res)
    with pytest.raises(abi.ArError):
        abi.ar_probe_litmus(work, 10, 0, 1, 5, res)


def test_floor_probes():
    hz = abi.ar_wallclock_hz()
    assert hz > 1e6
    work = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    res = torch.zeros(8, dtype=torch.int64, device="cuda")
    abi.ar_probe_pingpong(work, 500, 0, 3, res)
    torch.cuda.synchronize()
    r = res.cpu().tolist()
    assert r[4] == 0 and r[1] == 500
    rtt_us = r[0] / 500 / hz * 1e6
    assert 0.01 < rtt_us < 100
    chain = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    res.zero_()
    abi.ar_probe_loadchain(chain, 1 << 22, 500, res)
    torch.cuda.synchronize()
    r = res.cpu().tolist()
    assert r[1] == 500 and 0.01 < r[0] / 500 / hz * 1e6 < 100


def test_copy_probe():
    src = torch.randint(-2 ** 15, 2 ** 15, (1 << 20,), dtype=torch.int16, device="cuda")
    dst = torch.zeros_like(src)
    abi.ar_probe_copy(src, dst, src.numel() * 2)
    abi.ar_probe_empty()
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("proto", ["ll", "ll128", "sentinel", "barrier"])
@pytest.mark.parametrize("nranks,count", [(8, 4096), (16, 4096), (16, 32768 + 3)])
def test_sim_cooperative_launch(proto, nranks, count):
    """A cooperative launch may fill the occupancy the runtime reports (an
    ordinary one keeps half), so its grid is at least as large."""
    nops = 6
    ws = buffers.Workspace(nranks, count, proto, nranks)
    x = inputs.payload(77 + count, (nops, nranks, count), "normal")
    xd, stride = buffers.rows_to_device(x)
    outd = torch.zeros((nops * nranks, stride), dtype=torch.int16, device="cuda")
    coop = abi.ar_sim_geometry(ws.sim_params(nops, xd, stride, outd, stride,
                                             flags=abi.AR_SIM_COOPERATIVE))
    plain = abi.ar_sim_geometry(ws.sim_params(nops, xd, stride, outd, stride))
    print(f"[coop] {proto} N={nranks} count={count} coop={coop} plain={plain}", flush=True)
    if coop["kernel"] == plain["kernel"]:
        assert coop["blocks"] >= plain["blocks"]
        assert coop["tiles_per_wave"] <= plain["tiles_per_wave"]
    ws.sim(nops, xd, stride, outd, stride, timeout_ns=2_000_000_000,
           flags=abi.AR_SIM_COOPERATIVE)
    torch.cuda.synchronize()
    assert ws.status() == 0
    got = buffers.rows_from_device(outd, count, (nops, nranks))
    want = oracle.allreduce_ops(x, proto)
    for i in range(nops):
        for c in range(nranks):
            assert np.array_equal(got[i, c], want[i]), (i, c)


def test_sim_launch_choice():
    """Without a launch flag the library launches cooperatively when the
    launch holds at least 32 ops and the cooperative grid lets each workgroup
    walk fewer tiles (16 ranks, LL, [1,4096]: 2 tiles at half the occupancy,
    1 at all of it); otherwise, or with AR_SIM_ORDINARY, ordinarily."""
    nranks, count = 16, 4096
    ws = buffers.Workspace(nranks, count, "ll", nranks)
    xd = torch.zeros((64 * nranks, count), dtype=torch.int16, device="cuda")
    outd = torch.zeros_like(xd)

    def geo(nops, flags=0):
        return abi.ar_sim_geometry(ws.sim_params(nops, xd, count, outd, count, flags=flags))

    long_auto, short_auto = geo(64), geo(8)
    forced_ord, forced_coop = geo(64, abi.AR_SIM_ORDINARY), geo(8, abi.AR_SIM_COOPERATIVE)
    print(f"[launch] {long_auto} {short_auto} {forced_ord} {forced_coop}", flush=True)
    assert short_auto["launch"] == "ordinary" and forced_ord["launch"] == "ordinary"
    assert forced_coop["launch"] == "cooperative"
    assert forced_coop["tiles_per_wave"] <= short_auto["tiles_per_wave"]
    if forced_coop["tiles_per_wave"] < short_auto["tiles_per_wave"]:
        assert long_auto["launch"] == "cooperative"
        assert long_auto["tiles_per_wave"] == forced_coop["tiles_per_wave"]
    else:
        assert long_auto["launch"] == "ordinary"
    # many tiles per wave either way (8 ranks, 4 MiB, sentinel): the same
    # geometry both ways, so the launch stays ordinary
    big = buffers.Workspace(8, 1 << 21, "sentinel", 8)
    xb = torch.zeros((1, 1 << 21), dtype=torch.int16, device="cuda")
    gb = lambda nops, flags=0: abi.ar_sim_geometry(
        big.sim_params(nops, xb, 0, xb, 0, flags=flags))
    ord_big, coop_big, auto_big = gb(64, abi.AR_SIM_ORDINARY), \
        gb(64, abi.AR_SIM_COOPERATIVE), gb(64)
    print(f"[launch 4 MiB] {ord_big} {coop_big} {auto_big}", flush=True)
    assert ord_big["tiles_per_wave"] > 1
    fewer = coop_big["tiles_per_wave"] < ord_big["tiles_per_wave"]
    assert auto_big["launch"] == ("cooperative" if fewer else "ordinary")


@pytest.mark.parametrize("blocks,threads", [(64, 512), (128, 1024), (2048, 64), (384, 512)])
def test_workgroup_xcd_placement(blocks, threads):
    """The simulators place the producer and the consumers of a tile on
    different XCDs by assuming that consecutive workgroups are dispatched to
    consecutive XCDs (round robin over the eight XCDs of one partition).  The
    round robin continues from earlier dispatches, so workgroup b runs on XCD
    (s + b) mod 8 for a start s of the launch; the XCC_ID register confirms
    it."""
    work = torch.zeros(256, dtype=torch.uint8, device="cuda")
    res = torch.full((blocks,), -2, dtype=torch.int32, device="cuda")
    abi.ar_probe_placement(blocks, threads, work, res)
    torch.cuda.synchronize()
    x = res.cpu().numpy()
    print(f"[placement] {blocks}x{threads}: xcds {sorted(set(x.tolist()))}", flush=True)
    assert np.all(x >= 0)
    assert np.array_equal(x, (x[0] + np.arange(blocks)) % 8)
