"""GPU parity of the standalone all-gather and the two-shot all-reduce
against the CPU oracle, through the C ABI.

Bit-exact comparisons throughout (integer encodings; one fixed-order
binary32 sum per element, done by the share owner):
* two-shot packing: every reduce-scatter slot holds the oracle's encoding
  of its share; the all-gather region holds the oracle's encoding of each
  reduced share after the reduce step;
* stream-ordered all-gather and two-shot over several ops on alternating
  parities, ragged counts, empty shares, special values;
* the persistent simulators (system mode) over many back-to-back ops, two
  launches in a row (the epoch carries over), with producer skew;
* the full-size workloads: 16 ranks [8,4096] two-shot with 0-20 us skew,
  8 ranks [1,4096] all-gather over 64 ops.
"""
import numpy as np
import pytest
import torch

import oracle
from collective_synchronization_amd import abi, buffers, inputs

pytestmark = pytest.mark.gpu

PROTOS = ("ll", "ll128", "sentinel")
TIMEOUT_NS = 2_000_000_000
SPECIALS = (0xFFFF, 0xFFC0, 0xFF81, 0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x8001)


def _x(seed, shape, specials=True):
    x = inputs.payload(seed, shape, "normal")
    if specials:
        x = inputs.inject(x, seed + 7, 1 / 64, values=SPECIALS)
    return x


SHAPES = [(8, 4096), (3, 1000), (4, 5), (16, 777), (1, 61), (2, 4099), (16, 100),
          (5, 60 * 17 + 1)]


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("nranks,count", SHAPES)
def test_twoshot_pack_and_stream_ordered(proto, nranks, count):
    print(f"[twoshot-stream] {proto} N={nranks} count={count}", flush=True)
    ws = buffers.Workspace(nranks, count, proto, nranks, collective="twoshot")
    stride = buffers.row_stride(count)
    outd = torch.zeros((nranks, stride), dtype=torch.int16, device="cuda")
    slot = abi.ar_desc_slot_bytes(ws.desc)
    fill = 0xFF if proto == "sentinel" else 0
    for op in range(4):                              # both parities, twice
        x = _x(31 * op + count + nranks, (nranks, count), specials=(op % 2 == 1))
        xd, _ = buffers.rows_to_device(x)
        ws.pack(xd, stride)
        torch.cuda.synchronize()
        seq, par = ws.epoch.seq, ws.epoch.parity
        if op == 0:                                  # reduce-scatter slots
            v = ws.slot_view()
            for c in range(nranks):
                lo, hi = oracle.shard_bounds(count, nranks, c)
                E = oracle.encoded_bytes(proto, hi - lo)
                for r in range(nranks):
                    want = oracle.encode(proto, x[r, lo:hi], seq)
                    assert np.array_equal(v[0, c, par, r, :E], want), (c, r)
                    assert np.all(v[0, c, par, r, E:] == fill)
            assert np.all(v[1] == fill)              # all-gather region untouched
        ws.reduce(outd, stride, timeout_ns=TIMEOUT_NS)
        torch.cuda.synchronize()
        assert ws.status() == 0, abi.status_string(ws.status())
        st, want = oracle.twoshot(x, proto, seq)
        assert st == oracle.READY
        got = buffers.rows_from_device(outd, count, (nranks,))
        for c in range(nranks):
            assert np.array_equal(got[c], want), (op, c)
        if op == 0 and proto != "sentinel":          # all-gather slots
            v = ws.slot_view()
            for k in range(nranks):
                lo, hi = oracle.shard_bounds(count, nranks, k)
                enc = oracle.encode(proto, want[lo:hi], seq)
                for c in range(nranks):
                    if c != k:
                        assert np.array_equal(v[1, c, par, k, :enc.size], enc), (c, k)
        ws.flip()
    if proto == "sentinel":                          # both regions re-armed
        assert np.all(ws.slot_view() == 0xFF)


@pytest.mark.parametrize("proto", PROTOS + ("barrier",))
@pytest.mark.parametrize("nranks,ncons,count", [(8, 8, 4096), (3, 1, 1000), (4, 4, 5),
                                                (16, 16, 777), (2, 2, 4099), (1, 1, 61)])
def test_allgather_stream_ordered(proto, nranks, ncons, count):
    print(f"[allgather-stream] {proto} N={nranks} C={ncons} count={count}", flush=True)
    ws = buffers.Workspace(nranks, count, proto, ncons, collective="allgather")
    stride = buffers.row_stride(count)
    ostride = ws.gather_stride()
    outd = torch.zeros((ncons, ostride), dtype=torch.int16, device="cuda")
    for op in range(4):
        x = _x(17 * op + count, (nranks, count), specials=(op % 2 == 0))
        xd, _ = buffers.rows_to_device(x)
        ws.pack(xd, stride)
        ws.gather(outd, ostride, timeout_ns=TIMEOUT_NS)
        torch.cuda.synchronize()
        assert ws.status() == 0, abi.status_string(ws.status())
        st, want = oracle.allgather(x, proto, ws.epoch.seq)
        assert st == oracle.READY
        got = outd.cpu().numpy().view(np.uint16).reshape(ncons, nranks, stride)[:, :, :count]
        for c in range(ncons):
            assert np.array_equal(got[c], want), (op, c)
        ws.flip()
    if proto == "sentinel":
        assert np.all(ws.slot_view() == 0xFF)


def test_twoshot_missing_producer_times_out():
    ws = buffers.Workspace(4, 4096, "ll", 4, collective="twoshot")
    stride = buffers.row_stride(4096)
    outd = torch.full((4, stride), 7, dtype=torch.int16, device="cuda")
    ws.reduce(outd, stride, timeout_ns=2_000_000)       # nothing was packed
    torch.cuda.synchronize()
    assert ws.status() == abi.AR_ETIMEOUT
    assert torch.all(outd == 7)


SIM_CASES = [(8, 4096, 8), (4, 8192, 6), (16, 32768, 3), (3, 1000, 5), (2, 60, 7),
             (1, 100, 3), (16, 100, 4), (8, 131072, 2), (16, 262144 + 13, 2)]


@pytest.mark.parametrize("kernel", ["auto", "narrow", "wide"])
@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("nranks,count,nops", SIM_CASES)
def test_sim_twoshot(proto, nranks, count, nops, kernel):
    print(f"[sim-twoshot] {kernel} {proto} N={nranks} count={count} ops={nops}", flush=True)
    flags = {"auto": 0, "narrow": abi.AR_SIM_NARROW, "wide": abi.AR_SIM_WIDE}[kernel]
    ws = buffers.Workspace(nranks, count, proto, nranks, collective="twoshot")
    x = _x(3 * count + nops + nranks, (nops, nranks, count))
    xd, stride = buffers.rows_to_device(x)
    outd = torch.zeros((nops * nranks, stride), dtype=torch.int16, device="cuda")
    seq0 = ws.epoch.seq
    want = oracle.twoshot_ops(x, proto, seq0)
    geo = abi.ar_sim_geometry(ws.sim_params(nops, xd, stride, outd, stride, flags=flags))
    if kernel != "auto":
        assert geo["kernel"] == kernel
    for run in range(2):                                 # the epoch carries over
        ws.sim(nops, xd, stride, outd, stride, timeout_ns=TIMEOUT_NS, flags=flags)
        torch.cuda.synchronize()
        assert ws.status() == 0, abi.status_string(ws.status())
        got = buffers.rows_from_device(outd, count, (nops, nranks))
        for i in range(nops):
            for c in range(nranks):
                assert np.array_equal(got[i, c], want[i]), (run, i, c)
        outd.zero_()
    if proto == "sentinel":
        assert np.all(ws.slot_view() == 0xFF)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("nranks,count,nops", SIM_CASES)
def test_sim_allgather(proto, nranks, count, nops):
    print(f"[sim-allgather] {proto} N={nranks} count={count} ops={nops}", flush=True)
    ws = buffers.Workspace(nranks, count, proto, nranks, collective="allgather")
    x = _x(5 * count + nops + nranks, (nops, nranks, count))
    xd, stride = buffers.rows_to_device(x)
    ostride = ws.gather_stride()
    outd = torch.zeros((nops * nranks, ostride), dtype=torch.int16, device="cuda")
    want = oracle.allgather_ops(x, proto, ws.epoch.seq)
    for run in range(2):
        ws.sim(nops, xd, stride, outd, ostride, timeout_ns=TIMEOUT_NS)
        torch.cuda.synchronize()
        assert ws.status() == 0, abi.status_string(ws.status())
        got = outd.cpu().numpy().view(np.uint16).reshape(nops, nranks, nranks, stride)
        for i in range(nops):
            for c in range(nranks):
                assert np.array_equal(got[i, c, :, :count], want[i]), (run, i, c)
        outd.zero_()
    if proto == "sentinel":
        assert np.all(ws.slot_view() == 0xFF)


@pytest.mark.parametrize("collective,nranks,count", [("twoshot", 8, 4096),
                                                     ("twoshot", 16, 32768),
                                                     ("allgather", 8, 4096)])
@pytest.mark.parametrize("proto", PROTOS)
def test_sim_producer_past_the_deadline_times_out(collective, proto, nranks, count):
    """One producer held past the poll deadline (a 20 ms delay before its
    op-1 sends against a 2 ms timeout): the persistent two-shot or all-gather
    launch ends with AR_ETIMEOUT instead of waiting."""
    nops = 4
    ws = buffers.Workspace(nranks, count, proto, nranks, collective=collective)
    x = _x(71 + count, (nops, nranks, count))
    xd, stride = buffers.rows_to_device(x)
    ostride = ws.gather_stride() if collective == "allgather" else stride
    outd = torch.zeros((nops * nranks, ostride), dtype=torch.int16, device="cuda")
    hz = abi.ar_wallclock_hz()
    d = np.zeros((nops, nranks), dtype=np.int32)
    d[1, nranks - 1] = int(0.02 * hz)
    ticks = torch.from_numpy(d).to("cuda")
    print(f"[coll-deadline] {collective} {proto} N={nranks} count={count}", flush=True)
    ws.sim(nops, xd, stride, outd, ostride, timeout_ns=2_000_000, delay_ticks=ticks)
    torch.cuda.synchronize()
    assert ws.status() == abi.AR_ETIMEOUT


LARGEST = [("twoshot", 8, 1 << 21), ("twoshot", 16, 1 << 20),
           ("allgather", 8, 1 << 19), ("allgather", 16, 1 << 19)]


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("collective,nranks,count", LARGEST)
def test_sim_largest_sweep_sizes(collective, proto, nranks, count):
    """The two-shot and the all-gather at the largest sizes the selector
    sweep measures (two-shot: 4 MiB per rank at 8 ranks, 2 MiB at 16;
    all-gather: 1 MiB), with the sweep's 32 ops per launch, so in the
    launch the library picks there: distinct payloads (special values
    included) on every op, every op of every consumer bit-exact."""
    nops = 32
    ws = buffers.Workspace(nranks, count, proto, nranks, collective=collective)
    x = np.stack([_x(11 * i + nranks + count, (nranks, count)) for i in range(nops)])
    xd, stride = buffers.rows_to_device(x)
    ostride = ws.gather_stride() if collective == "allgather" else stride
    outd = torch.zeros((nops * nranks, ostride), dtype=torch.int16, device="cuda")
    geo = abi.ar_sim_geometry(ws.sim_params(nops, xd, stride, outd, ostride))
    print(f"[largest] {collective} {proto} N={nranks} count={count} geo={geo}", flush=True)
    seq0 = ws.epoch.seq
    ws.sim(nops, xd, stride, outd, ostride, timeout_ns=TIMEOUT_NS)
    torch.cuda.synchronize()
    assert ws.status() == 0, abi.status_string(ws.status())
    del xd
    want = (oracle.twoshot_ops if collective == "twoshot" else oracle.allgather_ops)(
        x, proto, seq0)
    for i in range(nops):
        w = torch.from_numpy(want[i].view(np.int16)).to("cuda")
        rows = outd[i * nranks:(i + 1) * nranks]
        if collective == "twoshot":
            got, ref = rows[:, :count], w[None, :]
        else:
            got = rows.view(nranks, nranks, stride)[:, :, :count]
            ref = w[None, :, :]
        bad = got != ref
        assert not bool(bad.any()), (i, [int(v) for v in bad.nonzero()[0].tolist()])
    if proto == "sentinel":
        assert np.all(ws.slot_view() == 0xFF)


@pytest.mark.parametrize("collective,nranks,count", [("twoshot", 16, 65536 + 9),
                                                     ("allgather", 8, 16384 + 3)])
@pytest.mark.parametrize("proto", PROTOS)
def test_sim_cooperative_launches(collective, nranks, count, proto):
    """Forced cooperative launches (whose grid may fill the occupancy) and the
    library's own choice over 32 ops, bit-exact against the oracle."""
    nops = 32
    ws = buffers.Workspace(nranks, count, proto, nranks, collective=collective)
    x = _x(11 * count + nranks, (nops, nranks, count), specials=True)
    xd, stride = buffers.rows_to_device(x)
    ostride = ws.gather_stride() if collective == "allgather" else stride
    outd = torch.zeros((nops * nranks, ostride), dtype=torch.int16, device="cuda")
    for flags in (abi.AR_SIM_COOPERATIVE, 0):
        seq0 = ws.epoch.seq
        geo = abi.ar_sim_geometry(ws.sim_params(nops, xd, stride, outd, ostride, flags=flags))
        print(f"[coll-coop] {collective} {proto} N={nranks} count={count} flags={flags} "
              f"geo={geo}", flush=True)
        if flags:
            assert geo["launch"] == "cooperative"
        ws.sim(nops, xd, stride, outd, ostride, timeout_ns=TIMEOUT_NS, flags=flags)
        torch.cuda.synchronize()
        assert ws.status() == 0, abi.status_string(ws.status())
        if collective == "allgather":
            want = oracle.allgather_ops(x, proto, seq0)
            got = outd.cpu().numpy().view(np.uint16).reshape(nops, nranks, nranks, stride)
            for i in range(nops):
                for c in range(nranks):
                    assert np.array_equal(got[i, c, :, :count], want[i]), (flags, i, c)
        else:
            want = oracle.twoshot_ops(x, proto, seq0)
            got = buffers.rows_from_device(outd, count, (nops, nranks))
            for i in range(nops):
                for c in range(nranks):
                    assert np.array_equal(got[i, c], want[i]), (flags, i, c)
        outd.zero_()


@pytest.mark.parametrize("proto", PROTOS)
def test_twoshot_n16_8x4096_skewed(proto):
    """16 ranks, bf16 [8,4096], 64 ops, seeded 0-20 us producer delays: every
    rank bit-identical to the oracle (two-shot and one-shot agree)."""
    n, count, nops, seed = 16, 8 * 4096, 64, 1005
    x = inputs.payload(seed, (nops, n, count), "normal")
    hz = abi.ar_wallclock_hz()
    d_us = inputs.delays_us(seed + 1, nops, n, 20.0)
    ticks = torch.from_numpy(np.round(d_us * hz * 1e-6).astype(np.int32)).to("cuda")
    ws = buffers.Workspace(n, count, proto, n, collective="twoshot")
    xd, stride = buffers.rows_to_device(x)
    outd = torch.zeros((nops * n, stride), dtype=torch.int16, device="cuda")
    trace = torch.zeros(nops * 2 * n + 1, dtype=torch.int64, device="cuda")
    trace[-1] = -1
    seq0 = ws.epoch.seq
    ws.sim(nops, xd, stride, outd, stride, timeout_ns=TIMEOUT_NS, delay_ticks=ticks,
           trace=trace)
    torch.cuda.synchronize()
    assert ws.status() == 0, abi.status_string(ws.status())
    got = buffers.rows_from_device(outd, count, (nops, n))
    want = oracle.allreduce_ops(x, proto, seq0)
    for i in range(nops):
        for c in range(n):
            assert np.array_equal(got[i, c], want[i]), (i, c)
    t = trace.cpu().numpy()[:-1].reshape(nops, 2, n).astype(np.float64)
    assert np.all(t[:, 0, :] > 0) and np.all(t[:, 1, :] > 0)
    post = (t[:, 1, :].max(axis=1) - t[:, 0, :].max(axis=1)) / hz * 1e6
    print(f"[twoshot n16 skew {proto}] median post-arrival latency {np.median(post):.3f} us",
          flush=True)


@pytest.mark.parametrize("proto", PROTOS)
def test_allgather_n8_1x4096_64ops(proto):
    n, count, nops, seed = 8, 4096, 64, 1002
    x = inputs.payload(seed, (nops, n, count), "normal")
    x = inputs.inject(x, seed + 1, 1 / 1024)
    ws = buffers.Workspace(n, count, proto, n, collective="allgather")
    xd, stride = buffers.rows_to_device(x)
    ostride = ws.gather_stride()
    outd = torch.zeros((nops * n, ostride), dtype=torch.int16, device="cuda")
    want = oracle.allgather_ops(x, proto, ws.epoch.seq)
    ws.sim(nops, xd, stride, outd, ostride, timeout_ns=TIMEOUT_NS)
    torch.cuda.synchronize()
    assert ws.status() == 0, abi.status_string(ws.status())
    got = outd.cpu().numpy().view(np.uint16).reshape(nops, n, n, stride)[..., :count]
    for i in range(nops):
        for c in range(n):
            assert np.array_equal(got[i, c], want[i]), (i, c)
    if proto == "sentinel":
        assert not np.any(got == 0xFFFF)


@pytest.mark.parametrize("collective,nranks,count", [("twoshot", 16, 32768),
                                                     ("allgather", 8, 4096)])
def test_sim_pairwise_tiny_deadline_then_reset(collective, nranks, count):
    """LL with one tile per workgroup runs the pairwise loops (the two-shot
    with one barrier per op, the all-gather with none).  A poll deadline of
    one wall-clock tick, set from the host, makes every wait give up at once
    or find its data: the launch ends with OK or AR_ETIMEOUT, never a hang.
    After ar_state_reset the same buffers run bit-exact again."""
    nops = 16
    ws = buffers.Workspace(nranks, count, "ll", nranks, collective=collective)
    x = _x(6900, (nops, nranks, count), specials=False)
    xd, stride = buffers.rows_to_device(x)
    ostride = ws.gather_stride() if collective == "allgather" else stride
    outd = torch.zeros((nops * nranks, ostride), dtype=torch.int16, device="cuda")
    geo = abi.ar_sim_geometry(ws.sim_params(nops, xd, stride, outd, ostride))
    print(f"[pairwise-deadline] {collective} N={nranks} count={count} geo={geo}", flush=True)
    assert geo["tiles_per_wave"] == 1 and geo["kernel"] == "wide"
    ws.sim(nops, xd, stride, outd, ostride, timeout_ns=1)
    torch.cuda.synchronize()
    assert ws.status() in (0, abi.AR_ETIMEOUT), abi.status_string(ws.status())
    print(f"  one-tick deadline: {abi.status_string(ws.status())}", flush=True)
    ws.reset_state()
    seq0 = ws.epoch.seq
    ws.sim(nops, xd, stride, outd, ostride, timeout_ns=TIMEOUT_NS)
    torch.cuda.synchronize()
    assert ws.status() == 0, abi.status_string(ws.status())
    if collective == "twoshot":
        want = oracle.twoshot_ops(x, "ll", seq0)
        got = buffers.rows_from_device(outd, count, (nops, nranks))
        for i in range(nops):
            for c in range(nranks):
                assert np.array_equal(got[i, c], want[i]), (i, c)
    else:
        want = oracle.allgather_ops(x, "ll", seq0)
        rs = buffers.row_stride(count)
        got = outd.cpu().numpy().view(np.uint16).reshape(nops, nranks, nranks, rs)[..., :count]
        for i in range(nops):
            for c in range(nranks):
                assert np.array_equal(got[i, c], want[i]), (i, c)
