"""GPU: sequences of library calls captured in a HIP graph and replayed.

A replay repeats the epochs its calls were captured with; ar_state_reset at
the head of the sequence returns the control block, the receive buffers and
the linear work buffer to their initial state (fill kernels, no memset
nodes), so every replay starts afresh.  Each test captures once, then
replays several times with new inputs copied in between, runs other eager
work and synchronizes between replays, and checks every op of every
consumer of every replay against the oracle, bit for bit.  Covered: single-
and multi-op persistent launches for all four protocols, stream-ordered
pack + reduce, the two-shot all-reduce and the all-gather, a cooperative
launch, the linear-layer chain, the scaled chain, and the allocation-free
entry point (which clears its own buffers).  An eager op on the same buffers
after the replays continues from the epoch that followed the capture.
"""
import numpy as np
import pytest
import torch

import oracle
from collective_synchronization_amd import abi, buffers, inputs

pytestmark = pytest.mark.gpu

TIMEOUT_NS = 2_000_000_000
REPLAYS = 3
N, COUNT = 8, 4096


def _eager_work(k):
    """Unrelated eager work between replays: a small all-reduce of its own,
    checked, and a synchronization."""
    ws = buffers.Workspace(4, 1000, "ll", 4)
    x = inputs.payload(880 + k, (2, 4, 1000), "normal")
    xd, s = buffers.rows_to_device(x)
    out = torch.zeros((8, s), dtype=torch.int16, device="cuda")
    ws.sim(2, xd, s, out, s, timeout_ns=TIMEOUT_NS)
    torch.cuda.synchronize()
    assert ws.status() == 0, abi.status_string(ws.status())
    got = buffers.rows_from_device(out, 1000, (2, 4))
    want = oracle.allreduce_ops(x, "ll", 1)
    for i in range(2):
        for c in range(4):
            assert np.array_equal(got[i, c], want[i])


def _check_ops(outd, count, nops, ncons, want, where):
    got = buffers.rows_from_device(outd, count, (nops, ncons))
    for i in range(nops):
        for c in range(ncons):
            assert np.array_equal(got[i, c], want[i]), (where, i, c)


def _replays(g, ws, load, expect, seed):
    """Replay g REPLAYS times: load(new inputs) eagerly, replay, check."""
    for r in range(REPLAYS):
        print(f"[graph] replay {r}", flush=True)
        x = load(seed + r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if ws is not None:
            assert ws.status() == 0, abi.status_string(ws.status())
        expect(x, r)
        _eager_work(r)


@pytest.mark.parametrize("proto", ["ll", "ll128", "sentinel", "barrier"])
def test_graph_persistent_launches(proto):
    """Eight one-op launches and one four-op launch in one graph; then an
    eager launch that continues from the capture's last epoch."""
    print(f"[graph] persistent {proto}", flush=True)
    ws = buffers.Workspace(N, COUNT, proto, N)
    nops = 12
    stride = buffers.row_stride(COUNT)
    xd = torch.zeros((nops * N, stride), dtype=torch.int16, device="cuda")
    outd = torch.zeros((nops * N, stride), dtype=torch.int16, device="cuda")
    seq0 = ws.epoch.seq
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ws.reset_state()
        for j in range(8):
            ws.sim(1, xd[j * N:], stride, outd[j * N:], stride, timeout_ns=TIMEOUT_NS)
        ws.sim(4, xd[8 * N:], stride, outd[8 * N:], stride, timeout_ns=TIMEOUT_NS)

    def load(seed):
        x = inputs.payload(seed, (nops, N, COUNT), "normal")
        xd.copy_(buffers.rows_to_device(x)[0])
        outd.fill_(-1)
        return x

    _replays(g, ws, load,
             lambda x, r: _check_ops(outd, COUNT, nops, N,
                                     oracle.allreduce_ops(x, proto, seq0), r), 6100)
    # the buffers hold what the captured ops left: an eager op continues
    x = inputs.payload(6199, (2, N, COUNT), "normal")
    xe, _ = buffers.rows_to_device(x)
    oe = torch.zeros((2 * N, stride), dtype=torch.int16, device="cuda")
    seq = ws.epoch.seq
    ws.sim(2, xe, stride, oe, stride, timeout_ns=TIMEOUT_NS)
    torch.cuda.synchronize()
    assert ws.status() == 0, abi.status_string(ws.status())
    _check_ops(oe, COUNT, 2, N, oracle.allreduce_ops(x, proto, seq), "eager")


@pytest.mark.parametrize("proto", ["ll", "ll128", "sentinel", "barrier"])
def test_graph_stream_ordered(proto):
    """Four stream-ordered ops (pack, reduce, flip) per replay."""
    print(f"[graph] stream-ordered {proto}", flush=True)
    ws = buffers.Workspace(N, COUNT, proto, N)
    nops = 4
    stride = buffers.row_stride(COUNT)
    xd = torch.zeros((nops * N, stride), dtype=torch.int16, device="cuda")
    outd = torch.zeros((nops * N, stride), dtype=torch.int16, device="cuda")
    seq0 = ws.epoch.seq
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ws.reset_state()
        for i in range(nops):
            ws.pack(xd[i * N:], stride)
            ws.reduce(outd[i * N:], stride, timeout_ns=TIMEOUT_NS)
            ws.flip()

    def load(seed):
        x = inputs.payload(seed, (nops, N, COUNT), "normal")
        xd.copy_(buffers.rows_to_device(x)[0])
        outd.fill_(-1)
        return x

    _replays(g, ws, load,
             lambda x, r: _check_ops(outd, COUNT, nops, N,
                                     oracle.allreduce_ops(x, proto, seq0), r), 6200)


def test_graph_twoshot_and_allgather():
    """Three two-shot all-reduces (LL, whose consumers wait on each other
    inside one launch) and three all-gathers (LL128), one graph."""
    print("[graph] two-shot + all-gather", flush=True)
    nops, count = 3, 1000
    stride = buffers.row_stride(count)
    ts = buffers.Workspace(N, count, "ll", N, collective="twoshot")
    ag = buffers.Workspace(N, count, "ll128", N, collective="allgather")
    xd = torch.zeros((nops * N, stride), dtype=torch.int16, device="cuda")
    out_ts = torch.zeros((nops * N, stride), dtype=torch.int16, device="cuda")
    gs = ag.gather_stride()
    out_ag = torch.zeros((nops * N, gs), dtype=torch.int16, device="cuda")
    s_ts, s_ag = ts.epoch.seq, ag.epoch.seq
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ts.reset_state()
        ag.reset_state()
        for i in range(nops):
            ts.pack(xd[i * N:], stride)
            ts.reduce(out_ts[i * N:], stride, timeout_ns=TIMEOUT_NS)
            ts.flip()
            ag.pack(xd[i * N:], stride)
            ag.gather(out_ag[i * N:], gs, timeout_ns=TIMEOUT_NS)
            ag.flip()

    def load(seed):
        x = inputs.payload(seed, (nops, N, count), "normal")
        xd.copy_(buffers.rows_to_device(x)[0])
        out_ts.fill_(-1)
        out_ag.fill_(-1)
        return x

    def expect(x, r):
        assert ag.status() == 0, abi.status_string(ag.status())
        _check_ops(out_ts, count, nops, N, oracle.twoshot_ops(x, "ll", s_ts), r)
        want = oracle.allgather_ops(x, "ll128", s_ag)
        rs = buffers.row_stride(count)
        got = out_ag.cpu().numpy().view(np.uint16).reshape(nops, N, N, rs)[..., :count]
        for i in range(nops):
            for c in range(N):
                assert np.array_equal(got[i, c], want[i]), (r, i, c)

    _replays(g, ts, load, expect, 6300)


def test_graph_cooperative_launch():
    """16 ranks [1,4096] LL128 over 64 ops: the library launches this grid
    cooperatively, and the graph holds a cooperative kernel node."""
    print("[graph] cooperative", flush=True)
    n, nops = 16, 64
    ws = buffers.Workspace(n, COUNT, "ll128", n)
    stride = buffers.row_stride(COUNT)
    xd = torch.zeros((nops * n, stride), dtype=torch.int16, device="cuda")
    outd = torch.zeros((nops * n, stride), dtype=torch.int16, device="cuda")
    geo = abi.ar_sim_geometry(ws.sim_params(nops, xd, stride, outd, stride))
    assert geo["launch"] == "cooperative", geo
    seq0 = ws.epoch.seq
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ws.reset_state()
        ws.sim(nops, xd, stride, outd, stride, timeout_ns=TIMEOUT_NS)

    def load(seed):
        x = inputs.payload(seed, (nops, n, COUNT), "normal")
        xd.copy_(buffers.rows_to_device(x)[0])
        outd.fill_(-1)
        return x

    _replays(g, ws, load,
             lambda x, r: _check_ops(outd, COUNT, nops, n,
                                     oracle.allreduce_ops(x, "ll128", seq0), r), 6400)


def test_graph_linear_chain():
    """Eight chained ops whose producer is a row-parallel linear shard
    (8 ranks, hidden 4096, two layers); the work buffer is reset too."""
    print("[graph] linear chain", flush=True)
    nops, layers = 8, 2
    ws = buffers.Workspace(N, COUNT, "ll", N)
    stride = buffers.row_stride(COUNT)
    w = inputs.weights(6507, layers, N, COUNT)
    wd = torch.from_numpy(w.view(np.int16)).to("cuda")
    xd = torch.zeros((N, stride), dtype=torch.int16, device="cuda")
    outd = torch.zeros((nops * N, stride), dtype=torch.int16, device="cuda")
    ws.linear_work()                      # allocated before the capture
    seq0 = ws.epoch.seq
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ws.reset_state()
        ws.sim_linear(nops, xd, stride, outd, stride, wd, layers, timeout_ns=TIMEOUT_NS)
    kr = COUNT // N

    def load(seed):
        x = np.full((N, COUNT), 0xFFFF, dtype=np.uint16)   # only the slices are read
        body = inputs.payload(seed, (N, COUNT), "normal")
        for r in range(N):
            x[r, r * kr:(r + 1) * kr] = body[r, r * kr:(r + 1) * kr]
        xd.copy_(buffers.rows_to_device(x)[0])
        outd.fill_(-1)
        return x

    _replays(g, ws, load,
             lambda x, r: _check_ops(outd, COUNT, nops, N,
                                     oracle.linear_chain_ops(x, w, nops, "ll", seq0), r),
             6500)


def test_graph_scaled_chain():
    """Sixteen chained ops with the per-rank scale as the producer (sentinel)."""
    print("[graph] scaled chain", flush=True)
    nops = 16
    ws = buffers.Workspace(N, COUNT, "sentinel", N)
    stride = buffers.row_stride(COUNT)
    rng = np.random.default_rng(6600)
    scales = rng.uniform(0.75, 1.25, (nops, N)).astype(np.float32)
    sd = torch.from_numpy(scales.reshape(-1)).to("cuda")
    xd = torch.zeros((N, stride), dtype=torch.int16, device="cuda")
    outd = torch.zeros((nops * N, stride), dtype=torch.int16, device="cuda")
    seq0 = ws.epoch.seq
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ws.reset_state()
        ws.sim_chain(nops, xd, stride, outd, stride, sd, timeout_ns=TIMEOUT_NS)

    def load(seed):
        x = inputs.payload(seed, (N, COUNT), "normal")
        xd.copy_(buffers.rows_to_device(x)[0])
        outd.fill_(-1)
        return x

    _replays(g, ws, load,
             lambda x, r: _check_ops(outd, COUNT, nops, N,
                                     oracle.chain_ops(x, scales, "sentinel", seq0), r),
             6600)


def test_graph_allocation_free_entry():
    """ar_sim_run_static clears its own buffers on every call, so two calls
    of different sizes replay without ar_state_reset."""
    print("[graph] allocation-free entry", flush=True)
    calls = [(8, 4096, "ll", 6), (4, 1000, "sentinel", 3)]
    bufs = []
    for n, count, proto, nops in calls:
        s = buffers.row_stride(count)
        bufs.append((torch.zeros((nops * n, s), dtype=torch.int16, device="cuda"),
                     torch.zeros((nops * n, s), dtype=torch.int16, device="cuda"),
                     torch.full((1,), -99, dtype=torch.int32, device="cuda"), s))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (n, count, proto, nops), (xd, outd, st, s) in zip(calls, bufs):
            desc = abi.make_desc(n, count, proto, n)
            p = abi.sim_params(desc, nops, xd, s, outd, s, None, None, abi.ar_epoch_init(),
                               timeout_ns=TIMEOUT_NS)
            abi.ar_sim_run_static(p, st)

    def load(seed):
        xs = []
        for k, ((n, count, proto, nops), (xd, outd, st, s)) in enumerate(zip(calls, bufs)):
            x = inputs.payload(seed + 10 * k, (nops, n, count), "normal")
            xd.copy_(buffers.rows_to_device(x)[0])
            outd.fill_(-1)
            st.fill_(-99)
            xs.append(x)
        return xs

    def expect(xs, r):
        for (n, count, proto, nops), (xd, outd, st, s), x in zip(calls, bufs, xs):
            assert int(st.item()) == 0, abi.status_string(int(st.item()))
            _check_ops(outd, count, nops, n, oracle.allreduce_ops(x, proto, 1), (r, proto))

    _replays(g, None, load, expect, 6700)
