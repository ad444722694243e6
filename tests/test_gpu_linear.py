"""GPU parity of the chained all-reduce whose producer is a row-parallel
linear layer shard (ar_sim_linear_run), through the C ABI, against the
oracle's linear_chain_ops, bit for bit on every op and every rank's output.

Each rank reads only its slice of its own input row: the rest of every row
holds the sentinel pattern and other negative NaNs, which would poison the
result if read.  Cases: one to sixteen ranks (at sixteen, LL and LL128 with
exchange workgroups that take two tiles each), slices of 256 to 2048 inputs
(the GEMV's four lane widths), several layers taken in turn, two launches
in a row (the epoch, the receive slots and the work buffer carry over), the
decode workload's full size (8 ranks, hidden 4096, 64 ops), inputs with
signed zeros and subnormals, and an infinity that turns the chain into NaN
(canonical 0x7FC0 through every protocol)."""
import numpy as np
import pytest
import torch

import oracle
from collective_synchronization_amd import abi, buffers, inputs

pytestmark = pytest.mark.gpu

PROTOS = ("ll", "ll128", "sentinel")
TIMEOUT_NS = 2_000_000_000


def _rows(seed, nranks, count, specials=None):
    """Per-rank input rows: N(0,1) in rank r's slice, negative NaNs elsewhere."""
    kr = count // nranks
    x = np.full((nranks, count), 0xFFFF, dtype=np.uint16)
    x[:, 1::3] = 0xFFC0
    body = inputs.payload(seed, (nranks, count), "normal")
    if specials is not None:
        body = inputs.inject(body, seed + 1, 1 / 32, values=specials)
    for r in range(nranks):
        x[r, r * kr:(r + 1) * kr] = body[r, r * kr:(r + 1) * kr]
    return x


def _run(proto, nranks, count, nops, layers, seed, runs=2, specials=None, flags=0):
    ws = buffers.Workspace(nranks, count, proto, nranks)
    x0 = _rows(seed, nranks, count, specials)
    w = inputs.weights(seed + 7, layers, nranks, count)
    wd = torch.from_numpy(w.view(np.int16)).to("cuda")
    xd, stride = buffers.rows_to_device(x0)
    outd = torch.zeros((nops * nranks, stride), dtype=torch.int16, device="cuda")
    p = ws.sim_params(nops, xd, stride, outd, stride, flags=flags)
    geo = abi.ar_sim_linear_geometry(p, wd, layers, ws.linear_work())
    print(f"[linear] {proto} N={nranks} count={count} ops={nops} layers={layers} geo={geo}",
          flush=True)
    want = oracle.linear_chain_ops(x0, w, nops, proto, ws.epoch.seq)
    for run in range(runs):
        ws.sim_linear(nops, xd, stride, outd, stride, wd, layers, timeout_ns=TIMEOUT_NS,
                      flags=flags)
        torch.cuda.synchronize()
        assert ws.status() == 0, abi.status_string(ws.status())
        got = buffers.rows_from_device(outd, count, (nops, nranks))
        for i in range(nops):
            for c in range(nranks):
                assert np.array_equal(got[i, c], want[i]), (run, i, c)
        outd.zero_()
    if proto == "sentinel":
        assert np.all(ws.slot_view() == 0xFF)
    return want


CASES = [(1, 256, 4, 2), (2, 512, 5, 2), (3, 768, 5, 3), (4, 1024, 6, 2), (5, 1280, 4, 2),
         (8, 2048, 6, 3), (16, 4096, 5, 2), (4, 4096, 5, 2), (8, 4096, 6, 2), (4, 8192, 3, 2)]


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("nranks,count,nops,layers", CASES)
def test_sim_linear_parity(proto, nranks, count, nops, layers):
    # (16 ranks, LL / LL128: an exchange workgroup takes two tiles in turn)
    _run(proto, nranks, count, nops, layers, seed=5100 + count + nranks)


@pytest.mark.parametrize("proto", PROTOS)
def test_sim_linear_decode_size_64_ops(proto):
    """8 ranks, hidden 4096 (slices of 512), 64 chained ops over 4 layers."""
    out = _run(proto, 8, 4096, 64, 4, seed=5200, runs=1)
    # the chain keeps its scale: the last op is neither flushed nor blown up
    f = (out[-1].astype(np.uint32) << 16).view(np.float32)
    assert np.isfinite(f).all() and 0.05 < float(np.abs(f).mean()) < 20.0


@pytest.mark.parametrize("proto", PROTOS)
def test_sim_linear_signed_zeros_and_subnormals(proto):
    _run(proto, 4, 1024, 4, 2, seed=5300, specials=(0x8000, 0x0000, 0x0001, 0x8001, 0x007F))


@pytest.mark.parametrize("proto", PROTOS)
def test_sim_linear_infinity_becomes_canonical_nan(proto):
    want = _run(proto, 2, 512, 3, 1, seed=5400, runs=1, specials=(0x7F80,))
    assert (want[-1] == 0x7FC0).all()


def test_sim_linear_cooperative_launch():
    _run("ll", 8, 4096, 8, 2, seed=5500, runs=1, flags=abi.AR_SIM_COOPERATIVE)


def test_sim_linear_one_op_launches_in_a_row():
    """nops = 1, five launches: each launch's op 0 reads the input rows; the
    epoch, the slots and the work buffer carry over."""
    nranks, count = 8, 4096
    ws = buffers.Workspace(nranks, count, "sentinel", nranks)
    w = inputs.weights(5601, 1, nranks, count)
    wd = torch.from_numpy(w.view(np.int16)).to("cuda")
    for k in range(5):
        x0 = _rows(5600 + k, nranks, count)
        xd, stride = buffers.rows_to_device(x0)
        outd = torch.zeros((nranks, stride), dtype=torch.int16, device="cuda")
        want = oracle.linear_chain_ops(x0, w, 1, "sentinel", ws.epoch.seq)
        ws.sim_linear(1, xd, stride, outd, stride, wd, 1, timeout_ns=TIMEOUT_NS)
        torch.cuda.synchronize()
        assert ws.status() == 0, abi.status_string(ws.status())
        got = buffers.rows_from_device(outd, count, (1, nranks))
        for c in range(nranks):
            assert np.array_equal(got[0, c], want[0]), (k, c)


@pytest.mark.parametrize("proto", PROTOS)
def test_sim_linear_tiny_deadline_ends_cleanly(proto):
    """A poll deadline of one wall-clock tick, set from the host: every wait
    gives up at once or finds its data, the launch ends, and the status is
    OK or AR_ETIMEOUT -- never a hang."""
    nranks, count, nops = 8, 4096, 16
    ws = buffers.Workspace(nranks, count, proto, nranks)
    w = torch.zeros((2, nranks, count, count // nranks), dtype=torch.int16, device="cuda")
    xd, stride = buffers.rows_to_device(_rows(5700, nranks, count))
    outd = torch.zeros((nops * nranks, stride), dtype=torch.int16, device="cuda")
    ws.sim_linear(nops, xd, stride, outd, stride, w, 2, timeout_ns=1)
    torch.cuda.synchronize()
    assert ws.status() in (0, abi.AR_ETIMEOUT), abi.status_string(ws.status())


@pytest.mark.parametrize("proto", PROTOS)
def test_sim_linear_impossible_slice_flag_is_corrupt(proto):
    """A slice word holding an epoch that can never be there (planted from
    the host in the work buffer before the launch) is reported as
    AR_ECORRUPT by the workers that read it, and the launch ends."""
    nranks, count, nops = 4, 1024, 3
    ws = buffers.Workspace(nranks, count, proto, nranks)
    work = ws.linear_work()
    kr = count // nranks
    # slice words [nranks][2][kr/2] of 8 bytes after the payload words
    act0 = 8 * nranks * count
    words = work[act0:act0 + 8 * count].view(torch.int32).view(nranks, 2, kr // 2, 2)
    words[:, :, :, 1] = 0x5A5A5A5A          # neither this op's, two ops before, nor 0
    w = torch.zeros((1, nranks, count, kr), dtype=torch.int16, device="cuda")
    xd, stride = buffers.rows_to_device(_rows(5800, nranks, count))
    outd = torch.zeros((nops * nranks, stride), dtype=torch.int16, device="cuda")
    ws.sim_linear(nops, xd, stride, outd, stride, w, 1, timeout_ns=TIMEOUT_NS)
    torch.cuda.synchronize()
    assert ws.status() == abi.AR_ECORRUPT, abi.status_string(ws.status())
