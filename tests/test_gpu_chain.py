"""GPU parity of the chained all-reduce simulator (ar_sim_chain_run): op 0
all-reduces the inputs, op i+1's payload of rank r is op i's result scaled
by scales[i+1, r], all inside one persistent launch.  Through the C ABI,
against the oracle's chain_ops, bit for bit on every op and every consumer:
ragged counts, one rank, 16 ranks (a cooperative grid where the ordinary one
is too small), special values in op 0's payloads, a zero factor and an
infinite one late in the chain (so NaN and infinities travel through the
encodings), two launches in a row (the epoch carries over).  Then the
argument and capacity errors the header documents."""
import numpy as np
import pytest
import torch

import oracle
from collective_synchronization_amd import abi, buffers, inputs

pytestmark = pytest.mark.gpu

PROTOS = ("ll", "ll128", "sentinel")
TIMEOUT_NS = 2_000_000_000
SPECIALS = (0xFFFF, 0xFFC0, 0xFF81, 0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x8001)


def _scales(seed, K, n):
    """Factors of size about 1/n with random signs (the chain stays in
    range); row 0 is never read (NaN); a zero factor and an infinite one in
    the last two ops."""
    rng = np.random.default_rng(seed)
    s = rng.uniform(0.5, 1.5, size=(K, n)) / n * rng.choice([-1.0, 1.0], size=(K, n))
    s = s.astype(np.float32)
    s[0] = np.nan
    if K >= 3:
        s[K - 2, 0] = 0.0
        s[K - 1, n - 1] = np.inf
    return s


CASES = [(8, 4096, 64), (4, 4096, 16), (16, 4096, 8), (3, 1000, 5), (2, 60, 7),
         (1, 100, 3), (4, 32768, 6), (5, 61, 4)]


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("nranks,count,nops", CASES)
def test_sim_chain_parity(proto, nranks, count, nops):
    ws = buffers.Workspace(nranks, count, proto, nranks)
    x0 = inputs.inject(inputs.payload(41 + count + nranks, (nranks, count), "normal"),
                       48 + count, 1 / 64, values=SPECIALS)
    xd, stride = buffers.rows_to_device(x0)
    s = _scales(43 + nops, nops, nranks)
    sd = torch.from_numpy(s).to("cuda")
    outd = torch.zeros((nops * nranks, stride), dtype=torch.int16, device="cuda")
    geo = abi.ar_sim_chain_geometry(ws.sim_params(nops, xd, stride, outd, stride))
    print(f"[chain] {proto} N={nranks} count={count} ops={nops} geo={geo}", flush=True)
    want = oracle.chain_ops(x0, s, proto, ws.epoch.seq)
    for run in range(2):                                 # the epoch carries over
        ws.sim_chain(nops, xd, stride, outd, stride, sd, timeout_ns=TIMEOUT_NS)
        torch.cuda.synchronize()
        assert ws.status() == 0, abi.status_string(ws.status())
        got = buffers.rows_from_device(outd, count, (nops, nranks))
        for i in range(nops):
            for c in range(nranks):
                assert np.array_equal(got[i, c], want[i]), (run, i, c)
        outd.zero_()
    if proto == "sentinel":
        assert np.all(ws.slot_view() == 0xFF)


def _chain_error(ws, nops=4, **kw):
    count = ws.desc.count
    n = ws.desc.nranks
    xd, stride = buffers.rows_to_device(np.zeros((n, count), np.uint16))
    outd = torch.zeros((nops * ws.desc.nconsumers, stride), dtype=torch.int16, device="cuda")
    sd = kw.pop("scales", torch.ones((nops, n), dtype=torch.float32, device="cuda"))
    p = ws.sim_params(nops, xd, stride, outd, stride, timeout_ns=TIMEOUT_NS, **kw)
    with pytest.raises(abi.ArError) as e:
        abi.ar_sim_chain_run(p, sd)
    return e.value.code


def test_sim_chain_argument_errors():
    ws = buffers.Workspace(8, 4096, "sentinel", 8)
    assert _chain_error(ws, scales=None) == abi.AR_EINVAL
    assert _chain_error(ws, flags=abi.AR_SIM_NARROW) == abi.AR_EINVAL
    assert _chain_error(ws, waves_per_rank=8) == abi.AR_EINVAL
    delays = torch.zeros(4 * 8, dtype=torch.int32, device="cuda")
    assert _chain_error(ws, delay_ticks=delays) == abi.AR_EINVAL
    assert _chain_error(buffers.Workspace(8, 4096, "barrier", 8)) == abi.AR_EINVAL
    assert _chain_error(buffers.Workspace(8, 4096, "sentinel", 1)) == abi.AR_EINVAL
    assert _chain_error(buffers.Workspace(8, 4096, "sentinel", 8,
                                          collective="twoshot")) == abi.AR_EINVAL
    # every tile needs its own resident workgroup
    big = buffers.Workspace(16, 65536, "ll", 16)
    assert _chain_error(big) == abi.AR_ECAPACITY
    assert ws.status() == 0


@pytest.mark.parametrize("proto", PROTOS)
def test_sim_chain_tiny_deadline_then_reset(proto):
    """A poll deadline of one wall-clock tick, set from the host (LL and
    LL128 at 8 ranks run the one-barrier form, the sentinel the two-barrier
    one): every wait gives up at once or finds its data, and the launch ends
    with OK or AR_ETIMEOUT, never a hang.  After ar_state_reset the same
    buffers run bit-exact again."""
    nranks, count, nops = 8, 4096, 16
    ws = buffers.Workspace(nranks, count, proto, nranks)
    x0 = inputs.payload(6950, (nranks, count), "normal")
    xd, stride = buffers.rows_to_device(x0)
    s = _scales(6951, nops, nranks)
    sd = torch.from_numpy(s).to("cuda")
    outd = torch.zeros((nops * nranks, stride), dtype=torch.int16, device="cuda")
    print(f"[chain-deadline] {proto}", flush=True)
    ws.sim_chain(nops, xd, stride, outd, stride, sd, timeout_ns=1)
    torch.cuda.synchronize()
    assert ws.status() in (0, abi.AR_ETIMEOUT), abi.status_string(ws.status())
    print(f"  one-tick deadline: {abi.status_string(ws.status())}", flush=True)
    ws.reset_state()
    seq0 = ws.epoch.seq
    ws.sim_chain(nops, xd, stride, outd, stride, sd, timeout_ns=TIMEOUT_NS)
    torch.cuda.synchronize()
    assert ws.status() == 0, abi.status_string(ws.status())
    want = oracle.chain_ops(x0, s, proto, seq0)
    got = buffers.rows_from_device(outd, count, (nops, nranks))
    for i in range(nops):
        for c in range(nranks):
            assert np.array_equal(got[i, c], want[i]), (i, c)
