"""The allocation-free entry point ar_sim_run_static, through the C ABI.

It runs the same persistent simulator as ar_sim_run on receive buffers and a
control block of the library's own device array.  Each call is checked bit
for bit against ar_sim_run on the same inputs (caller-owned buffers) and
against the oracle, over several calls in a row whose sizes shrink and whose
protocols change, so that a call that does not clear what the previous one
left in the shared array would show.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from collective_synchronization_amd import abi, buffers, inputs

pytestmark = pytest.mark.gpu

TIMEOUT_NS = 2_000_000_000

# (nranks, nconsumers, count, proto, nops, seed): the first is the largest
CALLS = [
    (8, 8, 4096, "sentinel", 64, 501),
    (4, 4, 1000, "ll", 8, 502),
    (3, 1, 333, "ll128", 5, 503),
    (8, 8, 2048, "barrier", 4, 504),
    (8, 8, 4096, "ll", 16, 505),
]


def _existing(x, nranks, ncons, count, proto, nops):
    ws = buffers.Workspace(nranks, count, proto, ncons)
    xd, stride = buffers.rows_to_device(x)
    out = torch.zeros((nops * ncons, stride), dtype=torch.int16, device="cuda")
    ws.sim(nops, xd, stride, out, stride, timeout_ns=TIMEOUT_NS)
    torch.cuda.synchronize()
    assert ws.status() == 0, abi.status_string(ws.status())
    return out


def _static(x, nranks, ncons, count, proto, nops):
    xd, stride = buffers.rows_to_device(x)
    out = torch.full((nops * ncons, stride), -1, dtype=torch.int16, device="cuda")
    status = torch.full((1,), -99, dtype=torch.int32, device="cuda")
    desc = abi.make_desc(nranks, count, proto, ncons)
    p = abi.sim_params(desc, nops, xd, stride, out, stride, None, None, abi.ar_epoch_init(),
                       timeout_ns=TIMEOUT_NS)
    abi.ar_sim_run_static(p, status)
    torch.cuda.synchronize()
    return out, int(status.item())


def test_static_matches_sim_run_on_calls_in_a_row():
    for nranks, ncons, count, proto, nops, seed in CALLS:
        print(f"[no-alloc] N={nranks} C={ncons} count={count} {proto} ops={nops}", flush=True)
        x = inputs.payload(seed, (nops, nranks, count), "normal")
        got, st = _static(x, nranks, ncons, count, proto, nops)
        assert st == 0, abi.status_string(st)
        ref = _existing(x, nranks, ncons, count, proto, nops)
        assert torch.equal(got[:, :count], ref[:, :count]), (nranks, count, proto)
        want = oracle.allreduce_ops(x, proto, 1)
        rows = buffers.rows_from_device(got, count, (nops, ncons))
        for i in range(nops):
            for c in range(ncons):
                assert np.array_equal(rows[i, c], want[i]), (proto, i, c)


def test_static_rejects_what_it_cannot_hold():
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    big = abi.make_desc(16, 1 << 20, "ll", 16)          # 16 consumers x 2 x 16 x 2 MiB
    assert abi.ar_scratch_bytes(big) > abi.AR_STATIC_SCRATCH_BYTES
    p = abi.sim_params(big, 1, 1 << 20, 1 << 20, 1 << 20, 1 << 20, None, None,
                       abi.ar_epoch_init())
    lib = abi.raw()
    assert lib.ar_sim_run_static(ctypes.byref(p), status.data_ptr(), None) == abi.AR_ESIZE
    # a caller-owned buffer is refused: the call uses the library's own
    small = abi.make_desc(4, 64, "ll", 4)
    ws = buffers.Workspace(4, 64, "ll", 4)
    q = abi.sim_params(small, 1, ws.scratch, 64, ws.scratch, 64, ws.scratch, None,
                       abi.ar_epoch_init())
    assert lib.ar_sim_run_static(ctypes.byref(q), status.data_ptr(), None) == abi.AR_EINVAL
