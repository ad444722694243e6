"""GPU parity of the in-kernel send path (include/ar_dev.h) used from a
producer's epilogue, against the CPU oracle.

The producer is a per-rank scale y_r = bf16_rne(f32(x_r) * s_r).  Checked
bit-exactly:
* ar_scale_pack's slot bytes equal the oracle's encoding of the oracle's
  scaled payload, for every protocol, ragged counts and special values;
* fused (ar_scale_pack) and unfused (ar_scale_rows, then ar_pack_*)
  producers give the same slot bytes and the same all-reduce, which equals
  the oracle's all-reduce of the scaled payloads, over alternating epochs;
* the all-gather of scaled payloads.
"""
import numpy as np
import pytest
import torch

import oracle
from collective_synchronization_amd import abi, buffers, inputs

pytestmark = pytest.mark.gpu

TIMEOUT_NS = 2_000_000_000
PROTOS = ("ll", "ll128", "sentinel", "barrier")
SCALES = np.array([1.0, -0.5, 3.0, 1.0078125, 1e-30, 0.0, -7.25, 1e30, 2.0 ** -130,
                   0.1, -1.0, 65504.0, 1.5, -2.0, 0.25, 1e-3], dtype=np.float32)


def _x(seed, shape):
    x = inputs.payload(seed, shape, "normal")
    return inputs.inject(x, seed + 3, 1 / 64,
                         values=(0xFFFF, 0xFFC0, 0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001,
                                 0x7F7F, 0x0080))


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("nranks,ncons,count", [(8, 8, 4096), (3, 1, 1000), (16, 16, 777),
                                                (4, 4, 61), (1, 1, 5), (2, 2, 4099)])
def test_scale_pack_fused_vs_unfused_vs_oracle(proto, nranks, ncons, count):
    print(f"[epilogue] {proto} N={nranks} C={ncons} count={count}", flush=True)
    s = torch.from_numpy(SCALES[:nranks].copy()).to("cuda")
    stride = buffers.row_stride(count)
    fused = buffers.Workspace(nranks, count, proto, ncons)
    plain = buffers.Workspace(nranks, count, proto, ncons)
    outf = torch.zeros((ncons, stride), dtype=torch.int16, device="cuda")
    outp = torch.zeros((ncons, stride), dtype=torch.int16, device="cuda")
    yd = torch.zeros((nranks, stride), dtype=torch.int16, device="cuda")
    E = oracle.encoded_bytes(proto, count)
    for op in range(4):
        x = _x(100 * op + count + nranks, (nranks, count))
        y = np.stack([oracle.scale(x[r], float(SCALES[r])) for r in range(nranks)])
        xd, _ = buffers.rows_to_device(x)
        abi.ar_scale_pack(fused.desc, xd, stride, s, fused.scratch, fused.epoch)
        abi.ar_scale_rows(nranks, count, xd, stride, s, yd, stride)
        plain.pack(yd, stride)
        torch.cuda.synchronize()
        got_y = buffers.rows_from_device(yd, count, (nranks,))
        assert np.array_equal(got_y, y)
        if op < 2:
            sf, sp = fused.slot_view(), plain.slot_view()
            par = fused.epoch.parity
            for c in range(ncons):
                for r in range(nranks):
                    want = oracle.encode(proto, y[r], fused.epoch.seq)
                    assert np.array_equal(sf[c, par, r, :E], want), (op, c, r)
                    assert np.array_equal(sp[c, par, r, :E], want), (op, c, r)
        fused.reduce(outf, stride, timeout_ns=TIMEOUT_NS)
        plain.reduce(outp, stride, timeout_ns=TIMEOUT_NS)
        torch.cuda.synchronize()
        assert fused.status() == 0 and plain.status() == 0
        st, want = oracle.allreduce(y, proto, fused.epoch.seq)
        assert st == oracle.READY
        gf = buffers.rows_from_device(outf, count, (ncons,))
        gp = buffers.rows_from_device(outp, count, (ncons,))
        for c in range(ncons):
            assert np.array_equal(gf[c], want), (op, c)
            assert np.array_equal(gp[c], want), (op, c)
        fused.flip()
        plain.flip()


@pytest.mark.parametrize("proto", PROTOS)
def test_scale_pack_allgather(proto):
    nranks, count = 8, 1000
    s = torch.from_numpy(SCALES[:nranks].copy()).to("cuda")
    ws = buffers.Workspace(nranks, count, proto, nranks, collective="allgather")
    stride = buffers.row_stride(count)
    ostride = ws.gather_stride()
    outd = torch.zeros((nranks, ostride), dtype=torch.int16, device="cuda")
    for op in range(2):
        x = _x(7 + op, (nranks, count))
        y = np.stack([oracle.scale(x[r], float(SCALES[r])) for r in range(nranks)])
        xd, _ = buffers.rows_to_device(x)
        abi.ar_scale_pack(ws.desc, xd, stride, s, ws.scratch, ws.epoch)
        ws.gather(outd, ostride, timeout_ns=TIMEOUT_NS)
        torch.cuda.synchronize()
        assert ws.status() == 0
        st, want = oracle.allgather(y, proto, ws.epoch.seq)
        got = outd.cpu().numpy().view(np.uint16).reshape(nranks, nranks, stride)[..., :count]
        for c in range(nranks):
            assert np.array_equal(got[c], want), (op, c)
        ws.flip()
