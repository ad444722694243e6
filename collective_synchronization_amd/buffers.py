"""Device buffers for the C ABI, allocated with torch (marshalling only).

torch supplies device memory and streams; every step of the all-reduce runs
in the library's kernels.  bf16 payloads are held as int16 tensors of raw
bit patterns, rows padded to a multiple of 8 elements (16 bytes).
"""
from __future__ import annotations

import numpy as np
import torch

from . import abi

ALIGN = 256


def round_up(n: int, m: int) -> int:
    return (n + m - 1) // m * m


def row_stride(count: int) -> int:
    return max(8, round_up(count, 8))


def device_bytes(nbytes: int, device="cuda", fill: int = 0) -> torch.Tensor:
    """A uint8 device tensor of nbytes (>= 256), 256-byte aligned, filled."""
    t = torch.full((max(int(nbytes), ALIGN),), fill, dtype=torch.uint8, device=device)
    if t.data_ptr() % ALIGN:
        raise RuntimeError("allocator returned a buffer that is not 256-byte aligned")
    return t


def rows_to_device(x: np.ndarray, device="cuda"):
    """uint16 [..., count] -> (int16 device tensor [rows, stride], stride)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    count = x.shape[-1]
    stride = row_stride(count)
    flat = x.reshape(-1, count)
    host = np.zeros((flat.shape[0], stride), dtype=np.uint16)
    host[:, :count] = flat
    t = torch.from_numpy(host.view(np.int16)).to(device)
    return t, stride


def rows_from_device(t: torch.Tensor, count: int, shape) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)[:, :count].reshape(tuple(shape) + (count,))


class Workspace:
    """Receive buffers and control block for one descriptor on one device.

    The epoch advances by one flip per op issued through this workspace, as
    the C ABI requires for reused receive buffers.
    """

    def __init__(self, nranks: int, count: int, proto, nconsumers: int = 1,
                 device="cuda", collective=abi.AR_ALLREDUCE):
        self.desc = abi.make_desc(nranks, count, proto, nconsumers, collective)
        self.device = device
        self.scratch_bytes = abi.ar_scratch_bytes(self.desc)
        self.scratch = device_bytes(self.scratch_bytes, device)
        self.ctrl = device_bytes(abi.ar_ctrl_bytes(), device)
        self.epoch = abi.ar_epoch_init()
        if self.desc.proto == abi.AR_SENTINEL:
            abi.ar_arm_sentinel(self.desc, self.scratch, -1)

    @property
    def proto(self) -> int:
        return self.desc.proto

    @property
    def collective(self) -> int:
        return self.desc.collective

    def gather_stride(self) -> int:
        """Output row stride of one all-gather consumer: nranks rows of
        count rounded up to 8 elements."""
        return self.desc.nranks * row_stride(self.desc.count)

    def status(self) -> int:
        return int(self.ctrl[:4].view(torch.int32).item())

    def reset_ctrl(self, stream=None) -> None:
        abi.ar_ctrl_reset(self.ctrl, stream)

    def reset_state(self, stream=None) -> None:
        """Control block, receive buffers and (if allocated) the linear work
        buffer back to their initial state, with fill kernels on the stream.
        Put first in a captured graph, it makes every replay start afresh
        (a replay repeats the epochs captured).  The workspace's epoch stays
        where the capture left it, which is the state a replay leaves."""
        abi.ar_state_reset(self.desc, self.scratch, self.ctrl,
                           getattr(self, "_work", None), stream)

    def slot_view(self) -> np.ndarray:
        """Host copy of the receive buffers: uint8 [nconsumers, 2, nranks, slot]
        ([2 regions, nconsumers, 2, nranks, slot] for the two-shot all-reduce:
        reduce-scatter, then all-gather)."""
        d = self.desc
        slot = abi.ar_desc_slot_bytes(d)
        raw = self.scratch[: self.scratch_bytes].cpu().numpy()
        if d.collective == abi.AR_TWOSHOT:
            return raw.reshape(2, d.nconsumers, 2, d.nranks, slot)
        return raw.reshape(d.nconsumers, 2, d.nranks, slot)

    # -------------------------------------------------- stream-ordered op --
    def pack(self, x_dev, in_stride, stream=None) -> None:
        abi.PACK_BY_PROTO[self.desc.proto](self.desc, x_dev, in_stride, self.scratch,
                                           self.epoch, stream)

    def reduce(self, out_dev, out_stride, timeout_ns=0, rearm=True, stream=None) -> None:
        flags = abi.AR_FLAG_REARM if (rearm and self.desc.proto == abi.AR_SENTINEL) else 0
        abi.ar_reduce_validate(self.desc, self.scratch, out_dev, out_stride, self.epoch,
                               self.ctrl, timeout_ns, flags, stream)

    def gather(self, out_dev, out_stride, timeout_ns=0, rearm=True, stream=None) -> None:
        flags = abi.AR_FLAG_REARM if (rearm and self.desc.proto == abi.AR_SENTINEL) else 0
        abi.ar_gather_validate(self.desc, self.scratch, out_dev, out_stride, self.epoch,
                               self.ctrl, timeout_ns, flags, stream)

    def flip(self, nops: int = 1) -> None:
        abi.ar_epoch_advance(self.epoch, nops)

    # -------------------------------------------------------- simulator --
    def sim_params(self, nops, x_dev, in_stride, out_dev, out_stride, timeout_ns=0,
                   waves_per_rank=0, delay_ticks=None, tile_order=None, trace=None,
                   flags=0):
        return abi.sim_params(self.desc, nops, x_dev, in_stride, out_dev, out_stride,
                              self.scratch, self.ctrl, self.epoch, timeout_ns,
                              waves_per_rank, delay_ticks, tile_order, trace, flags)

    def sim(self, nops, x_dev, in_stride, out_dev, out_stride, stream=None, **kw) -> None:
        """nops back-to-back ops in one persistent launch; advances the epoch."""
        if self.desc.proto == abi.AR_BARRIER:
            self.reset_ctrl(stream)
        p = self.sim_params(nops, x_dev, in_stride, out_dev, out_stride, **kw)
        abi.ar_sim_run(p, stream)
        self.flip(nops)

    def linear_work(self) -> torch.Tensor:
        """The work buffer of ar_sim_linear_run for this descriptor (zeroed
        once, then kept with the epochs of this workspace)."""
        if getattr(self, "_work", None) is None:
            self._work = device_bytes(abi.ar_linear_work_bytes(self.desc), self.device)
        return self._work

    def sim_linear(self, nops, x_dev, in_stride, out_dev, out_stride, weights, layers,
                   stream=None, **kw) -> None:
        """nops chained ops whose producer is a row-parallel linear shard
        (weights: device bf16 [layers, nranks, count, count // nranks]), in
        one persistent launch; advances the epoch."""
        p = self.sim_params(nops, x_dev, in_stride, out_dev, out_stride, **kw)
        abi.ar_sim_linear_run(p, weights, layers, self.linear_work(), stream)
        self.flip(nops)

    def sim_chain(self, nops, x_dev, in_stride, out_dev, out_stride, scales, stream=None,
                  **kw) -> None:
        """nops chained ops in one persistent launch (op i+1's payload is op
        i's result scaled per rank by scales[i+1]); advances the epoch."""
        p = self.sim_params(nops, x_dev, in_stride, out_dev, out_stride, **kw)
        abi.ar_sim_chain_run(p, scales, stream)
        self.flip(nops)
