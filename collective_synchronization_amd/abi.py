"""ctypes binding of ``libcsync_ar.so`` (C ABI declared in ``include/ar.h``).

Argument marshalling only: every step of the all-reduce runs in the HIP
kernels of the library.  Functions keep the C names.  Device buffers may be
given as torch tensors (their ``data_ptr()`` is passed) or as integer device
addresses; ``stream=None`` means torch's current stream on the current
device.  A negative return code raises :class:`ArError`.

The library must be built first (``__graft_entry__.build()``); importing this
module without it raises ImportError -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# AR_LIBRARY: load a variant build instead (for example the library built
# with AR_FORMAL_FENCES=1); unset, the in-tree build
LIB_PATH = os.environ.get("AR_LIBRARY") or os.path.join(_HERE, "libcsync_ar.so")

AR_OK, AR_EINVAL, AR_EALIGN, AR_ESIZE, AR_ELAUNCH = 0, -1, -2, -3, -4
AR_ETIMEOUT, AR_ECORRUPT, AR_ENODEV, AR_ECAPACITY = -5, -6, -7, -8
AR_LL, AR_LL128, AR_SENTINEL, AR_BARRIER, AR_AUTO = 0, 1, 2, 3, 4
AR_FLAG_REARM = 1
AR_SIM_COOPERATIVE = 1
AR_SIM_NARROW = 2
AR_SIM_WIDE = 4
AR_SIM_ORDINARY = 8
AR_MAX_RANKS = 16
AR_MAX_TIMEOUT_NS = 60_000_000_000
AR_STATIC_SCRATCH_BYTES = 64 << 20
AR_ALLREDUCE, AR_ALLGATHER, AR_TWOSHOT = 0, 1, 2
COLLECTIVE_IDS = {"allreduce": AR_ALLREDUCE, "allgather": AR_ALLGATHER,
                  "twoshot": AR_TWOSHOT}
PROTO_IDS = {"ll": AR_LL, "ll128": AR_LL128, "sentinel": AR_SENTINEL,
             "barrier": AR_BARRIER}
PROTO_NAMES = {v: k for k, v in PROTO_IDS.items()}


class ar_desc(ctypes.Structure):
    _fields_ = [("nranks", ctypes.c_int32), ("nconsumers", ctypes.c_int32),
                ("count", ctypes.c_int64), ("proto", ctypes.c_int32),
                ("collective", ctypes.c_int32)]


class ar_epoch(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_uint32), ("parity", ctypes.c_uint32)]

    def __repr__(self):
        return f"ar_epoch(seq={self.seq}, parity={self.parity})"


class ar_sim_params(ctypes.Structure):
    _fields_ = [("desc", ar_desc), ("nops", ctypes.c_int32),
                ("waves_per_rank", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("in_", ctypes.c_void_p), ("in_stride", ctypes.c_int64),
                ("out", ctypes.c_void_p), ("out_stride", ctypes.c_int64),
                ("scratch", ctypes.c_void_p), ("ctrl", ctypes.c_void_p),
                ("epoch", ar_epoch), ("timeout_ns", ctypes.c_uint64),
                ("delay_ticks", ctypes.c_void_p), ("tile_order", ctypes.c_void_p),
                ("trace", ctypes.c_void_p)]


class ar_cost_entry(ctypes.Structure):
    _fields_ = [("nranks", ctypes.c_int32), ("collective", ctypes.c_int32),
                ("max_bytes", ctypes.c_int64),
                ("alpha_us", ctypes.c_double * 4),
                ("beta_us_per_byte", ctypes.c_double * 4)]


class ArError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = f"{where}: {status_string(code)} ({code})"
        if code == AR_ELAUNCH:
            msg += f", hipError {_lib.ar_last_hip_error()}"
        super().__init__(msg)


# torch is imported first so that the one HIP runtime in the process is the one
# torch uses (both carry the soname libamdhip64.so.7): the library then shares
# torch's device context, allocations and streams.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library with "
        "`python -c 'import __graft_entry__ as g; g.build()'` (no CPU fallback exists)")

_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i32, _i64, _u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
_SIGS = {
    "ar_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "ar_abi_version": ([], ctypes.c_int),
    "ar_last_hip_error": ([], ctypes.c_int),
    "ar_encoded_bytes": ([_i32, _i64], _i64),
    "ar_slot_bytes": ([_i32, _i64], _i64),
    "ar_scratch_bytes": ([ctypes.POINTER(ar_desc)], _i64),
    "ar_desc_slot_bytes": ([ctypes.POINTER(ar_desc)], _i64),
    "ar_shard_bounds": ([_i64, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)],
                        ctypes.c_int),
    "ar_ctrl_bytes": ([], _i64),
    "ar_ctrl_reset": ([_vp, _vp], ctypes.c_int),
    "ar_state_reset": ([ctypes.POINTER(ar_desc), _vp, _vp, _vp, _vp], ctypes.c_int),
    "ar_epoch_init": ([ctypes.POINTER(ar_epoch)], ctypes.c_int),
    "ar_epoch_flip": ([ctypes.POINTER(ar_epoch)], ctypes.c_int),
    "ar_epoch_advance": ([ctypes.POINTER(ar_epoch), _u64], ctypes.c_int),
    "ar_pack_ll": ([ctypes.POINTER(ar_desc), _vp, _i64, _vp, ar_epoch, _vp], ctypes.c_int),
    "ar_pack_ll128": ([ctypes.POINTER(ar_desc), _vp, _i64, _vp, ar_epoch, _vp], ctypes.c_int),
    "ar_pack_sentinel": ([ctypes.POINTER(ar_desc), _vp, _i64, _vp, ar_epoch, _vp], ctypes.c_int),
    "ar_pack_plain": ([ctypes.POINTER(ar_desc), _vp, _i64, _vp, ar_epoch, _vp], ctypes.c_int),
    "ar_arm_sentinel": ([ctypes.POINTER(ar_desc), _vp, _i32, _vp], ctypes.c_int),
    "ar_reduce_validate": ([ctypes.POINTER(ar_desc), _vp, _vp, _i64, ar_epoch, _vp,
                            _u64, _i32, _vp], ctypes.c_int),
    "ar_gather_validate": ([ctypes.POINTER(ar_desc), _vp, _vp, _i64, ar_epoch, _vp,
                            _u64, _i32, _vp], ctypes.c_int),
    "ar_scale_pack": ([ctypes.POINTER(ar_desc), _vp, _i64, _vp, _vp, ar_epoch, _vp],
                      ctypes.c_int),
    "ar_scale_rows": ([_i32, _i64, _vp, _i64, _vp, _vp, _i64, _vp], ctypes.c_int),
    "ar_sim_run": ([ctypes.POINTER(ar_sim_params), _vp], ctypes.c_int),
    "ar_sim_run_static": ([ctypes.POINTER(ar_sim_params), _vp, _vp], ctypes.c_int),
    "ar_sim_chain_run": ([ctypes.POINTER(ar_sim_params), _vp, _vp], ctypes.c_int),
    "ar_sim_chain_geometry": ([ctypes.POINTER(ar_sim_params), ctypes.POINTER(_i32),
                               ctypes.POINTER(_i32)], ctypes.c_int),
    "ar_linear_work_bytes": ([ctypes.POINTER(ar_desc)], _i64),
    "ar_sim_linear_run": ([ctypes.POINTER(ar_sim_params), _vp, _i32, _vp, _vp], ctypes.c_int),
    "ar_sim_linear_geometry": ([ctypes.POINTER(ar_sim_params), _vp, _i32, _vp,
                                ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                                ctypes.POINTER(_i32)], ctypes.c_int),
    "ar_sim_geometry": ([ctypes.POINTER(ar_sim_params), ctypes.POINTER(_i32),
                         ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                         ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                         ctypes.POINTER(_i32)], ctypes.c_int),
    "ar_wallclock_hz": ([ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    "ar_select_protocol": ([ctypes.POINTER(ar_cost_entry), _i32, _i64, _i32,
                            ctypes.POINTER(_i32), ctypes.POINTER(ctypes.c_double)],
                           ctypes.c_int),
    "ar_select_collective": ([ctypes.POINTER(ar_cost_entry), _i32, _i32, _i64, _i32,
                              ctypes.POINTER(_i32), ctypes.POINTER(ctypes.c_double)],
                             ctypes.c_int),
    "ar_select_allreduce": ([ctypes.POINTER(ar_cost_entry), _i32, _i64, _i32,
                             ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                             ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    "ar_probe_pingpong": ([_vp, _i32, _i32, _i32, _vp, _vp], ctypes.c_int),
    "ar_probe_loadchain": ([_vp, _i64, _i32, _vp, _vp], ctypes.c_int),
    "ar_probe_litmus": ([_vp, _i32, _i32, _i32, _i32, _vp, _vp], ctypes.c_int),
    "ar_probe_copy": ([_vp, _vp, _i64, _vp], ctypes.c_int),
    "ar_probe_empty": ([_vp], ctypes.c_int),
    "ar_probe_placement": ([_i32, _i32, _vp, _vp, _vp], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


def raw():
    """The ctypes CDLL handle (for tests of the bare C ABI)."""
    return _lib


# ------------------------------------------------------------ marshalling --

def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(code: int, where: str) -> int:
    if code < 0:
        raise ArError(code, where)
    return code


def status_string(code: int) -> str:
    return _lib.ar_status_string(code).decode()


def proto_id(p) -> int:
    return PROTO_IDS[p] if isinstance(p, str) else int(p)


def collective_id(c) -> int:
    return COLLECTIVE_IDS[c] if isinstance(c, str) else int(c)


def make_desc(nranks: int, count: int, proto, nconsumers: int = 1,
              collective=AR_ALLREDUCE) -> ar_desc:
    return ar_desc(nranks, nconsumers, count, proto_id(proto), collective_id(collective))


# ---------------------------------------------------------------- sizes ---

def ar_encoded_bytes(proto, count: int) -> int:
    return _check(_lib.ar_encoded_bytes(proto_id(proto), count), "ar_encoded_bytes")


def ar_slot_bytes(proto, count: int) -> int:
    return _check(_lib.ar_slot_bytes(proto_id(proto), count), "ar_slot_bytes")


def ar_scratch_bytes(desc: ar_desc) -> int:
    return _check(_lib.ar_scratch_bytes(ctypes.byref(desc)), "ar_scratch_bytes")


def ar_desc_slot_bytes(desc: ar_desc) -> int:
    return _check(_lib.ar_desc_slot_bytes(ctypes.byref(desc)), "ar_desc_slot_bytes")


def ar_shard_bounds(count: int, nranks: int, k: int):
    lo, hi = _i64(), _i64()
    _check(_lib.ar_shard_bounds(count, nranks, k, ctypes.byref(lo), ctypes.byref(hi)),
           "ar_shard_bounds")
    return lo.value, hi.value


def ar_ctrl_bytes() -> int:
    return _check(_lib.ar_ctrl_bytes(), "ar_ctrl_bytes")


# --------------------------------------------------------------- epochs ---

def ar_epoch_init() -> ar_epoch:
    e = ar_epoch()
    _check(_lib.ar_epoch_init(ctypes.byref(e)), "ar_epoch_init")
    return e


def ar_epoch_flip(e: ar_epoch) -> ar_epoch:
    _check(_lib.ar_epoch_flip(ctypes.byref(e)), "ar_epoch_flip")
    return e


def ar_epoch_advance(e: ar_epoch, nops: int) -> ar_epoch:
    _check(_lib.ar_epoch_advance(ctypes.byref(e), nops), "ar_epoch_advance")
    return e


# --------------------------------------------------------------- device ---

def ar_ctrl_reset(ctrl, stream=None) -> None:
    _check(_lib.ar_ctrl_reset(_ptr(ctrl), _stream(stream)), "ar_ctrl_reset")


def ar_state_reset(desc, scratch=None, ctrl=None, work=None, stream=None) -> None:
    """Initial state of the given buffers (None: left alone), with fill
    kernels: the head of a captured sequence that is to be replayed."""
    _check(_lib.ar_state_reset(ctypes.byref(desc), _ptr(scratch), _ptr(ctrl), _ptr(work),
                               _stream(stream)), "ar_state_reset")


def _pack(name, desc, inp, in_stride, scratch, epoch, stream):
    fn = getattr(_lib, name)
    _check(fn(ctypes.byref(desc), _ptr(inp), in_stride, _ptr(scratch), epoch,
              _stream(stream)), name)


def ar_pack_ll(desc, inp, in_stride, scratch, epoch, stream=None) -> None:
    _pack("ar_pack_ll", desc, inp, in_stride, scratch, epoch, stream)


def ar_pack_ll128(desc, inp, in_stride, scratch, epoch, stream=None) -> None:
    _pack("ar_pack_ll128", desc, inp, in_stride, scratch, epoch, stream)


def ar_pack_sentinel(desc, inp, in_stride, scratch, epoch, stream=None) -> None:
    _pack("ar_pack_sentinel", desc, inp, in_stride, scratch, epoch, stream)


def ar_pack_plain(desc, inp, in_stride, scratch, epoch, stream=None) -> None:
    _pack("ar_pack_plain", desc, inp, in_stride, scratch, epoch, stream)


PACK_BY_PROTO = {AR_LL: ar_pack_ll, AR_LL128: ar_pack_ll128,
                 AR_SENTINEL: ar_pack_sentinel, AR_BARRIER: ar_pack_plain}


def ar_arm_sentinel(desc, scratch, parity: int = -1, stream=None) -> None:
    _check(_lib.ar_arm_sentinel(ctypes.byref(desc), _ptr(scratch), parity,
                                _stream(stream)), "ar_arm_sentinel")


def ar_reduce_validate(desc, scratch, out, out_stride, epoch, ctrl,
                       timeout_ns: int = 0, flags: int = 0, stream=None) -> None:
    _check(_lib.ar_reduce_validate(ctypes.byref(desc), _ptr(scratch), _ptr(out),
                                   out_stride, epoch, _ptr(ctrl), timeout_ns, flags,
                                   _stream(stream)), "ar_reduce_validate")


def ar_gather_validate(desc, scratch, out, out_stride, epoch, ctrl,
                       timeout_ns: int = 0, flags: int = 0, stream=None) -> None:
    _check(_lib.ar_gather_validate(ctypes.byref(desc), _ptr(scratch), _ptr(out),
                                   out_stride, epoch, _ptr(ctrl), timeout_ns, flags,
                                   _stream(stream)), "ar_gather_validate")


def ar_scale_pack(desc, inp, in_stride, scales, scratch, epoch, stream=None) -> None:
    _check(_lib.ar_scale_pack(ctypes.byref(desc), _ptr(inp), in_stride, _ptr(scales),
                              _ptr(scratch), epoch, _stream(stream)), "ar_scale_pack")


def ar_scale_rows(nranks, count, inp, in_stride, scales, out, out_stride,
                  stream=None) -> None:
    _check(_lib.ar_scale_rows(nranks, count, _ptr(inp), in_stride, _ptr(scales), _ptr(out),
                              out_stride, _stream(stream)), "ar_scale_rows")


def sim_params(desc, nops, inp, in_stride, out, out_stride, scratch, ctrl, epoch,
               timeout_ns=0, waves_per_rank=0, delay_ticks=None, tile_order=None,
               trace=None, flags=0) -> ar_sim_params:
    return ar_sim_params(desc, nops, waves_per_rank, flags, 0, _ptr(inp), in_stride,
                         _ptr(out), out_stride, _ptr(scratch), _ptr(ctrl), epoch,
                         timeout_ns, _ptr(delay_ticks), _ptr(tile_order), _ptr(trace))


def ar_sim_run(params: ar_sim_params, stream=None) -> None:
    _check(_lib.ar_sim_run(ctypes.byref(params), _stream(stream)), "ar_sim_run")


def ar_sim_run_static(params: ar_sim_params, status, stream=None) -> None:
    """ar_sim_run on the library's own receive buffers (params.scratch and
    params.ctrl must be None); status: device int32, written after the run."""
    _check(_lib.ar_sim_run_static(ctypes.byref(params), _ptr(status), _stream(stream)),
           "ar_sim_run_static")


def ar_sim_chain_run(params: ar_sim_params, scales, stream=None) -> None:
    """scales: device float32 [nops, nranks] (op 0's row unused)."""
    _check(_lib.ar_sim_chain_run(ctypes.byref(params), _ptr(scales), _stream(stream)),
           "ar_sim_chain_run")


def ar_sim_chain_geometry(params: ar_sim_params) -> dict:
    b, coop = _i32(), _i32()
    _check(_lib.ar_sim_chain_geometry(ctypes.byref(params), ctypes.byref(b), ctypes.byref(coop)),
           "ar_sim_chain_geometry")
    return {"blocks": b.value, "launch": "cooperative" if coop.value else "ordinary"}


def ar_linear_work_bytes(desc: ar_desc) -> int:
    return _check(_lib.ar_linear_work_bytes(ctypes.byref(desc)), "ar_linear_work_bytes")


def ar_sim_linear_run(params: ar_sim_params, weights, layers: int, work, stream=None) -> None:
    """weights: device bf16 [layers, nranks, count, count // nranks]; work:
    device, ar_linear_work_bytes(desc) bytes, zero-filled when allocated."""
    _check(_lib.ar_sim_linear_run(ctypes.byref(params), _ptr(weights), layers, _ptr(work),
                                  _stream(stream)), "ar_sim_linear_run")


def ar_sim_linear_geometry(params: ar_sim_params, weights, layers: int, work) -> dict:
    b, wk, coop = _i32(), _i32(), _i32()
    _check(_lib.ar_sim_linear_geometry(ctypes.byref(params), _ptr(weights), layers, _ptr(work),
                                       ctypes.byref(b), ctypes.byref(wk), ctypes.byref(coop)),
           "ar_sim_linear_geometry")
    return {"blocks": b.value, "workers": wk.value,
            "launch": "cooperative" if coop.value else "ordinary"}


def ar_sim_geometry(params: ar_sim_params) -> dict:
    w, t, tpw, b, wide, coop = _i32(), _i32(), _i32(), _i32(), _i32(), _i32()
    _check(_lib.ar_sim_geometry(ctypes.byref(params), ctypes.byref(w), ctypes.byref(t),
                                ctypes.byref(tpw), ctypes.byref(b), ctypes.byref(wide),
                                ctypes.byref(coop)),
           "ar_sim_geometry")
    return {"waves_per_rank": w.value, "tiles_per_rank": t.value,
            "tiles_per_wave": tpw.value, "blocks": b.value,
            "kernel": "wide" if wide.value else "narrow",
            "launch": "cooperative" if coop.value else "ordinary"}


def ar_wallclock_hz() -> float:
    hz = ctypes.c_double()
    _check(_lib.ar_wallclock_hz(ctypes.byref(hz)), "ar_wallclock_hz")
    return hz.value


def cost_table(entries) -> "ctypes.Array":
    """entries: iterable of dicts {nranks, alpha_us[4], beta_us_per_byte[4]}
    and optionally max_bytes (upper end of the size range; absent or <= 0:
    no upper end) and collective (name or id; absent: one-shot all-reduce).
    A None coefficient (an unavailable protocol) is passed as NaN."""
    entries = list(entries)
    arr = (ar_cost_entry * len(entries))()
    for i, e in enumerate(entries):
        arr[i].nranks = int(e["nranks"])
        arr[i].collective = collective_id(e.get("collective", AR_ALLREDUCE))
        arr[i].max_bytes = int(e.get("max_bytes", 0))
        for p in range(4):
            a, b = e["alpha_us"][p], e["beta_us_per_byte"][p]
            arr[i].alpha_us[p] = float("nan") if a is None else float(a)
            arr[i].beta_us_per_byte[p] = float("nan") if b is None else float(b)
    return arr


def ar_select_protocol(table, payload_bytes: int, nranks: int):
    """Returns (protocol id, predicted microseconds)."""
    out = _i32()
    pred = ctypes.c_double()
    _check(_lib.ar_select_protocol(table, len(table), payload_bytes, nranks,
                                   ctypes.byref(out), ctypes.byref(pred)),
           "ar_select_protocol")
    return out.value, pred.value


def ar_select_collective(table, collective, payload_bytes: int, nranks: int):
    """Returns (protocol id, predicted microseconds) for one collective."""
    out = _i32()
    pred = ctypes.c_double()
    _check(_lib.ar_select_collective(table, len(table), collective_id(collective),
                                     payload_bytes, nranks, ctypes.byref(out),
                                     ctypes.byref(pred)), "ar_select_collective")
    return out.value, pred.value


def ar_select_allreduce(table, payload_bytes: int, nranks: int):
    """Returns (collective id, protocol id, predicted microseconds)."""
    coll, out = _i32(), _i32()
    pred = ctypes.c_double()
    _check(_lib.ar_select_allreduce(table, len(table), payload_bytes, nranks,
                                    ctypes.byref(coll), ctypes.byref(out),
                                    ctypes.byref(pred)), "ar_select_allreduce")
    return coll.value, out.value, pred.value


def ar_probe_pingpong(work, iters, xcd_a, xcd_b, result, stream=None) -> None:
    _check(_lib.ar_probe_pingpong(_ptr(work), iters, xcd_a, xcd_b, _ptr(result),
                                  _stream(stream)), "ar_probe_pingpong")


def ar_probe_loadchain(work, nbytes, iters, result, stream=None) -> None:
    _check(_lib.ar_probe_loadchain(_ptr(work), nbytes, iters, _ptr(result),
                                   _stream(stream)), "ar_probe_loadchain")


def ar_probe_litmus(work, iters, xcd_a, xcd_b, kind, result, stream=None) -> None:
    _check(_lib.ar_probe_litmus(_ptr(work), iters, xcd_a, xcd_b, kind, _ptr(result),
                                _stream(stream)), "ar_probe_litmus")


def ar_probe_copy(src, dst, nbytes, stream=None) -> None:
    _check(_lib.ar_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)),
           "ar_probe_copy")


def ar_probe_empty(stream=None) -> None:
    _check(_lib.ar_probe_empty(_stream(stream)), "ar_probe_empty")


def ar_probe_placement(blocks: int, threads: int, work, result, stream=None) -> None:
    _check(_lib.ar_probe_placement(blocks, threads, _ptr(work), _ptr(result), _stream(stream)),
           "ar_probe_placement")
