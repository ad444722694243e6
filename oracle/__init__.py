"""CPU oracle for the self-synchronizing bf16 all-reduce (one-shot and
two-shot) and all-gather.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``collective_synchronization_amd``) never imports it, and this package
never imports the product: the two share no code.

This module is a thin ctypes/numpy wrapper over ``oracle/ar_oracle.c`` (plain
C, one element at a time).  Every function here only marshals arrays; the
arithmetic is in the C file, which cites the pages it follows:

* "Why Microseconds Matter in AI Infrastructure", section "Latency can matter
  more than bandwidth" -- LL flag packing, LL128 lines, the negative-NaN
  sentinel, double buffering;
* "flash-comm: Self-Synchronizing Collective Communication for LLM Decoding",
  abstract -- per-block readiness evidence, fixed reduction order;
* "SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM Inference",
  abstract -- one-shot all-reduce with dual buffering; the two-shot form
  (reduce-scatter of shares, then all-gather) for more GPUs;
* flash-comm abstract again -- the same transfers carry a standalone
  all-gather;
* "Why Microseconds Matter in AI Infrastructure", section "Communication is
  becoming part of GPU execution" -- send/receive/reduce called from inside
  the producing kernel (the producer epilogue used for it: a per-rank scale),
  and the chain in which each all-reduce's result feeds that producer for
  the next all-reduce (``chain_ops``);
* "SiFAR" abstract -- communication and model execution designed together,
  the all-reduce result being the next layer's input: the chain whose
  producer is a row-parallel linear layer shard (``linear_chain_ops``; its
  dot products are pairwise binary32 sums, ``linear_dot``).

Pins: every function is checked by ``tests/test_oracle_*.py`` against
something other than itself (exhaustive sweeps against torch and numpy, an
exact rational emulation of binary32 addition, closed forms and hand-written
golden byte vectors under ``tests/golden/``).  The byte layouts have no
counterpart on the pages (they print none), so their parity with the pages is
unpinned; they are pinned to the stated layout by the golden vectors.
"""
from __future__ import annotations

import ctypes
import os
import time

import numpy as np

LL, LL128, SENTINEL, BARRIER = 0, 1, 2, 3
PROTOS = {"ll": LL, "ll128": LL128, "sentinel": SENTINEL, "barrier": BARRIER}
READY, NOT_READY, CORRUPT = 0, 1, 2
SENTINEL_BITS = 0xFFFF
CANON_NAN = 0x7FC0

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libar_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # compile on first use (CPU only)
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    f32p = ctypes.POINTER(ctypes.c_float)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64 = ctypes.c_int64
    lib.o_bf16_rne.argtypes = [ctypes.c_float]
    lib.o_bf16_rne.restype = ctypes.c_uint16
    lib.o_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.o_bf16_to_f32.restype = ctypes.c_float
    lib.o_canon_in.argtypes = [ctypes.c_uint16]
    lib.o_canon_in.restype = ctypes.c_uint16
    lib.o_epoch_next.argtypes = [ctypes.c_uint32]
    lib.o_epoch_next.restype = ctypes.c_uint32
    lib.o_epoch_prev.argtypes = [ctypes.c_uint32]
    lib.o_epoch_prev.restype = ctypes.c_uint32
    lib.o_encoded_bytes.argtypes = [ctypes.c_int, i64]
    lib.o_encoded_bytes.restype = i64
    lib.o_encode.argtypes = [ctypes.c_int, u16p, i64, ctypes.c_uint32, u8p]
    lib.o_encode.restype = i64
    lib.o_decode.argtypes = [ctypes.c_int, u8p, i64, ctypes.c_uint32, u16p]
    lib.o_decode.restype = ctypes.c_int
    lib.o_reduce.argtypes = [ctypes.c_int, u16p, i64, u16p]
    lib.o_reduce.restype = None
    lib.o_allreduce.argtypes = [ctypes.c_int, u16p, i64, ctypes.c_int,
                                ctypes.c_uint32, i32p, u16p]
    lib.o_allreduce.restype = ctypes.c_int
    lib.o_shard_bounds.argtypes = [i64, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.o_shard_bounds.restype = None
    lib.o_allgather.argtypes = [ctypes.c_int, u16p, i64, ctypes.c_int,
                                ctypes.c_uint32, i32p, u16p]
    lib.o_allgather.restype = ctypes.c_int
    lib.o_twoshot.argtypes = [ctypes.c_int, u16p, i64, ctypes.c_int,
                              ctypes.c_uint32, u16p]
    lib.o_twoshot.restype = ctypes.c_int
    lib.o_scale.argtypes = [u16p, i64, ctypes.c_float, u16p]
    lib.o_scale.restype = None
    lib.o_linear_dot.argtypes = [u16p, u16p, i64]
    lib.o_linear_dot.restype = ctypes.c_float
    lib.o_linear_shard.argtypes = [u16p, i64, u16p, i64, u16p]
    lib.o_linear_shard.restype = None
    lib.o_bf16_rne_array.argtypes = [f32p, i64, u16p]
    lib.o_bf16_rne_array.restype = None
    lib.o_canon_in_array.argtypes = [u16p, i64, u16p]
    lib.o_canon_in_array.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bf16 bit patterns, got {a.dtype}")
    return a


def proto_id(p) -> int:
    return PROTOS[p] if isinstance(p, str) else int(p)


# ----------------------------------------------------------------- scalars --

def bf16_rne_scalar(f: float) -> int:
    return int(_load().o_bf16_rne(ctypes.c_float(f)))


def canon_in_scalar(b: int) -> int:
    return int(_load().o_canon_in(b))


def epoch_next(seq: int) -> int:
    return int(_load().o_epoch_next(seq))


def epoch_prev(seq: int) -> int:
    return int(_load().o_epoch_prev(seq))


def encoded_bytes(proto, count: int) -> int:
    return int(_load().o_encoded_bytes(proto_id(proto), count))


# ------------------------------------------------------------------ arrays --

def bf16_rne(f: np.ndarray) -> np.ndarray:
    """binary32 array -> bf16 bit patterns (uint16), RNE, NaN -> 0x7FC0."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    _load().o_bf16_rne_array(_ptr(f, ctypes.c_float), f.size, _ptr(out, ctypes.c_uint16))
    return out


def canon_in(b: np.ndarray) -> np.ndarray:
    b = _u16(b)
    out = np.empty(b.shape, dtype=np.uint16)
    _load().o_canon_in_array(_ptr(b, ctypes.c_uint16), b.size, _ptr(out, ctypes.c_uint16))
    return out


def encode(proto, x: np.ndarray, seq: int) -> np.ndarray:
    """Encode one rank's payload (uint16 [count]) -> uint8 [E]."""
    x = _u16(x).reshape(-1)
    p = proto_id(proto)
    E = encoded_bytes(p, x.size)
    out = np.zeros(max(E, 1), dtype=np.uint8)
    _load().o_encode(p, _ptr(x, ctypes.c_uint16), x.size, seq, _ptr(out, ctypes.c_uint8))
    return out[:E]


def decode(proto, wire: np.ndarray, count: int, seq: int):
    """Validate + decode one slot -> (status, uint16 [count])."""
    p = proto_id(proto)
    E = encoded_bytes(p, count)
    wire = np.ascontiguousarray(wire, dtype=np.uint8).reshape(-1)
    if wire.size < E:
        raise ValueError(f"slot has {wire.size} bytes, encoding needs {E}")
    y = np.zeros(max(count, 1), dtype=np.uint16)
    st = _load().o_decode(p, _ptr(wire, ctypes.c_uint8), count, seq, _ptr(y, ctypes.c_uint16))
    return int(st), y[:count]


def reduce(y: np.ndarray) -> np.ndarray:
    """Fixed-order fp32 sum of n rank rows (uint16 [n, count]) -> uint16 [count]."""
    y = _u16(y)
    n, count = y.shape
    out = np.zeros(max(count, 1), dtype=np.uint16)
    _load().o_reduce(n, _ptr(y, ctypes.c_uint16), count, _ptr(out, ctypes.c_uint16))
    return out[:count]


def allreduce(x: np.ndarray, proto="ll", seq: int = 1, perm=None):
    """Encode, deliver in `perm` order, validate, decode, reduce in rank order.

    x: uint16 [n, count].  Returns (status, uint16 [count]).
    """
    x = _u16(x)
    n, count = x.shape
    out = np.zeros(max(count, 1), dtype=np.uint16)
    pp = None
    if perm is not None:
        perm = np.ascontiguousarray(perm, dtype=np.int32)
        if perm.shape != (n,):
            raise ValueError("perm must be a permutation of range(n)")
        pp = _ptr(perm, ctypes.c_int32)
    st = _load().o_allreduce(n, _ptr(x, ctypes.c_uint16), count, proto_id(proto),
                             seq, pp, _ptr(out, ctypes.c_uint16))
    return int(st), out[:count]


def allreduce_ops(x: np.ndarray, proto="ll", seq0: int = 1) -> np.ndarray:
    """Expected outputs of K back-to-back ops: x uint16 [K, n, count] -> [K, count].

    Op i uses epoch seq0 advanced i times (the result does not depend on it).
    """
    x = _u16(x)
    K, n, count = x.shape
    out = np.empty((K, count), dtype=np.uint16)
    seq = seq0
    for i in range(K):
        st, out[i] = allreduce(x[i], proto, seq)
        if st != READY:
            raise RuntimeError(f"oracle op {i} not ready: status {st}")
        seq = epoch_next(seq)
    return out


def scale(x: np.ndarray, s: float) -> np.ndarray:
    """Producer epilogue: bf16_rne(f32(x) * s), one binary32 multiply per
    element.  x: uint16 [count] -> uint16 [count]."""
    x = _u16(x).reshape(-1)
    out = np.zeros(max(x.size, 1), dtype=np.uint16)
    _load().o_scale(_ptr(x, ctypes.c_uint16), x.size, ctypes.c_float(s),
                    _ptr(out, ctypes.c_uint16))
    return out[:x.size]


def chain_ops(x0: np.ndarray, scales: np.ndarray, proto="ll", seq0: int = 1) -> np.ndarray:
    """Expected outputs of K chained all-reduces, each op's result feeding the
    next op's producer ("Why Microseconds Matter in AI Infrastructure",
    section "Communication is becoming part of GPU execution": the producing
    computation and the communication in one kernel; the producer is the
    per-rank scale above).  x0: uint16 [n, count], op 0's payloads; scales:
    float32 [K, n], row 0 unused.  Op 0 all-reduces x0; op i+1's payload of
    rank r is scale(out_i, scales[i+1, r]).  Returns uint16 [K, count]."""
    x = _u16(x0)
    n, count = x.shape
    s = np.asarray(scales, dtype=np.float32)
    if s.ndim != 2 or s.shape[1] != n:
        raise ValueError("scales must be [K, n]")
    K = s.shape[0]
    out = np.empty((K, count), dtype=np.uint16)
    seq = seq0
    for i in range(K):
        st, out[i] = allreduce(x, proto, seq)
        if st != READY:
            raise RuntimeError(f"oracle chained op {i} not ready: status {st}")
        if i + 1 < K:
            x = np.stack([scale(out[i], float(s[i + 1, r])) for r in range(n)])
        seq = epoch_next(seq)
    return out


def linear_dot(v: np.ndarray, w: np.ndarray) -> float:
    """Pairwise binary32 sum of the products f32(v[k]) * f32(w[k]) (the
    linear producer's dot product before its bf16 rounding).  v, w: uint16
    [kr], kr >= 1.  Returns the binary32 value as a Python float."""
    v = _u16(v).reshape(-1)
    w = _u16(w).reshape(-1)
    if v.size != w.size or v.size < 1:
        raise ValueError("v and w must have the same length >= 1")
    return float(_load().o_linear_dot(_ptr(v, ctypes.c_uint16), _ptr(w, ctypes.c_uint16),
                                      v.size))


def linear_shard(v: np.ndarray, wt: np.ndarray) -> np.ndarray:
    """One rank's row-parallel linear partial output: v uint16 [kr] (its
    input slice), wt uint16 [count, kr] (row j = output j's weights over the
    slice) -> uint16 [count], y[j] = bf16_rne(linear_dot(v, wt[j]))."""
    v = _u16(v).reshape(-1)
    wt = _u16(wt)
    if wt.ndim != 2 or wt.shape[1] != v.size or v.size < 1:
        raise ValueError("wt must be [count, kr] with kr = len(v) >= 1")
    count = wt.shape[0]
    out = np.zeros(max(count, 1), dtype=np.uint16)
    _load().o_linear_shard(_ptr(v, ctypes.c_uint16), v.size, _ptr(wt, ctypes.c_uint16),
                           count, _ptr(out, ctypes.c_uint16))
    return out[:count]


def linear_chain_ops(x0: np.ndarray, weights: np.ndarray, nops: int, proto="ll",
                     seq0: int = 1) -> np.ndarray:
    """Expected outputs of `nops` chained all-reduces whose producer is a
    row-parallel linear layer shard ("SiFAR" abstract: the all-reduce result
    is the next layer's input; "Why Microseconds Matter in AI
    Infrastructure", section "Communication is becoming part of GPU
    execution": the producer sends from its own kernel).

    x0: uint16 [n, count], the layer input of op 0 as rank r holds it (rank
    r reads only its slice [r*kr, (r+1)*kr), kr = count / n).  weights:
    uint16 [L, n, count, kr]; op i uses layer i % L, rank r's shard
    weights[i % L, r].  Op i: rank r's payload is linear_shard(slice r of
    its layer input, weights[i % L, r]); the payloads are all-reduced
    (allreduce); op i+1's layer input, on every rank, is op i's result.
    Returns uint16 [nops, count]."""
    x = _u16(x0)
    w = _u16(weights)
    n, count = x.shape
    if w.ndim != 4 or w.shape[1] != n or w.shape[2] != count or w.shape[3] * n != count:
        raise ValueError("weights must be [L, n, count, count // n]")
    L, kr = w.shape[0], w.shape[3]
    out = np.empty((nops, count), dtype=np.uint16)
    seq = seq0
    inputs = [x[r] for r in range(n)]
    for i in range(nops):
        y = np.stack([linear_shard(inputs[r][r * kr:(r + 1) * kr], w[i % L, r])
                      for r in range(n)])
        st, out[i] = allreduce(y, proto, seq)
        if st != READY:
            raise RuntimeError(f"oracle linear op {i} not ready: status {st}")
        inputs = [out[i]] * n
        seq = epoch_next(seq)
    return out


def shard_bounds(count: int, n: int, k: int):
    """[lo, hi) of the share rank k owns in a two-shot all-reduce."""
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    _load().o_shard_bounds(count, n, k, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def allgather(x: np.ndarray, proto="ll", seq: int = 1, perm=None):
    """Encode, deliver in `perm` order, validate and decode every rank's
    payload.  x: uint16 [n, count].  Returns (status, uint16 [n, count])."""
    x = _u16(x)
    n, count = x.shape
    out = np.zeros((n, max(count, 1)), dtype=np.uint16)
    pp = None
    if perm is not None:
        perm = np.ascontiguousarray(perm, dtype=np.int32)
        if perm.shape != (n,):
            raise ValueError("perm must be a permutation of range(n)")
        pp = _ptr(perm, ctypes.c_int32)
    st = _load().o_allgather(n, _ptr(x, ctypes.c_uint16), count, proto_id(proto),
                             seq, pp, _ptr(out, ctypes.c_uint16))
    return int(st), out[:, :count]


def allgather_ops(x: np.ndarray, proto="ll", seq0: int = 1) -> np.ndarray:
    """Expected outputs of K back-to-back all-gathers: [K, n, count] -> [K, n, count]."""
    x = _u16(x)
    K = x.shape[0]
    out = np.empty_like(x)
    seq = seq0
    for i in range(K):
        st, out[i] = allgather(x[i], proto, seq)
        if st != READY:
            raise RuntimeError(f"oracle all-gather {i} not ready: status {st}")
        seq = epoch_next(seq)
    return out


def twoshot(x: np.ndarray, proto="ll", seq: int = 1):
    """Two-shot all-reduce: reduce-scatter of shares, then all-gather of the
    reduced shares.  x: uint16 [n, count].  Returns (status, uint16 [count])."""
    x = _u16(x)
    n, count = x.shape
    out = np.zeros(max(count, 1), dtype=np.uint16)
    st = _load().o_twoshot(n, _ptr(x, ctypes.c_uint16), count, proto_id(proto), seq,
                           _ptr(out, ctypes.c_uint16))
    return int(st), out[:count]


def twoshot_ops(x: np.ndarray, proto="ll", seq0: int = 1) -> np.ndarray:
    """Expected outputs of K back-to-back two-shot all-reduces: [K, n, count] -> [K, count]."""
    x = _u16(x)
    K, n, count = x.shape
    out = np.empty((K, count), dtype=np.uint16)
    seq = seq0
    for i in range(K):
        st, out[i] = twoshot(x[i], proto, seq)
        if st != READY:
            raise RuntimeError(f"oracle two-shot {i} not ready: status {st}")
        seq = epoch_next(seq)
    return out


def time_collective(x: np.ndarray, proto="sentinel", collective="allreduce",
                    seconds: float = 10.0, seq0: int = 1):
    """Time the oracle (single thread) on x uint16 [K, n, count] for ~seconds,
    as seen by one receiving rank: "allreduce" (o_allreduce), "allgather"
    (o_allgather) or "twoshot" (o_twoshot: every share's reduce-scatter,
    reduce and all-gather).  Returns (microseconds per op, ops run)."""
    if collective == "allreduce":
        return time_allreduce(x, proto, seconds, seq0)
    x = _u16(x)
    K, n, count = x.shape
    lib = _load()
    p = proto_id(proto)
    if collective == "allgather":
        out = np.zeros((n, max(count, 1)), dtype=np.uint16)
    elif collective == "twoshot":
        out = np.zeros(max(count, 1), dtype=np.uint16)
    else:
        raise ValueError(f"unknown collective {collective!r}")
    optr = _ptr(out, ctypes.c_uint16)
    rows = [np.ascontiguousarray(x[i]) for i in range(K)]
    ptrs = [_ptr(r, ctypes.c_uint16) for r in rows]
    seq = seq0
    ops = 0
    t0 = time.perf_counter()
    deadline = t0 + seconds
    while True:
        for i in range(K):
            if collective == "allgather":
                lib.o_allgather(n, ptrs[i], count, p, seq, None, optr)
            else:
                lib.o_twoshot(n, ptrs[i], count, p, seq, optr)
            seq = seq + 1 if seq != 0xFFFFFFFF else 1
            ops += 1
        if time.perf_counter() >= deadline:
            break
    dt = time.perf_counter() - t0
    return dt * 1e6 / ops, ops


def time_allreduce(x: np.ndarray, proto="sentinel", seconds: float = 10.0,
                   seq0: int = 1):
    """Time the oracle (single thread) on x uint16 [K, n, count] for ~seconds.

    Returns (microseconds per all-reduce, number of ops run).  Each op is one
    complete o_allreduce call: encode n + decode n + fixed-order reduce.
    """
    x = _u16(x)
    K, n, count = x.shape
    lib = _load()
    p = proto_id(proto)
    out = np.zeros(max(count, 1), dtype=np.uint16)
    optr = _ptr(out, ctypes.c_uint16)
    rows = [np.ascontiguousarray(x[i]) for i in range(K)]
    ptrs = [_ptr(r, ctypes.c_uint16) for r in rows]
    seq = seq0
    ops = 0
    t0 = time.perf_counter()
    deadline = t0 + seconds
    while True:
        for i in range(K):
            lib.o_allreduce(n, ptrs[i], count, p, seq, None, optr)
            seq = seq + 1 if seq != 0xFFFFFFFF else 1
            ops += 1
        if time.perf_counter() >= deadline:
            break
    dt = time.perf_counter() - t0
    return dt * 1e6 / ops, ops
