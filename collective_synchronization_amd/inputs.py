"""Seeded synthetic workloads for the all-reduce (tests and bench).

This module only draws numbers: it holds none of the all-reduce arithmetic.
Payload values are drawn in binary32 with numpy's PCG64 generator and
converted to bf16 bit patterns by torch's CPU float->bfloat16 conversion (a
library routine, round to nearest even).  Decode-time activations of the
tensor-parallel models the pages discuss are the stand-in: normal(0, 1) or
uniform[-1, 1) rows of the hidden size, one row per token.
"""
from __future__ import annotations

import hashlib

import numpy as np


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    import torch
    f = np.ascontiguousarray(f, dtype=np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def payload(seed: int, shape, dist: str = "normal") -> np.ndarray:
    """bf16 bit patterns (uint16) of the given shape: 'normal' N(0,1) or
    'uniform' U[-1,1), drawn in binary32."""
    rng = _rng(seed)
    shape = tuple(int(s) for s in shape)
    if dist == "normal":
        f = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "uniform":
        f = (2 * rng.random(shape, dtype=np.float32) - 1).astype(np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return f32_to_bf16_bits(f)


def weights(seed: int, layers: int, nranks: int, count: int) -> np.ndarray:
    """bf16 bit patterns [layers, nranks, count, count // nranks] of
    row-parallel linear layers: N(0, 1/count) in binary32 (random
    initialisation at the hidden size, so a chain of layers keeps its scale);
    [l, r, j] is output j's row over rank r's input slice."""
    kr = count // nranks
    if layers * nranks * count * kr > (1 << 32):
        raise ValueError(f"{layers} layers of a hidden size of {count} need more than "
                         "8 GiB of weights")
    rng = _rng(seed)
    out = np.empty((layers, nranks, count, kr), dtype=np.uint16)
    scale = np.float32(1.0 / np.sqrt(count))
    for l in range(layers):
        f = rng.standard_normal((nranks, count, kr), dtype=np.float32) * scale
        out[l] = f32_to_bf16_bits(f)
    return out


def inject(x: np.ndarray, seed: int, rate: float,
           values=(0xFFFF, 0xFFC0, 0xFF81)) -> np.ndarray:
    """Copy of x with a `rate` fraction of positions replaced by `values`
    (negative NaNs by default, which the sentinel protocol must never send)."""
    rng = _rng(seed)
    y = np.array(x, dtype=np.uint16, copy=True)
    flat = y.reshape(-1)
    k = max(1, int(round(flat.size * rate)))
    idx = rng.choice(flat.size, size=k, replace=False)
    flat[idx] = rng.choice(np.asarray(values, dtype=np.uint16), size=k)
    return y


def delays_us(seed: int, nops: int, nranks: int, max_us: float = 20.0) -> np.ndarray:
    """Per (op, producer) start delay, continuous U[0, max_us) microseconds."""
    return _rng(seed).random((nops, nranks)) * max_us


def tile_orders(seed: int, nops: int, nranks: int, tiles_per_wave: int) -> np.ndarray:
    """Per (op, producer) permutation of 0..tiles_per_wave-1 (uint16)."""
    rng = _rng(seed)
    out = np.empty((nops, nranks, tiles_per_wave), dtype=np.uint16)
    for i in range(nops):
        for r in range(nranks):
            out[i, r] = rng.permutation(tiles_per_wave)
    return out


def arrival_perms(seed: int, nops: int, nranks: int) -> np.ndarray:
    rng = _rng(seed)
    return np.stack([rng.permutation(nranks) for _ in range(nops)]).astype(np.int32)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
