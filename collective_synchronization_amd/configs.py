"""The five workloads of the all-reduce path (sizes of TP decode steps).

Shapes follow decode-time activations: one [B, H] bf16 tensor per rank per
all-reduce, two all-reduces per transformer layer (after attention and after
the MLP), so 32 layers give 64 back-to-back ops and 80 layers give 160.
"""
from __future__ import annotations

KIB = 1024
MIB = 1024 * 1024

CONFIGS = {
    "n4_ll_1x4096": dict(name="n4_ll_1x4096", nranks=4, batches=(1,), hidden=4096,
            dist="normal", protos=("ll",), nops=1, seed=1001),
    "n8_sentinel_1x4096_64ops": dict(name="n8_sentinel_1x4096_64ops", nranks=8, batches=(1,), hidden=4096,
            dist="normal", protos=("sentinel",), nops=64, seed=1002),
    "n4_ll128_Bx8192_160ops": dict(name="n4_ll128_Bx8192_160ops", nranks=4, batches=(1, 4, 16), hidden=8192,
            dist="normal", protos=("ll128",), nops=160, seed=1003),
    "n8_sweep_2KiB_4MiB": dict(name="n8_sweep_2KiB_4MiB", nranks=8,
            sizes=tuple(2 ** k for k in range(11, 23)),   # payload bytes per rank
            dist="uniform", protos=("ll", "ll128", "sentinel", "barrier"), nops=64,
            seed=1004),
    "n16_skew_8x4096_64ops": dict(name="n16_skew_8x4096_64ops", nranks=16, batches=(8,), hidden=4096,
            dist="normal", protos=("ll", "ll128", "sentinel"), nops=64, seed=1005,
            delay_max_us=20.0, shuffle=True),
}
