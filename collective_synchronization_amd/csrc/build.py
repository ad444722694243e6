"""Build the HIP library libcsync_ar.so for gfx950 (in-tree).

hipcc cross-compiles for gfx950 without a GPU.  Flags:
  -fno-gpu-flush-denormals-to-zero  keep binary32 denormals in the reduction
  -ffp-contract=off                 no fused or reassociated arithmetic
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                    no packed fp32 instructions
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
LIB = os.path.join(PKG, "libcsync_ar.so")
SOURCES = [os.path.join(HERE, "ar_kernels.hip"), os.path.join(HERE, "ar_collectives.hip"),
           os.path.join(HERE, "ar_select.cpp")]
HEADERS = [os.path.join(HERE, "ar_device.h"), os.path.join(HERE, "ar_protocols.h"),
           os.path.join(HERE, "ar_host.h"),
           os.path.join(os.path.dirname(PKG), "include", "ar.h")]
ARCH = os.environ.get("AR_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def device_asm(out_path: str) -> str:
    """Write the gfx950 assembly of ar_kernels.hip (for inspection)."""
    cmd = ["hipcc", *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "-S",
           "--cuda-device-only", "-o", out_path, SOURCES[0]]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
