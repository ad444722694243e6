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
           os.path.join(HERE, "ar_static.hip"), os.path.join(HERE, "ar_state.hip"),
           os.path.join(HERE, "ar_linear.hip"),
           os.path.join(HERE, "ar_select.cpp")]
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
HEADERS = [os.path.join(INCLUDE, "ar_device.h"), os.path.join(INCLUDE, "ar_protocols.h"),
           os.path.join(HERE, "ar_host.h"), os.path.join(INCLUDE, "ar.h"),
           os.path.join(INCLUDE, "ar_dev.h")]
ARCH = os.environ.get("AR_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(proc):
    _, stderr = proc.communicate()
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    return err


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile the sources in parallel (one object each), then link `out`.
    `defines`: extra -D options (a variant build, e.g. AR_FORMAL_FENCES=1)."""
    tag = os.path.splitext(os.path.basename(out))[0]
    objdir = os.path.join(PKG, "_build", tag)
    os.makedirs(objdir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    cflags = [f for f in FLAGS if f != "-shared"]
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        procs.append(_run(["hipcc", *cflags, *dflags, "-c", "-o", obj, src], verbose))
    errs = [_finish(p) for p in procs]
    tmp = out + ".tmp"
    errs.append(_finish(_run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC",
                              "-o", tmp, *objs], verbose)))
    err = "\n".join(e for e in errs if e.strip())
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def device_asm(out_path: str) -> str:
    """Write the gfx950 assembly of ar_kernels.hip (for inspection)."""
    cmd = ["hipcc", *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "-S",
           "--cuda-device-only", "-o", out_path, SOURCES[0]]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
