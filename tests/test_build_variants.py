"""Builds that the CPU suite compiles (hipcc cross-compiles for gfx950 here)
but does not run:

* a translation unit outside the package that includes only the public
  device header include/ar_dev.h (a producer kernel that sends from its
  epilogue and a consumer kernel that receives and reduces): the header is
  self-contained;
* the library built with AR_FORMAL_FENCES=1, where every ordering point is
  the memory model's agent-scope release or acquire fence instead of a wait
  for the wave's own accesses: it compiles, links and exports every function
  include/ar.h declares, so that build cannot rot unnoticed.
"""
import os
import re
import shutil
import subprocess

import pytest

from conftest import ROOT

INCLUDE = os.path.join(ROOT, "include")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fno-gpu-flush-denormals-to-zero",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

DEV_TU = r'''
#include "ar_dev.h"

// a producer that scales its payload and sends it from the epilogue
__global__ void produce(ar_dev::buffer b, const uint16_t* in, int rank) {
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x;
  int64_t first;
  int n;
  ar_dev::lane_elements<AR_SENTINEL>(tile, lane, &first, &n);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int k = 0; k < n && first + k < b.count; ++k) {
    const uint32_t h = in[first + k];
    w[k >> 1] |= (k & 1) ? (h << 16) : h;
  }
  ar_dev::broadcast<AR_SENTINEL>(b, rank, tile, lane, w);
}

// a consumer that receives every rank's tile and reduces it in rank order
__global__ void consume(ar_dev::buffer b, int c, int* ctrl, uint16_t* out) {
  const int lane = threadIdx.x & 63;
  ar_dev::recv_reduce<AR_SENTINEL, 8>(b, c, blockIdx.x, lane, true, ctrl, 1000000ull, out);
}
'''


def _hipcc():
    exe = shutil.which("hipcc")
    if not exe:
        pytest.skip("hipcc is not installed")
    return exe


def test_public_device_header_is_self_contained(tmp_path):
    src = tmp_path / "uses_ar_dev.hip"
    src.write_text(DEV_TU)
    r = subprocess.run([_hipcc(), *FLAGS, "-I", INCLUDE, "-c", "-o",
                        str(tmp_path / "uses_ar_dev.o"), str(src)],
                       capture_output=True, text=True, timeout=600, cwd=str(tmp_path))
    assert r.returncode == 0, r.stderr[-3000:]
    # only include/ is on the path: nothing under the package was needed
    text = open(os.path.join(INCLUDE, "ar_dev.h")).read() + \
        open(os.path.join(INCLUDE, "ar_protocols.h")).read() + \
        open(os.path.join(INCLUDE, "ar_device.h")).read()
    assert "collective_synchronization_amd" not in text


def test_formal_fence_build_links_and_exports(tmp_path):
    _hipcc()
    from collective_synchronization_amd.csrc import build as hip_build
    out = str(tmp_path / "libcsync_ar_formal.so")
    hip_build.build(out=out, defines=("AR_FORMAL_FENCES=1",))
    nm = subprocess.run(["nm", "-D", "--defined-only", out], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r"\b(ar_[a-z0-9_]+)\b", nm))
    header = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, "ar.h")).read(), flags=re.S)
    declared = set(re.findall(r"\b(ar_[a-z0-9_]+)\s*\(", header))
    assert declared and declared <= exported, sorted(declared - exported)
