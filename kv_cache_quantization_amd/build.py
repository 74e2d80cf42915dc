"""Build the HIP library in-tree: kv_cache_quantization_amd/libpqhip.so for gfx950.

Run as ``python kv_cache_quantization_amd/build.py`` (or through
``__graft_entry__.build()``); importing the package first would load the library
being rebuilt.  hipcc cross-compiles for gfx950 without a GPU.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpqhip.so")
SOURCES = ["pq_kernels.hip", "pq_api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    # no packed fp32 VALU instructions (v_pk_add/mul/fma_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the kernels read every accumulator with VALU code
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        # hipcc treats .cpp as host C++ unless told otherwise; compile both as HIP
        srcs += ["-x", "hip", p]
    tmp = LIB + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
