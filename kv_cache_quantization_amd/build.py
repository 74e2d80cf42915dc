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

COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-result",
    # each kernel unit leaves out the file-local helpers the other units use
    "-Wno-unneeded-internal-declaration",
    # no packed fp32 VALU instructions (v_pk_add/mul/fma_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the kernels read every accumulator with VALU code
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]
# compile units, built in parallel: the kernel file in six parts (see PQ_UNIT in it) and the C ABI
UNITS = [("pq_kernels.hip", ["-DPQ_UNIT=%d" % u], "kernels_%d.o" % u) for u in range(6)] + [("pq_api.cpp", [], "api.o")]
NOISE = "is not a recognized feature for this target"


def _errors(stderr):
    return "\n".join(l for l in stderr.splitlines() if NOISE not in l)


def build(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    procs = []
    for src, extra, obj in UNITS:
        # hipcc treats .cpp as host C++ unless told otherwise; every unit compiles as HIP
        cmd = [hipcc] + COMMON_FLAGS + extra + ["-c", "-x", "hip", os.path.join(CSRC, src),
                                                "-o", os.path.join(obj_dir, obj)]
        if verbose:
            print(" ".join(cmd))
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    failed = []
    for (src, extra, _), p in zip(UNITS, procs):
        _, err = p.communicate()
        err = _errors(err)
        if p.returncode != 0:
            failed.append("%s %s:\n%s" % (src, " ".join(extra), err))
        elif err.strip() and verbose:
            print(err)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + [os.path.join(obj_dir, o) for _, _, o in UNITS] + \
        ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + _errors(res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
