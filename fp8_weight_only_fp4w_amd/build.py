"""Build libfp4w.so in-tree: hipcc for the gfx950 kernels, g++ for the host
dispatch, hipcc -shared for the link; and libhbmprobe.so, the bench's HBM
read-stream probe.

    python -m fp8_weight_only_fp4w_amd.build [-v]
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp4w.so")
PROBE_LIB = os.path.join(HERE, "libhbmprobe.so")
MFMA_PROBE_LIB = os.path.join(HERE, "libmfmaprobe.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-fno-gpu-rdc",
    # no implicit FMA contraction: every fused multiply-add is an explicit fmaf
    "-ffp-contract=off",
    # packed FP32 instructions off: the compiler emits only plain FP32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first kernel arguments arrive preloaded in scalar registers, so a
    # short kernel's waves start without a memory round trip for them (the
    # decode GEMV: about 0.1 us of 6.9 per call)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        line for line in (r.stdout + r.stderr).splitlines()
        if "is not a recognized feature for this target" not in line
    )
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libfp4w.so; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    hip, cpp = _sources()
    cmds, objs = [], []
    for f in hip:
        obj = os.path.join(BUILD_DIR, f + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, f), "-o", obj])
        objs.append(obj)
    cxx = shutil.which("g++") or "g++"
    for f in cpp:
        obj = os.path.join(BUILD_DIR, f + ".o")
        cmds.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, f), "-o", obj])
        objs.append(obj)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    # the bench's HBM read-stream probe, a library of its own
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", os.path.join(HERE, "probe", "hbm_read.hip"), "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    # the bench's MFMA-rate probe, a library of its own
    tmp = MFMA_PROBE_LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", os.path.join(HERE, "probe", "mfma_peak.hip"), "-o", tmp], verbose)
    os.replace(tmp, MFMA_PROBE_LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
