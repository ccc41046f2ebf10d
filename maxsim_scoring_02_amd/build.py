"""Build liblik.so (the C-ABI MaxSim library) for gfx950 with hipcc.

    python -m maxsim_scoring_02_amd.build

Compiles every .hip file under csrc/ to an object in _build/ (in parallel)
and links them into maxsim_scoring_02_amd/liblik.so, in-tree, so the library
travels with the source tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblik.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep hand-written float code off packed-FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the epilogue reads them with plain VALU ops
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblik.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return r.returncode, "\n".join(lines)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = []
    for f in srcs:
        obj = os.path.join(BUILD, f[:-4] + ".o")
        jobs.append([cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, f), "-o", obj])
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_run, jobs))
    for (rc, out), cmd in zip(results, jobs):
        if verbose or rc != 0:
            if out.strip():
                print(out, file=sys.stderr)
        if rc != 0:
            raise RuntimeError(f"hipcc failed: {' '.join(cmd)}")
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link of liblik.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
