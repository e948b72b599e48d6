"""Compile the HIP library libw4g.so for gfx950, in-tree, next to this file.

Usage: python -m w4_gemv_greedy_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4g.so")
SOURCES = ["gemv.hip", "gemv_mfma.hip", "gemm.hip", "argmax.hip", "abi.hip"]
# measurement kernels (HBM read and matrix-core ceilings), a library of their own
# that only the benchmark loads
CEILING_LIB = os.path.join(HERE, "libw4g_ceiling.so")
CEILING_SOURCE = "ceiling.hip"
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
# per-source extras: the prompt GEMM keeps its matrix-core results in VGPRs, where
# the fp32 scale FMA reads them (AGPR results would be copied every group)
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    return r.returncode, msgs


def build(quiet=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src in SOURCES + [CEILING_SOURCE]:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        jobs.append((obj, [hipcc] + FLAGS + EXTRA.get(src, []) +
                     ["-c", os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    out = []
    for (obj, _), (rc, msgs) in zip(jobs, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) on {os.path.basename(obj)}:\n{msgs}")
        if msgs.strip():
            out.append(msgs)
    for lib, objs in ((LIB, [j[0] for j in jobs[:len(SOURCES)]]), (CEILING_LIB, [jobs[-1][0]])):
        tmp = lib + ".tmp"
        rc, msgs = _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp])
        if rc != 0:
            raise RuntimeError(f"link of {os.path.basename(lib)} failed ({rc}):\n{msgs}")
        os.replace(tmp, lib)
    if out and not quiet:
        print("\n".join(out), file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build())
