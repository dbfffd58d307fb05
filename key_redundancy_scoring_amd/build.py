"""Build libtwinkv.so for gfx950 in-tree with hipcc.

    python -m key_redundancy_scoring_amd.build

Every HIP source under csrc/ is compiled to an object in csrc/_build/ (in
parallel) and linked into key_redundancy_scoring_amd/libtwinkv.so.  Packed
fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(CSRC, "_build")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libtwinkv.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "norms.hip", "gram.hip", "tri.hip", "resolve.hip", "select.hip", "repair.hip", "gather.hip", "alloc.hip", "stats.hip"]

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


# Gram sweep: MFMA results go straight to VGPRs, where the epilogue reads them,
# instead of AGPRs that would need a copy per accumulator; its inputs are finite
# (no NaN), so max trees need no NaN-quieting copies (infinities stay honoured).
PER_SOURCE = {"gram.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
              "tri.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"]}


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libtwinkv.so")
    return exe


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int | None = None, defines: dict | None = None, out: str | None = None) -> str:
    """Compile and link the library; ``defines`` adds -D macros (tile shapes),
    ``out`` writes the library somewhere other than the package directory."""
    hipcc = _hipcc()
    lib = out or LIB
    bdir = BUILD_DIR if out is None else os.path.join(os.path.dirname(os.path.abspath(out)), "_build")
    os.makedirs(bdir, exist_ok=True)
    dflags = [f"-D{k}={v}" for k, v in (defines or {}).items()]
    objs = []
    cmds = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(bdir, s.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *COMMON, *PER_SOURCE.get(s, []), *dflags, "-c", src, "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        for cmd, err in zip(cmds, ex.map(_run, cmds)):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    tmp = lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
