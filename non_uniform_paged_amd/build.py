"""Build ``libtg.so`` in-tree with hipcc for gfx950.

    python -m non_uniform_paged_amd.build

The HIP sources are compiled with packed-fp32 instructions disabled and IEEE
fp32 division/sqrt; the host planner is plain C++17.  Objects go to
``_build/`` at the repository root; the shared library is written next to
this file.
"""
from __future__ import annotations

import os
import shlex
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtg.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-Wno-unused-command-line-argument",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-Wall", "-Wextra"]

HIP_SOURCES = ["tg_decode.hip", "tg_split.hip", "tg_kvwrite.hip", "tg_bench.hip", "tg_zip.hip"]
CXX_SOURCES = ["tg_host.cpp"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    subprocess.run(cmd, check=True)


def _run_checking_scratch(cmd, verbose):
    """Compile with resource-usage remarks and refuse kernels that spill to
    scratch memory: every kernel here is meant to live in registers and LDS
    (a spill, or a by-value kernel-argument struct copied to scratch, costs
    a large share of the streaming rate)."""
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    r = subprocess.run([*cmd, "-Rpass-analysis=kernel-resource-usage"], capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    name, bad = None, []
    for line in r.stderr.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].strip()
        elif "ScratchSize [bytes/lane]:" in line:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if size > 0:
                bad.append(f"{name}: {size} bytes/lane")
    if bad:
        raise RuntimeError("kernels use scratch memory:\n  " + "\n  ".join(bad))


def build(verbose: bool = False) -> str:
    """Compile every source (the translation units in parallel) and link
    ``libtg.so``; returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append((_run_checking_scratch,
                     [HIPCC, *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append((_run, ["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futures = [ex.submit(fn, cmd, verbose) for fn, cmd, _ in jobs]
        for f in futures:
            f.result()
    objs = [obj for _, _, obj in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
