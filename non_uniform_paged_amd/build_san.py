"""Sanitizer build of ``libtg.so`` for the CPU tests (AddressSanitizer and
UndefinedBehaviorSanitizer on the host code).

    python -m non_uniform_paged_amd.build_san

Host code -- the C++ planner and the argument checks of every device entry
point -- is instrumented; device code is compiled unoptimised and is never
run (the tests that load this build only call entry points that return
before any launch).  The result goes to ``_build/san/libtg.so`` and is loaded
instead of the ordinary build when ``TG_LIB_PATH`` names it, with the
sanitizer runtime preloaded (``runtime()``).
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from .build import ARCH, CSRC, CXX_SOURCES, HIP_SOURCES, INCLUDE, ROOT

OUT_DIR = os.path.join(ROOT, "_build", "san")
LIB = os.path.join(OUT_DIR, "libtg.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
HIP_COMPILER = os.path.join(ROCM, "bin", "hipcc")

SAN = ["address", "undefined"]
HOST_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", "-I", INCLUDE,
              "-fno-sanitize-recover=undefined"] + [f"-fsanitize={s}" for s in SAN]
# the sanitizer options apply to the host pass only (each behind -Xarch_host)
HIP_HOST_SAN = []
for _flag in [f"-fsanitize={s}" for s in SAN] + ["-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]:
    HIP_HOST_SAN += ["-Xarch_host", _flag]
HIP_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
             "-Xarch_device", "-O0", "-Xarch_device", "-g0"] + HIP_HOST_SAN


def runtime() -> str:
    """Path of the sanitizer runtime to preload into an uninstrumented
    interpreter that loads this build."""
    found = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise FileNotFoundError("clang AddressSanitizer runtime not found under " + ROCM)
    return found[-1]


def _stamp() -> str:
    h = hashlib.sha256()
    for src in sorted(os.listdir(CSRC)) + ["tg.h"]:
        path = os.path.join(CSRC if src != "tg.h" else INCLUDE, src)
        with open(path, "rb") as f:
            h.update(src.encode() + f.read())
    h.update(" ".join(HOST_FLAGS + HIP_FLAGS).encode())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    """Build the sanitized library unless an up-to-date one exists; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    stamp_path = os.path.join(OUT_DIR, "stamp")
    stamp = _stamp()
    if os.path.exists(LIB) and os.path.exists(stamp_path) and open(stamp_path).read() == stamp:
        return LIB
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        jobs.append([HIP_COMPILER, *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        jobs.append([CLANG, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stderr)
            raise subprocess.CalledProcessError(r.returncode, cmd)
        return cmd[-1]

    with ThreadPoolExecutor(max_workers=max(1, min(len(jobs), os.cpu_count() or 1, 8))) as ex:
        objs = list(ex.map(run, jobs))
    tmp = LIB + ".tmp"
    run([CLANG, "-shared", "-shared-libsan", *[f"-fsanitize={s}" for s in SAN], *objs,
         "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", tmp])
    os.replace(tmp, LIB)
    with open(stamp_path, "w") as f:
        f.write(stamp)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
