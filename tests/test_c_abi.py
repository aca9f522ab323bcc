"""The host half of the C ABI used from a plain C99 program (tests/c/host_plan.c):
compiled with gcc against include/tg.h alone and linked to libtg.so, it
plans a hand-worked batch and checks every table value.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "non_uniform_paged_amd")


def test_host_abi_from_plain_c(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(LIBDIR, "libtg.so")):
        pytest.skip("libtg.so not built")
    exe = tmp_path / "host_plan"
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "host_plan.c"), "-L", LIBDIR, "-ltg",
                    f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
