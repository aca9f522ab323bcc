"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The sanitizer build of the library (``non_uniform_paged_amd.build_san``)
runs the host-side tests -- planner bit-exactness against the integer oracle,
the table check, the argument checks of the device entry points -- in a
child interpreter with the sanitizer runtime preloaded, and the plain C99
program of ``tests/c/host_plan.c`` linked against it.  Any report (an
out-of-bounds access, a use after free, signed overflow, a misaligned or
null access) fails the test.  A planted out-of-bounds read first shows that
the toolchain reports at all."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_host_parity.py", "tests/test_table_check.py", "tests/test_abi_errors.py"]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _env(lib):
    from non_uniform_paged_amd import build_san
    env = dict(os.environ)
    env.update(LD_PRELOAD=build_san.runtime(), TG_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


@pytest.fixture(scope="module")
def san_lib():
    if not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no ROCm toolchain")
    from non_uniform_paged_amd import build_san
    return build_san.build()


def test_sanitizer_reports_a_planted_overflow(tmp_path):
    from non_uniform_paged_amd import build_san
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\nint main(int c, char** v) { (void)v; int* p = malloc(4 * sizeof(int));"
                   " int x = p[c + 3]; free(p); return x == 12345; }\n")
    exe = tmp_path / "oob"
    subprocess.run([build_san.CLANG, "-x", "c", "-g", "-fsanitize=address", str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_host_tests_clean_under_sanitizers(san_lib):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *HOST_TESTS],
                       cwd=ROOT, env=_env(san_lib), capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for rep in REPORTS:
        assert rep not in out, out[-4000:]
    assert " passed" in out


def test_c_program_clean_under_sanitizers(san_lib, tmp_path):
    from non_uniform_paged_amd import build_san
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "host_plan"
    libdir = os.path.dirname(san_lib)
    subprocess.run([build_san.CLANG, "-x", "c", "-std=c99", "-g", "-fsanitize=address,undefined", "-shared-libsan",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "host_plan.c"),
                    "-L", libdir, "-ltg", f"-Wl,-rpath,{libdir}",
                    f"-Wl,-rpath,{os.path.dirname(build_san.runtime())}", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    env = _env(san_lib)
    env.pop("LD_PRELOAD")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    for rep in REPORTS:
        assert rep not in r.stderr, r.stderr
