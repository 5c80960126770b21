"""Host-compiled checks: the 32-bit modular-arithmetic core against 128-bit integer arithmetic, the
matrix-core conversion tables against conversion sums recomputed from the primes, and the library's
host half (tables and argument checks) built with AddressSanitizer and UndefinedBehaviorSanitizer."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_modarith_core_on_host(tmp_path):
    exe = tmp_path / "modarith_check"
    src = os.path.join(HERE, "native", "modarith_check.cpp")
    subprocess.run(["hipcc", "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", src, "-o", str(exe)], check=True,
                   capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_matrix_core_conversion_tables_on_host(tmp_path):
    # the library's operand tables for the int8 matrix-core conversion, emulated in the
    # instruction's lane layout, against conversion sums recomputed from the primes
    exe = tmp_path / "mx_tables_check"
    src = os.path.join(HERE, "native", "mx_tables_check.cpp")
    inc = os.path.join(HERE, "..", "include")
    subprocess.run(["hipcc", "-O2", "-std=c++17", "-I", inc, src, "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


# The library's host half under AddressSanitizer and UndefinedBehaviorSanitizer: the
# table builds and every argument check reached through the C-ABI, and the matrix-core
# table emulation.  The sanitizers instrument host code only (each flag follows
# -Xarch_host); these programs contain no device code.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
@pytest.mark.parametrize("name", ["abi_host_check", "mx_tables_check"])
def test_host_half_under_sanitizers(tmp_path, name):
    exe = tmp_path / name
    src = os.path.join(HERE, "native", name + ".cpp")
    inc = os.path.join(HERE, "..", "include")
    subprocess.run(["hipcc", "-O1", "-g", "-std=c++17", "-I", inc] + SANITIZE + [src, "-o", str(exe)], check=True,
                   capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr, r.stderr
