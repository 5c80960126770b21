"""Host-compiled checks: the 32-bit modular-arithmetic core against 128-bit integer arithmetic, and the
matrix-core conversion tables against conversion sums recomputed from the primes."""
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
