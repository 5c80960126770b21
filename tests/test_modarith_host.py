"""The library's 32-bit modular-arithmetic core, compiled for the host, against 128-bit integer arithmetic."""
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
