"""Host build of the selection row geometry (csrc/select_geom.h), checked in
every mode against a form written with early returns, with range checks on
the candidates and positions it produces (tests/host/row_geom_check.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc missing")
def test_row_geometry_host(tmp_path):
    exe = str(tmp_path / "row_geom_check")
    cmd = [HIPCC, "-std=c++17", "-O1", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "long_context_sparse_lsa_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "row_geom_check.cpp"), "-o", exe]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
