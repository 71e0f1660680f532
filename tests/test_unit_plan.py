"""The attention launch's work split, checked on the host: builds tests/unit_plan_check.hip
with hipcc (host code only runs) and runs it over random request layouts."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_unit_planners_cover_every_row_once(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "unit_plan_check")
    build = subprocess.run(
        [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
         "-Wno-unused-function", "-Wno-unneeded-internal-declaration",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", exe, os.path.join(HERE, "unit_plan_check.hip"),
         os.path.join(ROOT, "pass_typed_decision_amd", "csrc", "blink_host.cpp")],
        capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "two requests: 120 units, full 56 40, small 384 256" in run.stdout
    assert "ok: 100000 layouts each" in run.stdout
