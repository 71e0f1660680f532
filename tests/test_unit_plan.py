"""The attention launch's work split, checked on the host: builds tests/unit_plan_check.hip
with hipcc (host code only runs) and runs it over random request layouts (row re-cut, grouped
split, key split of the last round); then checks that the tests' restatement of the split
(helpers.attention_units and attention_split, which place the per-unit parity samples) matches
the launcher's own planners."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from helpers import attention_split, attention_units

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("plan") / "unit_plan_check")
    build = subprocess.run(
        [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
         "-Wno-unused-function", "-Wno-unneeded-internal-declaration",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", exe, os.path.join(HERE, "unit_plan_check.hip"),
         os.path.join(ROOT, "pass_typed_decision_amd", "csrc", "blink_attention_plain.hip"),
         os.path.join(ROOT, "pass_typed_decision_amd", "csrc", "blink_host.cpp")],
        capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    return exe


def test_unit_planners_cover_every_row_once(checker):
    run = subprocess.run([checker], capture_output=True, text=True, timeout=300)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "two requests: 120 units, full 56 40, small 384 256" in run.stdout
    assert "ok: 100000 layouts each" in run.stdout
    assert "27B-like split: full 128, split 14, ways 2, tiles 512" in run.stdout


def test_sample_plan_matches_launcher(checker):
    rng = np.random.default_rng(7)
    # The five workloads' rows per KV head (seeded tails; 4B-like 5338 x 4, long document
    # 21113 x 4, plain max packing 74300 x 4, 27B-like 10443 x 5), then random sizes.
    cases = [(5338 * 4, 8, 256, 2048), (21113 * 4, 8, 256, 18432), (74300 * 4, 8, 256, 0),
             (10443 * 5, 8, 256, 65536), (139 * 4, 1, 256, 256)]
    for _ in range(3000):
        cases.append((int(rng.integers(1, [64, 2000, 30000, 400000][rng.integers(4)])),
                      int(1 << rng.integers(4)), int(256 if rng.integers(3) == 0 else
                                                     rng.integers(1, 300)),
                      int(rng.integers(0, 70000))))
    stdin = "".join(f"{r} {h} {c} {p}\n" for r, h, c, p in cases)
    run = subprocess.run([checker, "plan"], input=stdin, capture_output=True, text=True,
                         timeout=300)
    assert run.returncode == 0, run.stderr
    lines = run.stdout.split("\n")
    for (rows, hkv, cus, prefix), line in zip(cases, lines):
        units, full, small, s_full, s_left, ways, tiles = (int(x) for x in line.split())
        split = attention_split(rows, hkv, cus, prefix)
        assert split == ((s_full, s_left, ways, tiles) if ways else None), (rows, hkv, cus, prefix)
        if split:  # the key split keeps whole 384-row units
            assert attention_units(rows, hkv, cus, prefix, True) == [
                (i * 384, min(rows, (i + 1) * 384)) for i in range(s_full + s_left)]
        plan = attention_units(rows, hkv, cus)
        assert len(plan) == units, (rows, hkv, cus)
        sizes = [b - a for a, b in plan]
        # Every unit but the last is whole: 384 rows up to `full`, then `small` rows each.
        assert all(s == (384 if k < full else small) for k, s in enumerate(sizes[:-1])), \
            (rows, hkv, cus)
        assert 0 < sizes[-1] <= (384 if units <= full else small), (rows, hkv, cus)
        assert plan[-1][1] == rows
