"""The copy maps of the single-launch batch-1 denoise (persist_plan.h), checked on the host:
every piece a workgroup copies into its LDS lies inside its weight matrix or cache block, fills
the LDS slot the kernel reads it from exactly once, and the 32 workgroups of a group together
copy exactly the rows their group owns (CPU only: g++ builds tests/persist_plan_check.cpp)."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT


def test_copy_maps_are_in_bounds_and_complete(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "persist_plan_check"
    subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Werror",
                    "-I" + os.path.join(ROOT, "dual_expert_merged_amd", "csrc"),
                    os.path.join(ROOT, "tests", "persist_plan_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    assert "all copy maps consistent" in r.stdout
