"""The 64-bit address split/join used by the kernels' scalar-based copies (addr_words.h),
checked on the host with addresses whose low word is >= 2^31 (CPU only: g++ builds
tests/addr_words_check.cpp).  The GPU side of the same case is in tests/test_gpu_tiny.py."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT


def test_address_words_round_trip_through_int(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "addr_words_check"
    subprocess.run([gxx, "-std=c++17", "-O1", "-Wall", "-Werror",
                    "-I" + os.path.join(ROOT, "dual_expert_merged_amd", "csrc"),
                    os.path.join(ROOT, "tests", "addr_words_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
