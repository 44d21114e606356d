"""Host check of the division by launch constants that the kernels use to
split workgroup and row indices (FastDiv in csrc/mgqa_internal.h): the
multiply-high form must give the exact quotient for every numerator below
2^31.  Compiles tests/fastdiv_check.cpp with the host compiler and runs it."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "masked_gqa_attention_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_fastdiv_exact(tmp_path):
    exe = tmp_path / "fastdiv_check"
    subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", os.path.join(HERE, "fastdiv_check.cpp"),
                    "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 wrong" in r.stdout
