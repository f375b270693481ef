"""Launch-time integer division of the forward kernel's work-item mapping
(`exact_io_aware_07_amd/csrc/attn_udiv.h`), checked on the host: the header is
plain C++, so g++ compiles the same functions the kernel uses and
`tests/udiv_check.cpp` compares them with `/` over exhaustive small ranges,
powers of two and a random sample up to 2^31."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_udiv_matches_division(tmp_path):
    exe = tmp_path / "udiv_check"
    src = os.path.join(ROOT, "tests", "udiv_check.cpp")
    inc = os.path.join(ROOT, "exact_io_aware_07_amd", "csrc")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", f"-I{inc}", src, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0" in r.stdout
