"""The staging loads' buffer offsets (csrc/offsets.h, the arithmetic the
kernels call) checked on the host: tests/offsets_check.cpp enumerates every
load of every tile config on tail shapes and asserts that each access that
passes the buffer range check lies inside its row and its buffer, that the
FP8 tiles land in LDS where the fragment reads look for them, and that those
reads are free of bank conflicts under gfx950's lane grouping."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_staging_offsets_stay_in_bounds():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "offsets_check")
        subprocess.run(["g++", "-O1", "-std=c++17", "-Wall",
                        "-I", os.path.join(ROOT, "fp4_grouped_gemm_amd", "csrc"),
                        os.path.join(ROOT, "tests", "offsets_check.cpp"), "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert " 0 failed" in r.stdout
