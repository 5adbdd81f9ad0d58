"""CPU proof of the kernels' exact division steps (aclnnDynamicQuantV2,
Formula: "/" is a correctly rounded binary32 division).

Compiles the kernels' own division header (csrc/dq_div.h) on the host
together with tests/division_check.cpp and runs it:
  - div_by_const against IEEE division for every binary32 in
    [2^-100, FLT_MAX] and each constant divisor 7, 15, 127, 255;
  - div_by_row (correctly rounded reciprocal + one fma correction) against
    IEEE division on 1.2e8 pairs, divisors with all-ones and near-all-ones
    mantissas and the 2^-60 / 2^60 edges, quotients placed around k + 1/2;
  - div_magic / div_by against integer division below 2^31.
No GPU is used.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "int4_quantization_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc (host compiler with the HIP headers) not found")
def test_division_steps_match_ieee(tmp_path):
    exe = tmp_path / "division_check"
    subprocess.run([HIPCC, "-O2", "-mfma", "-ffp-contract=off", "-std=c++17", "-pthread", f"-I{CSRC}",
                    os.path.join(HERE, "division_check.cpp"), "-o", str(exe)], check=True,
                   capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    assert len(lines) == 3 and all(" 0 mismatches" in ln for ln in lines), r.stdout
