"""CPU proof of the decode matmul's one-FMA dequantization with offset
(aclnnWeightQuantMatmulAllReduce, API function; the weight formula read
with the AntiQuantize arithmetic: W = RN(RN(code + o) * s) in binary32).

Compiles the kernel's own predicate header (csrc/wq_fma.h) on the host with
tests/fma_dequant_check.cpp and runs it for int4 and int8 codes under bf16
and fp16 parameters: every finite o of T against scales at a stride through
all of T, and every finite s against offsets at a stride.  Where
wq_fma_exact accepts (o, s), fma(code, s, RN(o * s)) must equal the
formula's two roundings bit for bit for every code (a zero may change
sign).  Halving the offset floor must produce mismatches, so the floors are
where the form stops being exact, and the check can see a failure.
No GPU is used.
"""
import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "int4_quantization_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc (host compiler with the HIP headers) not found")
    exe = tmp_path_factory.mktemp("fma") / "fma_dequant_check"
    subprocess.run([HIPCC, "-O2", "-mfma", "-ffp-contract=off", "-std=c++17", "-pthread", f"-I{CSRC}",
                    os.path.join(HERE, "fma_dequant_check.cpp"), "-o", str(exe)], check=True,
                   capture_output=True, text=True)
    return str(exe)


def run(checker, width, t, floor_scale):
    r = subprocess.run([checker, width, t, floor_scale], capture_output=True, text=True, timeout=300)
    m = re.fullmatch(r"(\d+) accepted, (\d+) mismatches\s*", r.stdout)
    assert m, r.stdout + r.stderr
    return r.returncode, int(m.group(1)), int(m.group(2)), r.stderr


@pytest.mark.parametrize("width", ["int4", "int8"])
@pytest.mark.parametrize("t", ["bf16", "fp16"])
def test_fma_form_exact_where_accepted(checker, width, t):
    rc, accepted, mismatches, err = run(checker, width, t, "1")
    print(f"{width} {t}: {accepted} accepted pairs, {mismatches} mismatches")
    assert rc == 0 and mismatches == 0, err
    assert accepted > 1_000_000


@pytest.mark.parametrize("width", ["int4", "int8"])
@pytest.mark.parametrize("t", ["bf16", "fp16"])
def test_fma_form_floor_is_needed(checker, width, t):
    rc, accepted, mismatches, _ = run(checker, width, t, "0.5")
    print(f"{width} {t}, floor halved: {mismatches} mismatches of {accepted}")
    assert rc == 1 and mismatches > 0
