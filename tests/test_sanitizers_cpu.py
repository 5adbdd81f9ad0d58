"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code.

Builds, with the host compilers only (no GPU code):
  - the oracle (oracle/dquant_oracle.c), and
  - the library's validation and planning layer (csrc/dquant_api.cpp) with
    the kernel launchers replaced by stubs that return an error,
both with -fsanitize=address,undefined and no recovery, then runs the
oracle pins and the phase-1 ABI tests (the hand-written cases and the
hypothesis fuzz) against them in a child Python with the sanitizer runtimes
preloaded.  Any report fails the child.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "int4_quantization_amd", "csrc")
ROCM = "/opt/rocm"

STUBS = """
#include "dq_ext_internal.h"
namespace dq {
hipError_t launch_dynamic_quant(const DqPlan&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ada_layernorm_quant(const AdaPlan&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_antiquantize(const AqPlan&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_copy_probe(void*, const void*, size_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_mx_quantize(const MxPlan&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_weight_quant_matmul(const WqPlan&, void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t wq_scratch_address(void**) { return hipErrorNotSupported; }
}
"""

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g",
       "-O1"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="no host compilers")
@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")),
                    reason="HIP headers not found")
def test_host_code_is_clean_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("sanitizer runtimes not installed")
    orc = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", *SAN,
                    "-o", str(orc), os.path.join(ROOT, "oracle", "dquant_oracle.c"), "-lm"], check=True)
    stub = tmp_path / "stubs.cpp"
    stub.write_text(STUBS)
    lib = tmp_path / "libdquant_san.so"
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
                    f"-I{ROOT}/include", f"-I{CSRC}", f"-I{ROCM}/include",
                    os.path.join(CSRC, "dquant_api.cpp"), str(stub), f"-L{ROCM}/lib", "-lamdhip64",
                    f"-Wl,-rpath,{ROCM}/lib", "-o", str(lib)], check=True)
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1", DQ_ORACLE_LIBRARY=str(orc), DQ_LIBRARY=str(lib))
    tests = [os.path.join(HERE, f) for f in ("test_oracle_pins.py", "test_abi_cpu.py", "test_abi_fuzz_cpu.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-q", "-x", "-p", "no:cacheprovider", "-m",
                        "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
