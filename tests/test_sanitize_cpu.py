"""The CPU oracle and the library's host-only argument checks built with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, no GPU code) and driven by tests/sanitize_driver.cpp: exact-size
buffers, ragged shapes, both scale layouts, and adversarial sizes for every check. Any
out-of-bounds access, leak, signed overflow or other undefined behaviour aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc and g++")
def test_oracle_and_host_checks_under_sanitizers(tmp_path):
    objs = []
    for src in ("oracle/mxfp8_oracle.c", "oracle/accum_bound.c"):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run(["gcc", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", *SAN, "-c",
                        os.path.join(ROOT, src), "-o", obj], check=True)
        objs.append(obj)
    exe = str(tmp_path / "sanitize_driver")
    subprocess.run(["g++", "-std=c++17", "-fopenmp", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "quant_mxfp8_gemm_amd", "csrc", "checks.cpp"),
                    os.path.join(ROOT, "tests", "sanitize_driver.cpp"), *objs, "-o", exe, "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitize ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
