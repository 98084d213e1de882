"""The host core (tq_host.cpp: codebooks, the splitmix64 / Box-Muller streams, layout
and size arithmetic, validation) built with AddressSanitizer and UndefinedBehaviorSanitizer
by g++ (no device code involved) and run through tests/host_sanitize_driver.cpp, which
calls every host entry point of that file with valid and invalid arguments and checks the
invariants callers rely on.  Any sanitizer report fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_domain_attention_kv_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"  # tq.h names hipStream_t from the HIP runtime API header


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_host_core_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "tq_host_sanitized"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", ROCM_INCLUDE,
           "-D__HIP_PLATFORM_AMD__", os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
           os.path.join(CSRC, "tq_host.cpp"), "-o", str(exe), "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)  # the sanitizer runtime must come first
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "all checks passed" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
