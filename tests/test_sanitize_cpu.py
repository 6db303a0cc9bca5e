"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the C-ABI layer (q8_api.cpp, with a fake HIP runtime and recording
stand-ins for the kernel launchers, tests/sanitize/api_harness.cpp) and the
oracle (q8_oracle.c, tests/sanitize/oracle_harness.c).  Both are built with the
host compilers here (no device code is compiled) into a temporary directory and
run; any sanitizer report fails the test.  Skipped in a process that has
initialised a GPU, where no compiler may be started."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


@pytest.fixture(autouse=True)
def _no_gpu_process():
    import sys
    torch = sys.modules.get("torch")
    if torch is not None and torch.cuda.is_initialized():
        pytest.skip("this process has initialised a GPU")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_api_layer_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "int8_weight_streaming_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    exe = str(tmp_path / "api_harness")
    _run(["g++", "-std=c++17", *SAN, *inc, os.path.join(ROOT, "int8_weight_streaming_amd", "csrc", "q8_api.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "api_harness.cpp"), "-o", exe], str(tmp_path))
    r = _run([exe], str(tmp_path))
    assert "api harness ok" in r.stdout
    assert "runtime error" not in r.stderr


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_harness")
    _run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN,
          os.path.join(ROOT, "oracle", "q8_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_harness.c"),
          "-lm", "-o", exe], str(tmp_path))
    r = _run([exe], str(tmp_path))
    assert "oracle harness ok" in r.stdout
    assert "runtime error" not in r.stderr
