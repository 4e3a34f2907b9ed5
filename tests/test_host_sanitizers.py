"""The C-ABI host layer under AddressSanitizer and UndefinedBehaviorSanitizer,
and under ThreadSanitizer for calls from several threads at once.

tests/host_harness/abi_harness.cpp links the host layer (zero_abi.cpp) with
stubs of the device side that record each launch's tables, and checks the
validation paths, the bucket and flatten batching, the bias tables (and
their per-thread cache), the accumulate modes, the host loss scaler and
concurrent calls with per-thread error text.  It is built with g++ (host
code only, no device code) and run here, on the CPU."""
import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HARNESS = os.path.join(ROOT, "tests", "host_harness", "abi_harness.cpp")
ABI = os.path.join(ROOT, "sharded_mixed_precision_step_amd", "csrc", "zero_abi.cpp")
INCLUDES = [os.path.join(ROOT, "include"),
            os.path.join(ROOT, "sharded_mixed_precision_step_amd", "csrc"),
            "/opt/rocm/include"]


def _build(tmp_path, name, sanitize):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path / name)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread",
           sanitize, "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__"]
    for inc in INCLUDES:
        cmd += ["-I", inc]
    cmd += [HARNESS, ABI, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    return exe


def test_abi_host_layer_under_sanitizers(tmp_path):
    exe = _build(tmp_path, "abi_harness", "-fsanitize=address,undefined")
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "abi harness: ok" in run.stdout


def test_abi_host_layer_from_many_threads_under_tsan(tmp_path):
    exe = _build(tmp_path, "abi_harness_tsan", "-fsanitize=thread")
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    run = subprocess.run([exe, "threads"], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "abi harness: ok" in run.stdout
    assert "ThreadSanitizer" not in run.stderr
