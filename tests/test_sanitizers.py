"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/sanitize/oracle_driver.c includes oracle/oracle.c and calls every
function on exactly-sized buffers (ragged tensors, empty and one-element
shards, special values, rejected arguments).  Built with gcc's ASan and
UBSan, any out-of-bounds access, leak or undefined operation fails the run.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_is_clean_under_asan_and_ubsan():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_driver")
        cmd = [gcc, "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wno-unknown-pragmas",
               "-o", exe, os.path.join(HERE, "sanitize", "oracle_driver.c"), "-lm"]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        proc = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert proc.returncode == 0, proc.stderr[-4000:]
        assert "runtime error" not in proc.stderr and "AddressSanitizer" not in proc.stderr, proc.stderr[-4000:]
        assert "oracle sanitizer drive: ok" in proc.stdout


def test_c_abi_validation_is_clean_under_asan_and_ubsan():
    """The library's host code (argument validation, overlap checks, scalar
    setup) built with the sanitizers on the host pass, driven through every
    rejecting path by tests/sanitize/abi_driver.cpp.  No call in the driver
    reaches a launch; it runs only where no GPU is visible all the same."""
    import torch
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    if torch.cuda.device_count() > 0:
        pytest.skip("host-only check: run where no GPU is visible")
    root = os.path.dirname(HERE)
    csrc = os.path.join(root, "fsdp_sharded_optimizer_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "abi_driver")
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
               "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(root, "include"), "-o", exe,
               os.path.join(HERE, "sanitize", "abi_driver.cpp"), *srcs]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
        proc = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert proc.returncode == 0, (proc.stdout + proc.stderr)[-4000:]
        assert "runtime error" not in proc.stderr and "AddressSanitizer" not in proc.stderr, proc.stderr[-4000:]
        assert "abi sanitizer drive: ok" in proc.stdout
