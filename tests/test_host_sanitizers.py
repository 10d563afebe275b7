"""The host code of the library under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with every -fsanitize= applied to the host pass only
(block_sparse_attention_select_amd/_build.py: build_sanitized), and a C++
driver built with the same sanitizers (tests/abi_host_check.cpp) exercises the
argument checks of every entry point: made-up aligned device pointers, each call
expected to return its status before launching anything.  Any sanitizer report
aborts the driver.  CPU only; slow (one sanitized rebuild)."""
import os
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = [pytest.mark.slow,
              pytest.mark.skipif(torch.cuda.is_available(), reason="uses fake device pointers; CPU-only host check")]


def test_abi_checks_under_asan_and_ubsan(tmp_path):
    from block_sparse_attention_select_amd import _build
    clang = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(clang) or shutil.which(_build.hipcc()) is None and not os.path.exists(_build.hipcc()):
        pytest.skip("ROCm clang not available")
    lib = _build.build_sanitized()
    exe = str(tmp_path / "abi_host_check")
    cmd = [clang, "-std=c++17", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "abi_host_check.cpp"), lib,
           "-Wl,-rpath," + os.path.dirname(lib), "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all statuses as expected" in r.stdout
