"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The whole library is compiled again with both sanitizers on the host pass only (device code is
unchanged) into a temporary directory, and tests/host_abi_driver.cpp is run against that copy.  The
driver covers argument checks, workspace layouts, varlen batch rules and status strings over a grid
of valid and invalid shapes, plus every entry point on arguments that validation rejects.  No call
reaches a kernel launch, and the check runs only where no GPU is visible.
"""

import os
import subprocess

import pytest
import torch

from token_sparse_attention_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang++"
# host pass only: each sanitizer flag goes right after -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.timeout(900)
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    if torch.cuda.is_available():
        pytest.skip("host-only check: it runs where no GPU is visible")
    if not os.path.exists(CLANG):
        pytest.fail(f"{CLANG} not found")
    lib = build.build(extra=SAN, lib_path=str(tmp_path / "libtsa_san.so"), obj_dir=str(tmp_path / "obj"))
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms, "the library copy is not instrumented"
    exe = str(tmp_path / "host_abi_driver")
    r = subprocess.run([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                        "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "host_abi_driver.cpp"), lib,
                        "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert "0 unexpected statuses" in r.stdout, out
