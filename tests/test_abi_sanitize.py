"""The C ABI's host code under the address and undefined-behaviour sanitizers
(CPU only): api.cpp is rebuilt with host sanitizers, linked with the kernel
objects of the last full build and tests/abi_sanitize_driver.cpp, and the
driver walks every entry point's validation and error paths, extreme sizes
included; any sanitizer report aborts it."""

import os
import shutil
import subprocess

import pytest
import torch

from bit_weight_quantized_qlq_amd import build as B

HIPCC_OK = os.path.exists(B.HIPCC) or shutil.which("hipcc") is not None
OBJS_OK = all(os.path.exists(os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o")) for s in B.SOURCES[1:])


@pytest.mark.skipif(not HIPCC_OK, reason="hipcc not available")
@pytest.mark.skipif(not OBJS_OK, reason="kernel objects not built (run the full build first)")
def test_abi_validation_under_host_sanitizers():
    exe = B.build_abi_sanitize_driver()
    syms = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "driver is not instrumented"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    args = [exe] if torch.cuda.is_available() else [exe, "--no-device"]
    r = subprocess.run(args, capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("PASS"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
