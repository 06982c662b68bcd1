"""libgmla's host code (validation, kernel choice, launch) built with AddressSanitizer
and UndefinedBehaviorSanitizer on the host pass only, driven through every C entry point
by tests/host_sanitize_driver.c.  Needs no GPU: calls that pass validation reach the
launch, which fails without a device and must return GMLA_ERR_HIP."""
import os
import shutil
import subprocess

import pytest
import torch

from causal_softmax_attention_gmla_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/lib/llvm/bin/clang"


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device launch path")
@pytest.mark.skipif(not os.path.exists(CLANG), reason="needs the ROCm clang")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    lib = tmp_path / "libgmla_sanitized.so"
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    # -Xarch_host before each -fsanitize=: instrument the host pass only
    cmd = [B.hipcc(), "-O1", "-g", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={B.ARCH}",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-I", B.INCLUDE, "-I", B.CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *srcs, "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = tmp_path / "driver"
    cmd = [CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-I", B.INCLUDE,
           os.path.join(ROOT, "tests", "host_sanitize_driver.c"), "-o", str(exe), f"-L{tmp_path}",
           "-lgmla_sanitized", "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{tmp_path}",
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    # the driver also checks for a device itself and exits 77 before any call if one is
    # visible; the environment hides every device from it as well
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1", ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    if run.returncode == 77:
        pytest.skip("a HIP device is visible")
    assert run.returncode == 0, run.stdout + run.stderr[-3000:]
    assert "0 failures" in run.stdout
