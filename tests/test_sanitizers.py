"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code,
run on the CPU.

* the oracle's C core (oracle/attention.c) under a driver that runs its
  forward and backward on small seeded inputs with every kind of
  visible-key count (tests/native/oracle_san_driver.c);
* the C ABI's host code (long_context_causal_amd/csrc/api.cpp: argument
  validation, the step schedule, workspace carving, the merge passes, the
  grid bounds) linked with host stand-ins for the kernel launchers
  (tests/native/launch_stubs.cpp) under a driver that calls every entry
  point with valid and invalid arguments (tests/native/abi_san_driver.cpp).

Both are built with gcc / g++ (host code only, no device code) with
-fsanitize=address,undefined and no recovery, so any report fails the run.
Also here: the build's check that no kernel spills to scratch memory.
"""
import os
import shutil
import subprocess

import pytest

from long_context_causal_amd import build as cbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_core_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "attention.c"),
          os.path.join(NATIVE, "oracle_san_driver.c"), "-o", exe, "-lm"])
    res = _run([exe], env=dict(os.environ, OMP_NUM_THREADS="2"))
    assert "ok" in res.stdout


@pytest.mark.skipif(shutil.which("g++") is None or
                    not os.path.exists(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime_api.h")),
                    reason="g++ or the HIP runtime headers are not installed")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    csrc = os.path.join(ROOT, "long_context_causal_amd", "csrc")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
          "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "api.cpp"),
          os.path.join(NATIVE, "launch_stubs.cpp"), os.path.join(NATIVE, "abi_san_driver.cpp"),
          "-o", exe])
    res = _run([exe])
    assert "ok" in res.stdout


def test_build_refuses_kernels_that_spill():
    remarks = "\n".join([
        "x.hip:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=...]",
        "x.hip:9:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=...]",
    ])
    assert cbuild.scratch_users(remarks) == [("kern_b", 16)]
    assert cbuild.scratch_users(remarks.replace(": 16 ", ": 0 ")) == []
