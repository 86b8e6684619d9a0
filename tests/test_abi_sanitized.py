"""The library's host-side argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU needed).

mss_api.hip is compiled again with the sanitizers on its host code only (each
-fsanitize= behind -Xarch_host, so no device code is instrumented) and linked
with the regular kernel objects into a separate library; abi_sanitized.cpp
drives every entry point into its rejection paths, including int64 size
products that overflow.  Any sanitizer report fails the run."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import mamba_selective_scan_causal_amd as mss
from mamba_selective_scan_causal_amd import build as hip_build

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = "address,undefined"


def _clangxx():
    for c in ("/opt/rocm/llvm/bin/clang++", "/opt/rocm/lib/llvm/bin/clang++"):
        if os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    cxx = _clangxx()
    if cxx is None or shutil.which(hip_build.hipcc()) is None:
        pytest.skip("hipcc / clang++ not available")
    mss.lib()  # the regular build must exist: its kernel objects are reused
    objdir = hip_build.OBJDIR
    kernels = [os.path.join(objdir, s.replace(".hip", ".o"))
               for s in hip_build.SOURCES if s != "mss_api.hip"]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        pytest.skip(f"kernel objects missing: {missing}")
    out = tmp_path_factory.mktemp("asan")
    api_o = str(out / "mss_api_san.o")
    lib = str(out / "libmss_san.so")
    exe = str(out / "abi_sanitized")
    hipcc = hip_build.hipcc()
    host_san = ["-Xarch_host", f"-fsanitize={SAN}", "-Xarch_host", "-fno-sanitize-recover=all",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    cmds = [
        [hipcc, *hip_build.FLAGS, *host_san, "-c",
         os.path.join(hip_build.CSRC, "mss_api.hip"), "-o", api_o],
        [hipcc, f"--offload-arch={hip_build.ARCH}", "-shared", "-fPIC", "-Xarch_host",
         f"-fsanitize={SAN}", "-o", lib, api_o, *kernels],
        [cxx, "-std=c++17", "-O1", "-g", f"-fsanitize={SAN}", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", hip_build.INCLUDE,
         "-I", "/opt/rocm/include", os.path.join(HERE, "abi_sanitized.cpp"), lib,
         f"-Wl,-rpath,{out}", "-Wl,-rpath,/opt/rocm/lib", "-L/opt/rocm/lib", "-lamdhip64",
         "-o", exe],
    ]
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        assert r.returncode == 0, " ".join(c) + "\n" + hip_build._quiet(r.stderr)[-3000:]
    return exe


def test_host_checks_clean_under_asan_ubsan(sanitized_driver):
    env = dict(os.environ)
    # the HIP runtime is not instrumented and keeps allocations until exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "all checks passed" in r.stdout, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
