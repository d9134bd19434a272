"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

qmoe_api.cpp (argument checks, workspace layout, path choice, launch order) is
compiled host-only with both sanitizers, linked with stand-ins for the kernel
launchers and the few HIP runtime calls it makes (tests/sanitize/stubs.cpp),
and driven through every entry point by tests/sanitize/host_check.cpp, which
also checks that every buffer a launcher receives lies inside the caller's
workspace and that the workspace size never decreases as T grows.  No GPU is
involved; the sanitizers abort the run on any finding.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = [
    os.path.join(ROOT, "quantized_mixture_experts_route_amd", "csrc", "qmoe_api.cpp"),
    os.path.join(ROOT, "tests", "sanitize", "stubs.cpp"),
    os.path.join(ROOT, "tests", "sanitize", "host_check.cpp"),
]
# host-only compilation of HIP sources; each -fsanitize applies to the host
# side only (there is no device code in these objects)
FLAGS = ["-x", "hip", "--cuda-host-only", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
         "-fno-omit-frame-pointer", "-w",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined",
         "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
         "-I" + os.path.join(ROOT, "quantized_mixture_experts_route_amd", "csrc"),
         "-I" + os.path.join(ROOT, "tests", "sanitize")]


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not installed")
def test_host_code_clean_under_asan_and_ubsan(tmp_path):
    objs = []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        res = subprocess.run([CLANG, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
        objs.append(obj)
    exe = str(tmp_path / "host_check")
    res = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "halt_on_error=1:detect_leaks=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "checks passed" in res.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    shutil.rmtree(tmp_path, ignore_errors=True)
