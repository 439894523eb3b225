"""The C ABI's host code built with AddressSanitizer and
UndefinedBehaviorSanitizer, exercised on the CPU by tests/cpp/abi_sanitize.cpp:
argument validation of every entry-point family, the index checks of the
debug mode (GDR_DEBUG_CHECKS), and that the debug mode engages before any
kernel launch.  The kernels' objects are the regular build's; only host code
is instrumented."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gated_delta_rule_amd")
CSRC = os.path.join(PKG, "csrc")


def _tool(name):
    for cand in (shutil.which(name), os.path.join("/opt/rocm/bin", name)):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.slow
def test_abi_under_host_sanitizers(tmp_path):
    hipcc, gxx = _tool("hipcc"), shutil.which("g++")
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "kernels_*.o")))
    if not hipcc or not gxx or not objs:
        pytest.skip("needs hipcc, g++ and the regular build's kernel objects")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api_o = str(tmp_path / "gdr_api_san.o")
    # host-side instrumentation only: each sanitizer flag is scoped to the host pass
    subprocess.run([hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-omit-frame-pointer", "-Wno-unused-command-line-argument",
                    *inc, "-c", os.path.join(CSRC, "gdr_api.cpp"), "-o", api_o],
                   check=True, capture_output=True, text=True)
    test_o = str(tmp_path / "abi_sanitize.o")
    subprocess.run([gxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    *inc, "-c", os.path.join(ROOT, "tests", "cpp", "abi_sanitize.cpp"), "-o", test_o],
                   check=True, capture_output=True, text=True)
    exe = str(tmp_path / "abi_sanitize")
    subprocess.run([gxx, "-fsanitize=address,undefined", test_o, api_o, *objs, "-L/opt/rocm/lib",
                    "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
