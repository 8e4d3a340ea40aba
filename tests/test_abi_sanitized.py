"""The host half of the C ABI built with AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

csrc/api.hip and csrc/stream_probe.hip are compiled with the sanitizers on
their host code only (device code unchanged), linked with stand-in kernel
launchers that record their arguments (tests/sanitize/stub_launch.cpp) and
driven by tests/sanitize/abi_host_check.cpp: every entry point with refused
arguments, accepted ones and sizes at the int32 / int64 edges.  Any
sanitizer report or failed check fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "paged_split_kv_decode_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                                reason="needs the ROCm compilers")

# sanitizers on the host side of a HIP source only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_host_abi_under_address_and_ub_sanitizers():
    if os.path.isdir(OUT):
        shutil.rmtree(OUT)
    os.makedirs(OUT)
    inc = ["-I", os.path.join(ROOT, "include")]
    objs = []
    for src in ("api.hip", "stream_probe.hip"):
        obj = os.path.join(OUT, src + ".o")
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++20", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN, *inc,
              "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in ("stub_launch.cpp", "abi_host_check.cpp"):
        obj = os.path.join(OUT, src + ".o")
        _run([CLANGXX, "-O1", "-g", "-std=c++20", "-D__HIP_PLATFORM_AMD__",
              "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-I", os.path.join(ROCM, "include"), *inc,
              "-c", os.path.join(SAN, src), "-o", obj])
        objs.append(obj)
    exe = os.path.join(OUT, "abi_host_check")
    _run([CLANGXX, "-fsanitize=address,undefined", *objs, "-L", os.path.join(ROCM, "lib"),
          "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"sanitized ABI check failed:\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "checks passed" in r.stdout, r.stdout
