"""The library's host code (argument validation, sizes, geometry: api.cpp)
built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
only, linked with tests/abi_sanitize.cpp, which calls every entry point on
the paths that need no GPU.  The run must end with every expectation met and
no sanitizer report.  No GPU."""

import os
import shutil
import subprocess

import pytest

from long_context_sparse_mog_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (os.path.exists(build_lib.HIPCC) and os.path.exists(CLANG)), reason="no ROCm compilers")
def test_host_abi_under_address_and_undefined_behavior_sanitizers(tmp_path):
    objs = [os.path.join(build_lib.OBJ_DIR, n) for n in ("decode.o", "build.o", "append.o")]
    if not all(os.path.exists(o) for o in objs):
        os.makedirs(build_lib.OBJ_DIR, exist_ok=True)
        for n in ("decode.hip", "build.hip", "append.hip"):
            build_lib._compile(n, [])
    api = tmp_path / "api_san.o"
    _run([build_lib.HIPCC, "-x", "hip", f"--offload-arch={build_lib.ARCH}", "-O1", "-g", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
          *HOST_SAN, "-c", os.path.join(build_lib.CSRC, "api.cpp"), "-o", str(api)])
    drv = tmp_path / "drv.o"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    _run([CLANG, "-std=c++17", "-O1", "-g", *san, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
          "-I", os.path.join(ROCM, "include"), "-c", os.path.join(ROOT, "tests", "abi_sanitize.cpp"), "-o", str(drv)])
    exe = tmp_path / "abi_sanitize"
    _run([CLANG, *san, str(drv), str(api), *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
