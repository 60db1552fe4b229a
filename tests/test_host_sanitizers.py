"""Host AddressSanitizer + UndefinedBehaviorSanitizer builds (CPU only):

* the oracle (oracle/oracle.c, gcc) driven through every function on tiny
  inputs (tests/sanitize/oracle_driver.c);
* the C ABI's host code (yoco_shared_kv_amd/csrc/api.cpp, host pass
  sanitized) linked with the library's kernel objects and driven through
  its helpers and the validation of every entry point
  (tests/sanitize/abi_driver.c); no call passes validation, so nothing is
  launched, and the test is skipped where a GPU is visible.

Any memory error, leak (oracle) or undefined behaviour aborts the driver."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, env=None, timeout=600):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert res.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({res.returncode}):\n{res.stdout}\n{res.stderr[-4000:]}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", *SAN, "-fopenmp", "-std=c11", "-Wall", "-o", exe,
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", OMP_NUM_THREADS="2")
    res = _run([exe], env=env)
    assert "all functions ran clean" in res.stdout


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not available")
@pytest.mark.skipif(_gpu_visible(), reason="host-only check; a visible GPU is not needed and is left alone")
def test_c_abi_host_code_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from yoco_shared_kv_amd import build as hip_build
    kernel_objs = [os.path.join(hip_build.BUILD_DIR, s + ".o") for s in hip_build.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in kernel_objs):
        hip_build.build()
    inc = os.path.join(ROOT, "include")
    api_o, drv_o, exe = str(tmp_path / "api_san.o"), str(tmp_path / "driver.o"), str(tmp_path / "abi_san")
    # device code of api.cpp is empty; the sanitizers go on the host pass only
    host_san = [f for flag in SAN for f in ("-Xarch_host", flag)]
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-I", inc, *host_san, "-c",
          os.path.join(ROOT, "yoco_shared_kv_amd", "csrc", "api.cpp"), "-o", api_o])
    _run([CLANG, "-O1", "-g", *SAN, "-Wall", "-I", inc, "-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"),
          "-o", drv_o])
    _run([CLANGXX, *SAN, "-o", exe, drv_o, api_o, *kernel_objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib"])
    # leak checking is off: the HIP runtime keeps allocations for the process lifetime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = _run([exe], env=env)
    assert "every host path ran clean" in res.stdout
