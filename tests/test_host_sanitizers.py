"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (oracle/oracle.c) built with gcc -fsanitize=address,undefined and driven on
  small odd-sized inputs of all three recurrences, fp64 and fp32, with every accepted count.
- The C ABI's host code (ssm_decode_amd/csrc/api.cpp) built host-only with the sanitizers
  (device code is not built: the kernel launchers are stand-ins that only count calls) and
  driven through every entry point with valid and invalid arguments, across configurations
  at and beyond each limit (tests/sanitize/abi_driver.cpp).
Any sanitizer report aborts the program (-fno-sanitize-recover=all), leaks included.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    rc, out = _run(["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    assert rc == 0, out
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and "checksum" in out, out


def test_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    flags = ["-x", "hip", "--cuda-host-only", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "ssm_decode_amd", "csrc")]
    objs = []
    for src in (os.path.join(ROOT, "ssm_decode_amd", "csrc", "api.cpp"), os.path.join(HERE, "abi_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        rc, out = _run([hipcc] + flags + ["-c", src, "-o", obj])
        assert rc == 0, out
        objs.append(obj)
    exe = str(tmp_path / "abi_san")
    rc, out = _run([clang, "-fsanitize=address,undefined", "-o", exe] + objs +
                   ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    assert rc == 0, out
    rc, out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"), timeout=300)
    assert rc == 0 and "failures=0" in out, out
