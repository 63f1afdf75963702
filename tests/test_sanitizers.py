"""Sanitizer runs on the CPU (no GPU is touched):

- the fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
  (every report fatal), with the oracle's pin tests run against it;
- the C ABI's host code built with the same sanitizers (``-Xarch_host``: the
  device code is compiled as usual) and driven by tests/sanitize/abi_driver.c
  through every entry point's argument errors.

Both builds go to a temporary directory, outside the tree."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    lib = tmp_path / "libswinoracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", *SAN, "-o", str(lib),
                    os.path.join(ROOT, "oracle", "swin_oracle.c"), "-lm", "-lpthread"], check=True)
    env = dict(os.environ, SWIN_ORACLE_LIB=str(lib), LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail


def test_c_abi_host_code_under_address_and_undefined_sanitizers(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc is not installed")
    sys.path.insert(0, os.path.join(ROOT, "shifted_window_attention_swin_amd"))
    try:
        import build as swa_build  # the library's own build command
    finally:
        sys.path.pop(0)
    lib = tmp_path / "libswinattn_san.so"
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    cmd = swa_build.command(str(lib), extra=host_san)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-3000:]
    # the ABI test program is built by the same clang, whose sanitizer runtime the
    # library's instrumentation expects (it is linked into the executable)
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    drv = tmp_path / "abi_driver"
    subprocess.run([clang, "-O1", "-g", *SAN, "-o", str(drv),
                    os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), str(lib),
                    f"-Wl,-rpath,{tmp_path}"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([str(drv)], capture_output=True, text=True, timeout=300, env=env)
    out = res.stdout + res.stderr
    print(out[-2000:])
    assert res.returncode == 0 and "clean" in res.stdout, out[-3000:]
