"""The CPU oracle and the C ABI's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only: no GPU code runs).

Each check builds the sanitizer variant (oracle/liboracle_san.so with gcc;
activation_sparse_moe_amd/libblockffn_hostsan.so with the host pass of
hipcc, the gfx950 code unchanged), then runs a test file in a child process
with the compiler's sanitizer runtime preloaded and the variant selected
(BLOCKFFN_ORACLE_LIB / BLOCKFFN_LIB).  A sanitizer report aborts the child,
and the child first proves that the variant and the runtime are the ones it
mapped.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _child(env_extra, code=None, pytest_args=None, timeout=900):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    cmd = [sys.executable, "-c", code] if code else [sys.executable, "-m", "pytest", "-q", "-x", "-p",
                                                       "no:cacheprovider", *pytest_args]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return r.stdout


def test_oracle_pins_under_asan_and_ubsan():
    import oracle
    runtime = _gcc_asan()
    if runtime is None:
        pytest.skip("gcc's ASan runtime is not installed")
    lib = oracle.build(force=False, sanitize=True)
    env = {"LD_PRELOAD": runtime, "BLOCKFFN_ORACLE_LIB": lib}
    maps = _child(env, code="import oracle; oracle.num_threads(); print(open('/proc/self/maps').read())")
    assert "liboracle_san.so" in maps and "libasan" in maps
    _child(env, pytest_args=["tests/test_oracle_pins.py", "tests/test_oracle_backward_pins.py",
                             "tests/test_oracle_cls_pins.py", "tests/test_oracle_fff_pins.py",
                             "tests/test_oracle_router_pins.py"])


def test_capi_host_validation_under_asan_and_ubsan():
    from activation_sparse_moe_amd import build
    runtime = _clang_asan()
    if runtime is None:
        pytest.skip("the ROCm clang ASan runtime is not installed")
    lib = build.build_host_sanitized()
    env = {"LD_PRELOAD": runtime, "BLOCKFFN_LIB": lib}
    maps = _child(env, code="from activation_sparse_moe_amd import _capi; _capi.load(); "
                            "print(open('/proc/self/maps').read())")
    assert "libblockffn_hostsan.so" in maps and "libclang_rt.asan" in maps
    _child(env, pytest_args=["tests/test_capi_cpu.py"])
