"""The C-ABI validation tests again, against the library built with
AddressSanitizer and UndefinedBehaviorSanitizer on its host code
(``build(sanitize=True)``), in a child process with the sanitizer runtime
preloaded. Any invalid memory access or undefined behaviour in the argument
validation and dispatch code aborts that run (no recovery), so the run must
finish clean. CPU only: no kernel is launched."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from exact_attention_104_amd import build as B  # noqa: E402

LIB = os.path.join(B.PKG, B.HOSTSAN_LIB_NAME)

CHECK = r"""
import ctypes, sys
lib = ctypes.CDLL(sys.argv[1])
maps = open("/proc/self/maps").read()
assert "libclang_rt.asan" in maps, "sanitizer runtime not mapped"
assert hasattr(ctypes.CDLL(None), "__asan_init"), "sanitizer runtime not loaded"
assert lib.fa_abi_version() >= 4
print("hostsan ok")
"""


def _env():
    rt = B.hostsan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    if not os.path.exists(LIB):
        B.build(verbose=False, sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1",
               FA_MI355X_LIB=LIB)
    return env


def test_hostsan_library_is_instrumented():
    env = _env()
    r = subprocess.run([sys.executable, "-c", CHECK, LIB], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "hostsan ok" in r.stdout, r.stdout + r.stderr


def test_abi_tests_clean_under_host_sanitizers():
    env = _env()
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
