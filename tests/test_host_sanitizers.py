"""The host layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): the host
ABI tests (tests/test_abi_host.py: validation, error paths, launch arguments, the batched
commit, through the recording launch backend) run in a subprocess against libll_fake_san.so,
the same host sources built with -fsanitize=address,undefined, with the ASan runtime preloaded.
Any sanitizer report fails the run (undefined behaviour aborts; ASan aborts on its first
error)."""
import os
import subprocess
import sys

import pytest

from windowed_attention_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "windowed_attention_kv_amd", "libll_fake_san.so")


def _libasan():
    try:
        path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                              timeout=30).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_abi_tests_pass_under_asan_and_ubsan():
    asan = _libasan()
    if not asan or not os.path.exists(SAN_LIB):
        pytest.skip("libasan or libll_fake_san.so not available")
    env = dict(os.environ)
    env.update({"LD_PRELOAD": asan, "LL_FAKE_LIB": SAN_LIB, "LL_NO_GPU_PROBE": "1",
                # Python allocates through malloc, so ASan sees the bounds of its buffers
                "PYTHONMALLOC": "malloc",
                # Python's own allocations are not the library's: leak checking off
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
    assert _lib.FAKE_PATH != SAN_LIB      # this process keeps the plain recording build
