"""The C-ABI's host layer (argument validation, handle bookkeeping) built with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only; the kernels
are the regular build) and test_abi_exports.py run against that build in a
child process that preloads the ASan runtime.  CPU only."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import ctypes, os
from gguf_quant_block_amd import binding
L = binding.lib()
maps = open("/proc/self/maps").read()
assert os.path.basename(binding.LIB_PATH) == "libfcgguf_san.so", binding.LIB_PATH
assert binding.LIB_PATH in maps
assert hasattr(ctypes.CDLL(None), "__asan_init")          # the runtime is live in this process
print("sanitized build loaded")
"""


@pytest.fixture(scope="module")
def san_env():
    from gguf_quant_block_amd import build
    lib = build.build_sanitized()
    rt = build.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env.update(FC_GGUF_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=ROOT + os.pathsep + env.get("PYTHONPATH", ""))
    return env


def test_sanitized_library_is_the_one_loaded(san_env):
    r = subprocess.run([sys.executable, "-c", PROBE], env=san_env, cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized build loaded" in r.stdout


def test_abi_exports_under_asan_ubsan(san_env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_exports.py")],
                       env=san_env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out
