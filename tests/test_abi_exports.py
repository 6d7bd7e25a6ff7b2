"""The C-ABI library loads and exports every symbol include/fc_gguf.h declares
(CPU only: host-side argument validation, no kernel launches)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "fc_gguf.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fc_gguf_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from gguf_quant_block_amd import binding, build
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return binding.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n


def test_strerror_codes(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.fc_gguf_strerror(code)
    assert L.fc_gguf_strerror(-1) == b"invalid argument"
    assert b"device" in L.fc_gguf_strerror(-6)


def test_host_validation_without_gpu(L):
    h = ctypes.c_void_p()
    buf = (ctypes.c_uint8 * 176)()
    # K not a multiple of 256, N <= 0, unknown qtype, NULL blocks, NULL out
    assert L.fc_gguf_create(1, 255, 5, buf, 0, ctypes.byref(h)) == -1
    assert L.fc_gguf_create(0, 256, 5, buf, 0, ctypes.byref(h)) == -1
    for qt in (0, 3, 7, 8, -1):
        assert L.fc_gguf_create(1, 256, qt, buf, 0, ctypes.byref(h)) == -2
    assert L.fc_gguf_create(1, 256, 5, None, 0, ctypes.byref(h)) == -1
    assert L.fc_gguf_create(1, 256, 5, buf, 0, None) == -1
    # NULL handle
    assert L.fc_gguf_run(None, None, 1, None, None, None) == -1
    assert L.fc_gguf_set_path(None, 0) == -1
    assert L.fc_gguf_destroy(None) == 0
    assert L.fc_gguf_info(None, None, None, None, None) == -1
    assert L.fc_gguf_run_grouped(None, None, 1, 0, None, 1, None, None) == -1
    assert L.fc_gguf_debug_quantize(None, 1, 33, None, None, None, None) == -1
