"""The C-ABI libraries load and export every symbol their headers declare:
include/fc_gguf.h (libfcgguf.so, the FC) and include/fc_gguf_ceilings.h
(libfcgceil.so, the benchmark's ceiling kernels).  CPU only: host-side
argument validation, no kernel launches."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header="fc_gguf.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fc_\w+)\s*\(", src)))


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


def test_every_header_has_its_library():
    # each header under include/ is served by one in-tree library
    from gguf_quant_block_amd import build
    libs = {"fc_gguf.h": build.LIB, "fc_gguf_ceilings.h": build.CEIL_LIB}
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(libs)
    if not os.path.exists(build.CEIL_LIB):
        build.build()
    C = ctypes.CDLL(build.CEIL_LIB)
    names = _declared("fc_gguf_ceilings.h")
    assert names == ["fc_ceiling_mfma", "fc_ceiling_stream_read"]
    for n in names:
        assert hasattr(C, n), n
    # argument checks (no launch): misaligned or ragged sizes, bad unroll, bad dtype
    C.fc_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    C.fc_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert C.fc_ceiling_stream_read(None, 16, 1, 1, None, None) == -1
    assert C.fc_ceiling_stream_read(16, 17, 1, 1, 16, None) == -1
    assert C.fc_ceiling_stream_read(16, 16, 1, 3, 16, None) == -1
    assert C.fc_ceiling_stream_read(8, 16, 1, 1, 16, None) == -1
    assert C.fc_ceiling_mfma(2, 1, 1, 16, None) == -1
    assert C.fc_ceiling_mfma(0, 0, 1, 16, None) == -1


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
    assert L.fc_gguf_debug_quantize(None, 1, 33, None, None, None, None, None) == -1


def test_size_limits_without_gpu(L):
    # sizes past the 32-bit indexing limits are rejected before any device call
    h = ctypes.c_void_p()
    buf = (ctypes.c_uint8 * 176)()
    assert L.fc_gguf_create(1 << 31, 256, 5, buf, 0, ctypes.byref(h)) == -5
    assert L.fc_gguf_create(1, 1 << 31, 5, buf, 0, ctypes.byref(h)) == -5
    assert L.fc_gguf_create(1 << 20, 1 << 20, 5, buf, 0, ctypes.byref(h)) == -5
    assert L.fc_gguf_create_grouped(1 << 20, 16, 256, 6, buf, 0, ctypes.byref(h)) == -5
    assert L.fc_gguf_create_grouped(0, 16, 256, 6, buf, 0, ctypes.byref(h)) == -1
    assert not h.value
    assert L.fc_gguf_run_grouped_noalloc(None, None, 1, 0, None, 1, None, None) == -1
    assert L.fc_gguf_debug_quantize(buf, 1, 33, buf, buf, buf, None, None) == -1
    assert L.fc_gguf_debug_quantize_f32(buf, -1, 32, buf, buf, buf, None, None) == -1


def test_bucketing_argument_checks_without_gpu(L):
    buf = (ctypes.c_int32 * 64)()
    assert L.fc_gguf_debug_bucketing(buf, 4, 8, 16, buf, buf, None, buf, None) == -1   # NULL tiles
    assert L.fc_gguf_debug_bucketing(buf, -1, 8, 16, buf, buf, buf, buf, None) == -1   # P < 0
    assert L.fc_gguf_debug_bucketing(buf, 4, 0, 16, buf, buf, buf, buf, None) == -1    # E < 1
    assert L.fc_gguf_debug_bucketing(buf, 4, 8, 0, buf, buf, buf, buf, None) == -1     # BM < 1
    assert L.fc_gguf_debug_bucketing(buf, 4, 8, 4097, buf, buf, buf, buf, None) == -1  # BM too large
    assert L.fc_gguf_debug_bucketing(buf, 4, 4097, 16, buf, buf, buf, buf, None) == -5  # E too large
    assert L.fc_gguf_debug_bucketing(buf, (1 << 30) + 1, 8, 16, buf, buf, buf, buf, None) == -5
    assert L.fc_gguf_debug_bucketing(None, 0, 8, 16, None, None, None, None, None) == 0  # P = 0: no-op
