"""Every single-device error code of the C-ABI, forced through the library on
the GPU: misaligned A / Y / R (FC_GGUF_EINVAL), sizes past the 32-bit
indexing limits (FC_GGUF_ERANGE), failed allocations (FC_GGUF_ENOMEM, by
FC_GGUF_TEST_FAIL_ALLOC), an unknown qtype or path (FC_GGUF_EUNSUPPORTED).
Each rejected call is checked to leave its output untouched and the handle
usable.  No kernel is launched for a rejected call."""

import ctypes

import numpy as np
import pytest

from gguf_quant_block_amd import synth
from gguf_quant_block_amd.binding import FcGguf, FcGgufError, lib
from helpers import DECODE_TOL, case, check_fro, maxrel
from oracle import fc as ofc

pytestmark = pytest.mark.gpu

EINVAL, EUNSUPPORTED, ENOMEM, ERANGE = -1, -2, -3, -5


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t, byte_offset=0):
    return ctypes.c_void_p(t.data_ptr() + byte_offset)


def _run(h, A, M, R, Y, f32=False):
    fn = lib().fc_gguf_run_f32 if f32 else lib().fc_gguf_run
    return fn(h.handle, A, M, R, Y, _stream())


@pytest.fixture
def small():
    import torch
    qtype, M, N, K = "q5_k", 3, 64, 512
    w, A, R = case(qtype, M, N, K, 80, 0)
    h = FcGguf(N, K, qtype, w)
    # buffers with room for a shifted view
    Ab = torch.zeros(M * K + 64, dtype=torch.float16, device="cuda")
    Rb = torch.zeros(M * N + 64, dtype=torch.float16, device="cuda")
    Yb = torch.full((M * N + 64,), 7.0, dtype=torch.float16, device="cuda")
    Ab[:M * K] = _dev(A).reshape(-1)
    Rb[:M * N] = _dev(R).reshape(-1)
    return dict(h=h, w=w, A=A, R=R, M=M, N=N, K=K, qtype=qtype, Ab=Ab, Rb=Rb, Yb=Yb)


@pytest.mark.parametrize("what,off", [("A", 2), ("A", 8), ("Y", 2), ("Y", 4), ("R", 2), ("R", 6)])
def test_misaligned_pointers_are_einval(gpu_lib, small, what, off):
    import torch
    s = small
    A = _p(s["Ab"], off if what == "A" else 0)
    R = _p(s["Rb"], off if what == "R" else 0)
    Y = _p(s["Yb"], off if what == "Y" else 0)
    before = s["Yb"].clone()
    assert _run(s["h"], A, s["M"], R, Y) == EINVAL
    torch.cuda.synchronize()
    assert torch.equal(s["Yb"], before)                  # nothing written
    # the handle still works on aligned pointers
    assert _run(s["h"], _p(s["Ab"]), s["M"], _p(s["Rb"]), _p(s["Yb"])) == 0
    torch.cuda.synchronize()
    y = s["Yb"][:s["M"] * s["N"]].reshape(s["M"], s["N"]).cpu().numpy()
    assert maxrel(y, ofc.fc_ref_int8(s["A"], s["w"], s["qtype"], s["R"])) <= DECODE_TOL


def test_misaligned_f32_pointers_are_einval(gpu_lib, small):
    import torch
    s = small
    A32 = torch.zeros(s["M"] * s["K"] + 16, dtype=torch.float32, device="cuda")
    Y32 = torch.zeros(s["M"] * s["N"] + 16, dtype=torch.float32, device="cuda")
    assert _run(s["h"], _p(A32, 4), s["M"], None, _p(Y32), f32=True) == EINVAL
    assert _run(s["h"], _p(A32), s["M"], None, _p(Y32, 2), f32=True) == EINVAL
    assert _run(s["h"], _p(A32), s["M"], _p(Y32, 2), _p(Y32), f32=True) == EINVAL
    assert _run(s["h"], _p(A32), s["M"], None, _p(Y32), f32=True) == 0


def test_null_and_negative_are_einval(gpu_lib, small):
    s = small
    assert _run(s["h"], None, s["M"], None, _p(s["Yb"])) == EINVAL
    assert _run(s["h"], _p(s["Ab"]), s["M"], None, None) == EINVAL
    assert _run(s["h"], _p(s["Ab"]), -1, None, _p(s["Yb"])) == EINVAL
    assert lib().fc_gguf_run(None, _p(s["Ab"]), s["M"], None, _p(s["Yb"]), _stream()) == EINVAL
    assert _run(s["h"], None, 0, None, None) == 0        # M == 0: a no-op


@pytest.mark.parametrize("M", [1 << 25, (1 << 31) // 64 + 1])
def test_oversized_rows_are_erange(gpu_lib, small, M):
    # M x N (or M x K) past 2^31 elements, or M past the row limit: rejected
    # before any access to A, R or Y (the buffers are far smaller)
    import torch
    s = small
    before = s["Yb"].clone()
    assert _run(s["h"], _p(s["Ab"]), M, _p(s["Rb"]), _p(s["Yb"])) == ERANGE
    torch.cuda.synchronize()
    assert torch.equal(s["Yb"], before)


def test_oversized_grouped_is_erange(gpu_lib):
    import torch
    E, N, K, T, top_k = 4, 64, 256, 4, 2
    w = synth.blocks("q4_k", E * N, K, synth.rng(81, 0, 0)).reshape(E, N, -1)
    fc = FcGguf(N, K, "q4_k", w, experts=E)
    A = torch.zeros((T, K), dtype=torch.float16, device="cuda")
    ids = torch.zeros((T, top_k), dtype=torch.int32, device="cuda")
    Y = torch.zeros((T, top_k, N), dtype=torch.float16, device="cuda")
    run = lib().fc_gguf_run_grouped
    assert run(fc.handle, _p(A), 1 << 40, 0, _p(ids), top_k, _p(Y), _stream()) == ERANGE
    assert run(fc.handle, _p(A), T, 0, _p(ids), top_k, _p(Y), _stream()) == 0


def test_unknown_qtype_and_path(gpu_lib):
    w = synth.blocks("q4_k", 16, 256, synth.rng(82, 0, 0))
    h = ctypes.c_void_p()
    rc = lib().fc_gguf_create(16, 256, 3, ctypes.c_void_p(w.ctypes.data), 0, ctypes.byref(h))
    assert rc == EUNSUPPORTED and not h.value
    fc = FcGguf(16, 256, "q4_k", w)
    assert lib().fc_gguf_set_path(fc.handle, 99) == EUNSUPPORTED


def test_failed_create_is_enomem(gpu_lib, monkeypatch):
    w = synth.blocks("q6_k", 32, 512, synth.rng(83, 0, 0))
    for env in ("create", "all"):
        monkeypatch.setenv("FC_GGUF_TEST_FAIL_ALLOC", env)
        with pytest.raises(FcGgufError) as ei:
            FcGguf(32, 512, "q6_k", w)
        assert ei.value.code == ENOMEM
    monkeypatch.setenv("FC_GGUF_TEST_FAIL_ALLOC", "workspace")
    FcGguf(32, 512, "q6_k", w)                           # weights only: no workspace yet
    monkeypatch.delenv("FC_GGUF_TEST_FAIL_ALLOC")
    FcGguf(32, 512, "q6_k", w)


@pytest.mark.parametrize("path", ["prefill", "int8", "scratch"])
def test_failed_workspace_is_enomem_and_recovers(gpu_lib, monkeypatch, path):
    # a first call that needs a workspace fails cleanly while allocation is
    # refused, leaves Y untouched, and succeeds once it is allowed again
    import torch
    qtype, M, N, K = "q5_k", 64, 128, 8192          # split-K grid: partials need workspace
    w, A, R = case(qtype, M, N, K, 84, 0)
    fc = FcGguf(N, K, qtype, w)
    fc.set_path(path)
    Ad, Rd = _dev(A), _dev(R)
    Y = torch.full((M, N), 3.0, dtype=torch.float16, device="cuda")
    monkeypatch.setenv("FC_GGUF_TEST_FAIL_ALLOC", "workspace")
    rc = lib().fc_gguf_run(fc.handle, _p(Ad), M, _p(Rd), _p(Y), _stream())
    torch.cuda.synchronize()
    assert rc == ENOMEM, rc
    assert bool((Y == 3.0).all())
    monkeypatch.delenv("FC_GGUF_TEST_FAIL_ALLOC")
    fc(Ad, Rd, out=Y)
    torch.cuda.synchronize()
    if path == "int8":
        assert maxrel(Y.cpu().numpy(), ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL
    else:
        check_fro(Y.cpu().numpy(), ofc.fc_gguf_ref(A, w, qtype, R))


def test_failed_grouped_workspace_is_enomem(gpu_lib, monkeypatch):
    import torch
    E, N, K, T, top_k = 8, 64, 256, 16, 2
    w = synth.blocks("q6_k", E * N, K, synth.rng(85, 0, 0)).reshape(E, N, -1)
    fc = FcGguf(N, K, "q6_k", w, experts=E)
    A = torch.zeros((T, K), dtype=torch.float16, device="cuda")
    ids = torch.zeros((T, top_k), dtype=torch.int32, device="cuda")
    Y = torch.zeros((T, top_k, N), dtype=torch.float16, device="cuda")
    monkeypatch.setenv("FC_GGUF_TEST_FAIL_ALLOC", "workspace")
    run = lib().fc_gguf_run_grouped
    assert run(fc.handle, _p(A), T, 0, _p(ids), top_k, _p(Y), _stream()) == ENOMEM
    # the allocation-free entry point does not allocate, so it still runs
    assert lib().fc_gguf_run_grouped_noalloc(fc.handle, _p(A), T, 0, _p(ids), top_k, _p(Y), _stream()) == 0
    monkeypatch.delenv("FC_GGUF_TEST_FAIL_ALLOC")
    assert run(fc.handle, _p(A), T, 0, _p(ids), top_k, _p(Y), _stream()) == 0
