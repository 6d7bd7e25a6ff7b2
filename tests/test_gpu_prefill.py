"""GPU parity of the prefill path (M >= 8) against the float64 oracle.

Relative Frobenius error <= 2e-3 against Y = A.W^T + R with W decoded exactly,
and no element off by more than 1e-2 of max(|y|, rms(y)).
Covers every tile step of the M ladder, ragged M and N tails, split-K grids,
the forced prefill path at M < 8, and the full-size prefill shapes at every
M on sampled output columns.
"""

import numpy as np
import pytest

from gguf_quant_block_amd import synth
from oracle import fc as ofc
from oracle import kquant as okq
from helpers import PREFILL_TOL, case, check_fro, extreme_scales, guarded, relfro, stratified_cols

pytestmark = pytest.mark.gpu

QTYPES = ["q4_k", "q5_k", "q6_k"]


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _fc(w, qtype, N, K):
    from gguf_quant_block_amd.binding import FcGguf
    return FcGguf(N, K, qtype, w)


@pytest.mark.parametrize("qtype", QTYPES)
def test_small_config_m16(gpu_lib, qtype):
    # single Q6_K/Q5_K FC N=512 K=2048 at M=16, no residual
    M, N, K = 16, 512, 2048
    w, A, _ = case(qtype, M, N, K, 0, 1, with_r=False)
    y = _host(_fc(w, qtype, N, K)(_dev(A)))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype))


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M,N,K", [(8, 80, 256), (37, 200, 768), (130, 384, 1024), (300, 64, 512),
                                   (64, 128, 2048), (17, 1000, 512), (24, 64, 14336)])
def test_prefill_ragged(gpu_lib, qtype, M, N, K):
    import torch
    w, A, R = case(qtype, M, N, K, 60, M * 7 + N)
    # Y and R inside guard bytes: no store past Y, nothing written to R
    Yd, y_ok = guarded((M, N), torch.float16, seed=M)
    Rd, r_ok = guarded((M, N), torch.float16, fill=R, seed=N)
    _fc(w, qtype, N, K)(_dev(A), Rd, out=Yd)
    y_ok()
    r_ok()
    assert np.array_equal(_host(Rd).view(np.uint16), R.view(np.uint16))
    check_fro(_host(Yd), ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M", [1, 3, 7])
def test_forced_prefill_for_small_m(gpu_lib, qtype, M):
    N, K = 96, 768
    w, A, R = case(qtype, M, N, K, 61, M)
    fcg = _fc(w, qtype, N, K)
    fcg.set_path("prefill")
    y = _host(fcg(_dev(A), _dev(R)))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", QTYPES)
def test_prefill_in_place_residual(gpu_lib, qtype):
    import torch
    M, N, K = 40, 130, 512
    w, A, R = case(qtype, M, N, K, 62, 0)
    Rd, ok = guarded((M, N), torch.float16, fill=R, seed=5)
    _fc(w, qtype, N, K)(_dev(A), Rd, out=Rd)
    ok()
    check_fro(_host(Rd), ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M", [16, 200])
def test_prefill_extreme_scales(gpu_lib, qtype, M):
    # scales at the limits of each format (Q6_K: -128 and 127) keep every
    # intermediate of the f16 decode finite
    N, K = 160, 1024
    w, A, R = case(qtype, M, N, K, 64, M)
    w = extreme_scales(w, qtype, M)
    y = _host(_fc(w, qtype, N, K)(_dev(A), _dev(R)))
    assert np.all(np.isfinite(y))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M,N,K,with_r", [(1, 96, 512, True), (37, 200, 768, False), (512, 384, 2048, True)])
def test_scratch_path_parity(gpu_lib, qtype, M, N, K, with_r):
    # the dequantise-once comparison path (f16 weights + library GEMM)
    w, A, R = case(qtype, M, N, K, 66, M + N, with_r=with_r)
    fcg = _fc(w, qtype, N, K)
    fcg.set_path("scratch")
    y = _host(fcg(_dev(A), None if R is None else _dev(R)))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))


def test_scratch_path_in_place_and_extreme_scales(gpu_lib):
    M, N, K = 24, 128, 1024
    w, A, R = case("q6_k", M, N, K, 67, 0)
    w = extreme_scales(w, "q6_k", 9)
    fcg = _fc(w, "q6_k", N, K)
    fcg.set_path("scratch")
    Rd = _dev(R)
    fcg(_dev(A), Rd, out=Rd)
    check_fro(_host(Rd), ofc.fc_gguf_ref(A, w, "q6_k", R))


def test_prefill_error_is_f16_sized(gpu_lib):
    # the error is the expected f16-rounding size, far inside the tolerance
    M, N, K = 256, 256, 2048
    w, A, R = case("q6_k", M, N, K, 63, 0)
    err = relfro(_host(_fc(w, "q6_k", N, K)(_dev(A), _dev(R))), ofc.fc_gguf_ref(A, w, "q6_k", R))
    assert err < 1e-3


# full-size prefill sweep: both qtypes, both weight shapes, every M step;
# sampled output columns against the oracle restricted to those W rows
SWEEP = [(q, s, M) for q in QTYPES for s in range(2) for M in synth.PREFILL_MS]


@pytest.mark.parametrize("qtype,shape,M", SWEEP)
def test_prefill_full_size_sampled(gpu_lib, qtype, shape, M):
    N, K = synth.PREFILL_SHAPES[shape]
    w, A, R = case(qtype, M, N, K, 3, 10 * shape + synth.PREFILL_MS.index(M))
    y = _host(_fc(w, qtype, N, K)(_dev(A), _dev(R)))
    # every 128-column weight tile: its first and last column and two inside
    cols = stratified_cols(N, N + M)
    ref = ofc.fc_ref(A, okq.dequantize(w[cols], qtype), R[:, cols])
    check_fro(y[:, cols], ref)


def test_auto_row_threshold_from_env(gpu_lib, monkeypatch):
    # AUTO sends M < 8 rows to the decode path (the page's threshold) unless
    # FC_GGUF_DECODE_ROWS, read when the handle is created, says otherwise
    qtype, M, N, K = "q5_k", 6, 256, 1024
    w, A, R = case(qtype, M, N, K, 91, 0)
    monkeypatch.delenv("FC_GGUF_PATH", raising=False)
    got = {}
    for env in (None, "5", "junk"):
        if env is None:
            monkeypatch.delenv("FC_GGUF_DECODE_ROWS", raising=False)
        else:
            monkeypatch.setenv("FC_GGUF_DECODE_ROWS", env)
        got[env] = _host(_fc(w, qtype, N, K)(_dev(A), _dev(R)))
    monkeypatch.delenv("FC_GGUF_DECODE_ROWS", raising=False)
    forced = {}
    for p in ("decode", "prefill"):
        f = _fc(w, qtype, N, K)
        f.set_path(p)
        forced[p] = _host(f(_dev(A), _dev(R)))
    assert not np.array_equal(forced["decode"], forced["prefill"])
    assert np.array_equal(got[None], forced["decode"])
    assert np.array_equal(got["junk"], forced["decode"])
    assert np.array_equal(got["5"], forced["prefill"])


def _fc_kernel(w, qtype, N, K, kernel, monkeypatch):
    # FC_GGUF_PREFILL_KERNEL is read when the handle is created
    monkeypatch.setenv("FC_GGUF_PREFILL_KERNEL", kernel)
    f = _fc(w, qtype, N, K)
    monkeypatch.delenv("FC_GGUF_PREFILL_KERNEL", raising=False)
    return f


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M,N,K", [(8, 80, 256), (16, 128, 512), (130, 200, 768), (129, 257, 1024),
                                   (256, 384, 2048), (300, 64, 512), (40, 1000, 4096), (513, 130, 256)])
def test_decode_once_tile_forced(gpu_lib, monkeypatch, qtype, M, N, K):
    # the decode-once (producer / consumer) tile at any row count: ragged
    # activation and weight tiles, split-K grids, a single super-block
    w, A, R = case(qtype, M, N, K, 68, M * 3 + N)
    f = _fc_kernel(w, qtype, N, K, "lds", monkeypatch)
    y = _host(f(_dev(A), _dev(R)))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M", [256, 512])
def test_loader_wave_tile_forced_at_large_m(gpu_lib, monkeypatch, qtype, M):
    # the loader-wave tile where AUTO would take the decode-once tile
    N, K = 384, 1024
    w, A, R = case(qtype, M, N, K, 69, M)
    f = _fc_kernel(w, qtype, N, K, "dma", monkeypatch)
    y = _host(f(_dev(A), _dev(R)))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", QTYPES)
def test_decode_once_tile_in_place_and_extreme_scales(gpu_lib, monkeypatch, qtype):
    M, N, K = 200, 256, 1024
    w, A, R = case(qtype, M, N, K, 70, 0)
    w = extreme_scales(w, qtype, 11)
    f = _fc_kernel(w, qtype, N, K, "lds", monkeypatch)
    Rd = _dev(R)
    f(_dev(A), Rd, out=Rd)
    y = _host(Rd)
    assert np.all(np.isfinite(y))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", ["q5_k", "q6_k"])
@pytest.mark.parametrize("shape", [0, 1])
def test_decode_once_tile_full_size_sampled(gpu_lib, monkeypatch, qtype, shape):
    # the decode-once tile on the full-size prefill shapes at M = 512 (a split-K
    # grid on [2048, 8192]), sampled output columns
    M = 512
    N, K = synth.PREFILL_SHAPES[shape]
    w, A, R = case(qtype, M, N, K, 71, shape)
    y = _host(_fc_kernel(w, qtype, N, K, "lds", monkeypatch)(_dev(A), _dev(R)))
    cols = stratified_cols(N, N + 7)
    ref = ofc.fc_ref(A, okq.dequantize(w[cols], qtype), R[:, cols])
    check_fro(y[:, cols], ref)


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("tile", ["1,1", "2,1", "2,2", "4,2", "4,4", "8,1", "8,8", "1,8",
                                  "3,2", "4,3", "8,64"])
def test_loader_wave_tile_forced_shapes(gpu_lib, monkeypatch, qtype, tile):
    # FC_GGUF_TILE=<mt>,<splits> (read when the handle is created) forces the
    # loader-wave tile's row count and K split, whatever the row-count rule
    # picks: every tile height, split-K from none to one stage per split, on
    # ragged M and N; malformed values ("3,2", "4,3") and a split count that
    # would leave parts of K empty ("8,64" over 8 stages) fall back to the rule
    M, N, K = 70, 200, 1024
    w, A, R = case(qtype, M, N, K, 71, len(tile))
    monkeypatch.setenv("FC_GGUF_TILE", tile)
    f = _fc(w, qtype, N, K)
    monkeypatch.delenv("FC_GGUF_TILE", raising=False)
    y = _host(f(_dev(A), _dev(R)))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))
