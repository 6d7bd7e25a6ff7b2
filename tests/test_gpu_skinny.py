"""GPU parity of the few-row prefill kernel (FC_GGUF_PREFILL_KERNEL=skinny)
against the float64 oracle, with the prefill bar (relative Frobenius error
<= 2e-3 and the element guard).

The kernel keeps each row tile's whole K in one workgroup (waves split K by
4-block tile and quarter, as the decode GEMV does) and runs the f16 matrix
cores on fragments whose K positions are the lanes' own blocks.  Covered:
one and two 16-row halves (M up to 32), ragged M and N, K with padding blocks
(K / 256 not a multiple of 4), one super-block, waves looping over several
tiles (K / 256 > 16), in place, no residual, extreme scales, guard bytes
around Y, the persistent loop over row tiles, the fallback where the rows
do not fit the LDS, and the full-size shapes on sampled columns; also that
the default picks this kernel exactly where it fits, and the loader-wave
tile forced at those row counts.
"""

import numpy as np
import pytest

from gguf_quant_block_amd import synth
from oracle import fc as ofc
from oracle import kquant as okq
from helpers import case, check_fro, extreme_scales, guarded, stratified_cols

pytestmark = pytest.mark.gpu

QTYPES = ["q4_k", "q5_k", "q6_k"]


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _fc(w, qtype, N, K, kernel, monkeypatch):
    # FC_GGUF_PREFILL_KERNEL is read when the handle is created
    from gguf_quant_block_amd.binding import FcGguf
    monkeypatch.setenv("FC_GGUF_PREFILL_KERNEL", kernel)
    f = FcGguf(N, K, qtype, w)
    monkeypatch.delenv("FC_GGUF_PREFILL_KERNEL", raising=False)
    f.set_path("prefill")
    return f


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M,N,K", [
    (8, 80, 256),        # one super-block, one row-tile group of 4 waves
    (16, 128, 512),      # two blocks per row: half of each tile is padding
    (9, 257, 768),       # three blocks, ragged rows
    (15, 1000, 1024),    # one full tile
    (17, 200, 2048),     # two 16-row halves
    (32, 96, 2048),
    (24, 130, 3072),     # 12 waves
    (12, 64, 4352),      # 17 blocks: 16 waves, some over two tiles, padding
    (8, 48, 8192),       # 16 waves over 8 tiles: two tiles each
    (1, 33, 1024),       # the prefill path forced at M < 8
    (3, 500, 2048),
])
def test_skinny_forced(gpu_lib, monkeypatch, qtype, M, N, K):
    w, A, R = case(qtype, M, N, K, 80, M * 7 + N)
    f = _fc(w, qtype, N, K, "skinny", monkeypatch)
    y = _host(f(_dev(A), _dev(R)))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", QTYPES)
def test_skinny_runs_and_differs_from_tile(gpu_lib, monkeypatch, qtype):
    # the two kernels sum K in different orders: both meet the bar, and their
    # outputs are not bit-identical (so the forced kernel is the one that ran)
    M, N, K = 16, 512, 2048
    w, A, R = case(qtype, M, N, K, 81, 0)
    ref = ofc.fc_gguf_ref(A, w, qtype, R)
    ys = {}
    for kernel in ("skinny", "dma"):
        ys[kernel] = _host(_fc(w, qtype, N, K, kernel, monkeypatch)(_dev(A), _dev(R)))
        check_fro(ys[kernel], ref)
    assert not np.array_equal(ys["skinny"], ys["dma"])


@pytest.mark.parametrize("qtype", QTYPES)
def test_skinny_deterministic_and_guarded(gpu_lib, monkeypatch, qtype):
    import torch
    M, N, K = 13, 300, 3072
    w, A, R = case(qtype, M, N, K, 82, 1)
    f = _fc(w, qtype, N, K, "skinny", monkeypatch)
    Y, check = guarded((M, N), torch.float16, seed=5)
    f(_dev(A), _dev(R), out=Y)
    y1 = _host(Y).copy()
    check()
    f(_dev(A), _dev(R), out=Y)
    assert np.array_equal(_host(Y), y1)
    check()
    check_fro(y1, ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", QTYPES)
def test_skinny_in_place_no_residual_extreme_scales(gpu_lib, monkeypatch, qtype):
    M, N, K = 20, 160, 1536
    w, A, R = case(qtype, M, N, K, 83, 2)
    w = extreme_scales(w, qtype, 12)
    f = _fc(w, qtype, N, K, "skinny", monkeypatch)
    Rd = _dev(R)
    f(_dev(A), Rd, out=Rd)
    y = _host(Rd)
    assert np.all(np.isfinite(y))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))
    y0 = _host(f(_dev(A)))
    check_fro(y0, ofc.fc_gguf_ref(A, w, qtype, None))


@pytest.mark.parametrize("qtype", ["q5_k", "q6_k"])
def test_skinny_falls_back_where_rows_do_not_fit(gpu_lib, monkeypatch, qtype):
    # 16 rows of K = 8192 halves do not fit the LDS: the loader-wave tile runs
    M, N, K = 16, 64, 8192
    w, A, R = case(qtype, M, N, K, 84, 3)
    ys = {}
    for kernel in ("skinny", "dma"):
        ys[kernel] = _host(_fc(w, qtype, N, K, kernel, monkeypatch)(_dev(A), _dev(R)))
    assert np.array_equal(ys["skinny"], ys["dma"])
    check_fro(ys["skinny"], ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", ["q5_k", "q6_k"])
@pytest.mark.parametrize("M", [8, 16, 32])
@pytest.mark.parametrize("shape", ["qkv", "down", "p0", "p1", "output"])
def test_skinny_full_size_sampled(gpu_lib, monkeypatch, qtype, M, shape):
    # the Phi-3.5 projections, the output projection [32064, 3072] and the
    # prefill shapes at full size (more row tiles than workgroups: the
    # persistent loop), sampled output columns
    if shape == "output":
        N, K = synth.PHI35_OUTPUT
    elif shape in synth.PHI35_LAYERS:
        N, K = synth.PHI35_LAYERS[shape]
    else:
        N, K = synth.PREFILL_SHAPES[int(shape[1])]
    w, A, R = case(qtype, M, N, K, 85, M + len(shape))
    y = _host(_fc(w, qtype, N, K, "skinny", monkeypatch)(_dev(A), _dev(R)))
    cols = stratified_cols(N, N + M)
    ref = ofc.fc_ref(A, okq.dequantize(w[cols], qtype), R[:, cols])
    check_fro(y[:, cols], ref)


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M,N,K", [(8, 200, 2048), (16, 130, 1024), (17, 64, 3072), (32, 257, 512)])
def test_loader_wave_tile_forced_at_few_rows(gpu_lib, monkeypatch, qtype, M, N, K):
    # where the default now takes the few-row kernel, the loader-wave tile
    # (16- and 32-row tiles with split-K grids) stays covered when forced
    w, A, R = case(qtype, M, N, K, 86, M + N)
    f = _fc(w, qtype, N, K, "dma", monkeypatch)
    y = _host(f(_dev(A), _dev(R)))
    check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))


@pytest.mark.parametrize("qtype", ["q5_k"])
def test_default_takes_skinny_where_it_fits(gpu_lib, monkeypatch, qtype):
    # AUTO (no kernel forced) gives the few-row kernel's bits where its rows
    # fit, and the loader-wave tile's where they do not
    from gguf_quant_block_amd.binding import FcGguf
    for M, N, K, kernel in [(16, 256, 2048, "skinny"), (33, 256, 2048, "dma"), (16, 64, 8192, "dma")]:
        w, A, R = case(qtype, M, N, K, 87, M + K)
        monkeypatch.delenv("FC_GGUF_PREFILL_KERNEL", raising=False)
        y_auto = _host(FcGguf(N, K, qtype, w)(_dev(A), _dev(R)))
        y_forced = _host(_fc(w, qtype, N, K, kernel, monkeypatch)(_dev(A), _dev(R)))
        assert np.array_equal(y_auto, y_forced), (M, N, K)
