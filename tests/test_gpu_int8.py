"""GPU parity of the int8 matrix-core prefill variant (FC_GGUF_PATH_INT8).

The variant quantises the activations with the decode path's per-32 routine,
sums codes times weight codes exactly on the int8 matrix cores and applies
the scales in f32 per group, so its result is the int8 emulation of the FC
(oracle.fc.fc_ref_int8) at any row count.  Metric and bar: the decode path's,
max |y - r| / max(|r|, rms(r)) <= 1e-3.  (Against the fp64 FC the per-32 int8
activations alone leave about 5e-3 relative Frobenius error, outside the f16
prefill path's 2e-3 bar; the variant is held to the int8 emulation instead.)
"""

import numpy as np
import pytest

from gguf_quant_block_amd import synth
from oracle import fc as ofc
from helpers import DECODE_TOL, case, extreme_scales, maxrel, relfro

pytestmark = pytest.mark.gpu

QTYPES = ["q4_k", "q5_k", "q6_k"]


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _fc_int8(w, qtype, N, K):
    from gguf_quant_block_amd.binding import FcGguf
    f = FcGguf(N, K, qtype, w)
    f.set_path("int8")
    return f


# every tile size (M = 1 .. 200 -> 16..128-row tiles), split-K grids (small
# M x N), ragged M and N, K with a padded last tile of blocks (1280, 768)
SHAPES = [(16, 512, 2048), (1, 37, 768), (8, 100, 3072), (37, 300, 1280), (130, 64, 512),
          (200, 256, 8192), (64, 1000, 2048), (8, 48, 256), (24, 64, 14336)]


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_int8_parity(gpu_lib, qtype, M, N, K):
    with_r = (M + N) % 2 == 0
    w, A, R = case(qtype, M, N, K, 80, M * 7 + N, with_r=with_r)
    y = _host(_fc_int8(w, qtype, N, K)(_dev(A), None if R is None else _dev(R)))
    assert maxrel(y, ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M", [9, 64])
def test_int8_extreme_scales(gpu_lib, qtype, M):
    N, K = 160, 2048
    w, A, R = case(qtype, M, N, K, 81, M)
    w = extreme_scales(w, qtype, M)
    y = _host(_fc_int8(w, qtype, N, K)(_dev(A), _dev(R)))
    assert maxrel(y, ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL


@pytest.mark.parametrize("qtype", QTYPES)
def test_int8_in_place_residual(gpu_lib, qtype):
    M, N, K = 24, 96, 1024
    w, A, R = case(qtype, M, N, K, 82, 0)
    Rd = _dev(R)
    _fc_int8(w, qtype, N, K)(_dev(A), Rd, out=Rd)
    assert maxrel(_host(Rd), ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL


def test_int8_row_count_changes(gpu_lib):
    # the workspace grows with M on one handle; results stay exact
    qtype, N, K = "q5_k", 256, 1024
    w, _, _ = case(qtype, 1, N, K, 83, 0, with_r=False)
    f = _fc_int8(w, qtype, N, K)
    for M in (16, 300, 8, 1):
        _, A, R = case(qtype, M, N, K, 83, M)
        y = _host(f(_dev(A), _dev(R)))
        assert maxrel(y, ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL, M


def test_int8_matches_decode_path(gpu_lib):
    # the decode path computes the same numbers (other summation order)
    from gguf_quant_block_amd.binding import FcGguf
    qtype, M, N, K = "q6_k", 5, 200, 3072
    w, A, R = case(qtype, M, N, K, 84, 0)
    y8 = _host(_fc_int8(w, qtype, N, K)(_dev(A), _dev(R))).astype(np.float64)
    yd = _host(FcGguf(N, K, qtype, w)(_dev(A), _dev(R))).astype(np.float64)
    assert maxrel(y8, yd) <= 2 * DECODE_TOL


def test_int8_error_is_quantisation_sized(gpu_lib):
    # against the fp64 FC the int8 path carries the activation quantisation
    # error (a few 1e-3), which the f16 prefill path does not
    qtype, M, N, K = "q5_k", 64, 256, 2048
    w, A, R = case(qtype, M, N, K, 85, 0, with_r=False)
    y = _host(_fc_int8(w, qtype, N, K)(_dev(A)))
    err = relfro(y, ofc.fc_gguf_ref(A, w, qtype, None))
    assert 1e-3 < err < 2e-2


# full-size prefill shapes at the benchmark's row counts, sampled columns
SWEEP = [(q, s, M) for q in QTYPES for s in range(2) for M in (64, 512)]


@pytest.mark.parametrize("qtype,shape,M", SWEEP)
def test_int8_full_size_sampled(gpu_lib, qtype, shape, M):
    N, K = synth.PREFILL_SHAPES[shape]
    w, A, R = case(qtype, M, N, K, 3, 10 * shape + synth.PREFILL_MS.index(M))
    y = _host(_fc_int8(w, qtype, N, K)(_dev(A), _dev(R)))
    cols = np.sort(np.random.default_rng(N + M).choice(N, size=128, replace=False))
    cols = np.unique(np.concatenate([cols, [0, N - 1]]))
    ref = ofc.fc_ref_int8(A, w[cols], qtype, R[:, cols])
    assert maxrel(y[:, cols], ref) <= DECODE_TOL
