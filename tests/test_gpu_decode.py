"""GPU parity of the decode path (M < 8, and f32 activations at any M) against
the CPU oracle; input ranks and row counts that change between calls.

Bit-exact: the int8 activation quantisation (codes, scales, group sums), the
integer sub-block dot sums, and the device weight layout (Q6_K plane regroup
plus the 16-row x 4-block tiling).  Outputs: max
relative error <= 1e-3 against the oracle's exact emulation of the int8 path
(metric max |y-r| / max(|r|, rms(r))).
"""

import numpy as np
import pytest

from gguf_quant_block_amd import synth
from oracle import fc as ofc
from oracle import kquant as okq
from helpers import DECODE_TOL, PREFILL_TOL, case, expected_device_bytes, extreme_scales, check_fro, guarded, maxrel, relfro, tile_bytes as _tile

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


# ------------------------------------------------------------ quantisation --

def _special_rows(K):
    g = np.random.default_rng(5)
    A = g.standard_normal((6, K)).astype(np.float16)
    A[0, :32] = 0                                                     # zero group
    A[1, :32] = np.array([(k - 16) / 16 for k in range(32)])           # exact ties
    A[2, 32:64] = np.float16(6e-8)                                    # f16 subnormals
    A[3, 64:96] = np.float16(65504) * np.sign(A[3, 64:96])            # largest f16
    A[4] *= np.float16(1e-3)
    A[5, 96:128] = np.float16(-1.0)                                   # constant group
    return A


@pytest.mark.parametrize("M,K", [(1, 256), (3, 3072), (7, 8192), (6, 512)])
def test_quantize_bit_exact(gpu_lib, M, K):
    from gguf_quant_block_amd.binding import debug_quantize
    A = synth.normal_f16((M, K), synth.rng(50, K, 1))
    if M == 6:
        A = _special_rows(K)
    qa, s, T, H = (_host(x) for x in debug_quantize(_dev(A)))
    qa0, s0, T0 = ofc.quantize_act(A)
    assert np.array_equal(qa, qa0)
    assert np.array_equal(s.view(np.uint32), s0.view(np.uint32))
    assert np.array_equal(T, T0)
    # the 16-value half sums the Q6_K GEMV takes its -32 offset from: the
    # oracle's codes summed per half group
    assert np.array_equal(H, qa0.reshape(A.shape[0], -1, 16).astype(np.int64).sum(axis=2))


# ---------------------------------------------------------------- regroup --

@pytest.mark.parametrize("N,K", [(3, 768), (512, 2048), (77, 1280), (40, 3072)])
def test_device_layout_bytes(gpu_lib, N, K):
    for i, qtype in enumerate(QTYPES):
        w = synth.blocks(qtype, N, K, synth.rng(51, N + i, 0))
        got = _host(_fc(w, qtype, N, K).debug_weights())
        assert np.array_equal(got, expected_device_bytes(w, qtype, N, K)), qtype


def test_layout_helper_is_a_permutation():
    # the expected-bytes helper itself: every canonical byte appears exactly
    # once, and piece p of block (n, kb) lands at ((t*P + p)*64 + l)*16 with
    # t = (n//16)*(KBp//4) + kb//4 and l = (kb%4)*16 + n%16
    N, KB, P = 37, 7, 11
    idx = np.arange(N * KB * 16 * P, dtype=np.int64).reshape(N * KB, 16 * P)
    x = _tile(idx, N, KB, P, fill=-1)
    Np, KBp = 48, 8
    assert x.size == Np * KBp * 16 * P
    assert np.array_equal(np.sort(x[x >= 0]), np.arange(N * KB * 16 * P))
    for n, kb, p in [(0, 0, 0), (5, 3, 3), (15, 6, 10), (16, 0, 0), (36, 4, 7), (20, 5, 1)]:
        t = (n // 16) * (KBp // 4) + kb // 4
        l = (kb % 4) * 16 + n % 16
        o = ((t * P + p) * 64 + l) * 16
        assert np.array_equal(x[o:o + 16], idx[n * KB + kb, 16 * p:16 * p + 16])
    w = synth.q5k_blocks(N, KB * 256, synth.rng(51, 0, 1))
    assert np.array_equal(expected_device_bytes(w, "q5_k", N, KB * 256)[x >= 0], w.reshape(-1)[x[x >= 0]])


# --------------------------------------------------------------- int sums --

@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M,N,K", [(1, 512, 2048), (7, 37, 768), (4, 16, 8192), (2, 100, 3072), (5, 24, 1024)])
def test_int_dots_bit_exact(gpu_lib, qtype, M, N, K):
    w, A, _ = case(qtype, M, N, K, 52, M * N, with_r=False)
    qa, _, _ = ofc.quantize_act(A)
    S = _host(_fc(w, qtype, N, K).debug_int_dots(_dev(qa)))
    assert np.array_equal(S.astype(np.int64), ofc.int_dots(qa, w, qtype))


# ----------------------------------------------------------------- GEMV ----

@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("N,K", [(37, 768), (512, 2048), (100, 3072), (24, 8192)])
def test_gemv_parity(gpu_lib, qtype, M, N, K):
    import torch
    with_r = (M + N) % 2 == 0
    w, A, R = case(qtype, M, N, K, 53, 100 * M + N, with_r=with_r)
    # Y inside guard bytes: no store past it
    Yd, ok = guarded((M, N), torch.float16, seed=M + N)
    _fc(w, qtype, N, K)(_dev(A), None if R is None else _dev(R), out=Yd)
    ok()
    ref = ofc.fc_ref_int8(A, w, qtype, R)
    assert maxrel(_host(Yd).astype(np.float64), ref) <= DECODE_TOL


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M", [1, 5])
def test_gemv_extreme_scales(gpu_lib, qtype, M):
    N, K = 96, 2048
    w, A, R = case(qtype, M, N, K, 65, M)
    w = extreme_scales(w, qtype, M)
    y = _host(_fc(w, qtype, N, K)(_dev(A), _dev(R)))
    assert maxrel(y, ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL


@pytest.mark.parametrize("qtype", QTYPES)
def test_gemv_in_place_residual(gpu_lib, qtype):
    import torch
    M, N, K = 3, 70, 512
    w, A, R = case(qtype, M, N, K, 54, 0)
    Rd, ok = guarded((M, N), torch.float16, fill=R, seed=3)
    fcg = _fc(w, qtype, N, K)
    fcg(_dev(A), Rd, out=Rd)
    ok()
    assert maxrel(_host(Rd), ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL


@pytest.mark.parametrize("qtype", QTYPES)
def test_forced_decode_for_larger_m(gpu_lib, qtype):
    M, N, K = 16, 40, 512
    w, A, R = case(qtype, M, N, K, 55, 0)
    fcg = _fc(w, qtype, N, K)
    fcg.set_path("decode")
    y = _host(fcg(_dev(A), _dev(R)))
    assert maxrel(y, ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL


@pytest.mark.parametrize("qtype", ["q5_k", "q6_k"])
def test_gemv_large_k_row_chunks(gpu_lib, qtype):
    # K = 16384: seven rows' quantised activations exceed one CU's LDS, so the
    # library takes the rows in chunks of six and one
    M, N, K = 7, 24, 16384
    w, A, R = case(qtype, M, N, K, 57, 0)
    y = _host(_fc(w, qtype, N, K)(_dev(A), _dev(R)))
    assert maxrel(y, ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL


def test_m_zero_is_noop(gpu_lib):
    import torch
    w, _, _ = case("q6_k", 1, 32, 256, 56, 0)
    fcg = _fc(w, "q6_k", 32, 256)
    Y = torch.full((0, 32), 7.0, dtype=torch.float16, device="cuda")
    fcg(torch.empty((0, 256), dtype=torch.float16, device="cuda"), out=Y)
    assert Y.shape == (0, 32)


# --------------------------------------- full-size layers, sampled outputs --
# Phi-3.5-mini layer shapes at the decode row counts; the whole matrix runs on
# the GPU in the benchmark's launch configuration, and a random sample of
# output columns is checked against the oracle restricted to those W rows.

FULL = [("q5_k", name, M) for name in synth.PHI35_LAYERS for M in (1, 2, 4, 7)]
FULL += [("q6_k", name, M) for name in synth.PHI35_LAYERS for M in (1, 4)]
FULL += [("q6_k", "output", M) for M in (1, 4)]
FULL += [("q4_k", name, M) for name in synth.PHI35_LAYERS for M in (1, 3)]


@pytest.mark.parametrize("qtype,name,M", FULL)
def test_gemv_full_size_sampled(gpu_lib, qtype, name, M):
    N, K = synth.PHI35_OUTPUT if name == "output" else synth.PHI35_LAYERS[name]
    with_r = name != "output"
    cfg = {"q5_k": 1, "q6_k": 2, "q4_k": 5}[qtype]
    w, A, R = case(qtype, M, N, K, cfg, list(synth.PHI35_LAYERS).index(name) if with_r else 9, with_r)
    y = _host(_fc(w, qtype, N, K)(_dev(A), None if R is None else _dev(R)))
    cols = np.sort(np.random.default_rng(N + M).choice(N, size=min(N, 192), replace=False))
    cols = np.unique(np.concatenate([cols, [0, N - 1]]))
    ref = ofc.fc_ref_int8(A, w[cols], qtype, None if R is None else R[:, cols])
    assert maxrel(y[:, cols], ref) <= DECODE_TOL


# ------------------------------------------------------ f32 activations ----
# OpenVINO PR #39119, section Implementation: f32 activations take the int8
# quantisation + GEMV path at every row count.

def _special_rows_f32(K):
    g = np.random.default_rng(6)
    A = g.standard_normal((6, K)).astype(np.float32)
    A[0, :32] = 0                                                     # zero group
    A[1, :32] = np.array([(k - 16) / 16 for k in range(32)])           # exact ties
    A[2, :32] *= np.float32(1e-37)                                    # 127/amax overflows: zero group
    A[2, 32:64] = np.float32(5e-37) * np.array([(k - 16) / 16 for k in range(32)])  # subnormal s
    A[3, 64:96] *= np.float32(1e30)                                   # beyond the f16 range
    A[4, 7] = np.float32(1e-40)                                       # subnormal value
    A[5, 96:128] = np.float32(-3.0)                                   # constant group
    return A


@pytest.mark.parametrize("M,K", [(1, 256), (3, 3072), (7, 8192), (6, 512)])
def test_quantize_f32_bit_exact(gpu_lib, M, K):
    from gguf_quant_block_amd.binding import debug_quantize
    A = synth.normal_f32((M, K), synth.rng(57, K, 1))
    if M == 6:
        A = _special_rows_f32(K)
    qa, s, T, H = (_host(x) for x in debug_quantize(_dev(A)))
    qa0, s0, T0 = ofc.quantize_act(A)
    assert np.array_equal(qa, qa0)
    assert np.array_equal(s.view(np.uint32), s0.view(np.uint32))
    assert np.array_equal(T, T0)
    # the 16-value half sums the Q6_K GEMV takes its -32 offset from: the
    # oracle's codes summed per half group
    assert np.array_equal(H, qa0.reshape(A.shape[0], -1, 16).astype(np.int64).sum(axis=2))


def _case_f32(qtype, M, N, K, idx, with_r):
    w = synth.blocks(qtype, N, K, synth.rng(58, idx, synth.TAG_BLOCKS))
    A = synth.normal_f32((M, K), synth.rng(58, idx, synth.TAG_A))
    R = synth.normal_f32((M, N), synth.rng(58, idx, synth.TAG_R)) if with_r else None
    return w, A, R


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("M", [1, 4, 7, 8, 20])
@pytest.mark.parametrize("N,K", [(37, 768), (512, 2048), (24, 8192)])
def test_gemv_f32_parity(gpu_lib, qtype, M, N, K):
    import torch
    with_r = (M + N) % 2 == 1
    w, A, R = _case_f32(qtype, M, N, K, 100 * M + N, with_r)
    y = _fc(w, qtype, N, K)(_dev(A), None if R is None else _dev(R))
    assert y.dtype == torch.float32
    assert maxrel(_host(y), ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL


def test_f32_ignores_forced_prefill_path(gpu_lib):
    M, N, K = 12, 64, 512
    w, A, R = _case_f32("q5_k", M, N, K, 1, True)
    fcg = _fc(w, "q5_k", N, K)
    y0 = _host(fcg(_dev(A), _dev(R)))
    fcg.set_path("prefill")
    y1 = _host(fcg(_dev(A), _dev(R)))
    assert np.array_equal(y0, y1)
    assert maxrel(y1, ofc.fc_ref_int8(A, w, "q5_k", R)) <= DECODE_TOL


def test_f32_in_place_residual(gpu_lib):
    M, N, K = 3, 96, 1024
    w, A, R = _case_f32("q6_k", M, N, K, 2, True)
    Rd = _dev(R)
    _fc(w, "q6_k", N, K)(_dev(A), Rd, out=Rd)
    assert maxrel(_host(Rd), ofc.fc_ref_int8(A, w, "q6_k", R)) <= DECODE_TOL


# ---------------------------------------- input ranks and changing row count --

@pytest.mark.parametrize("lead", [(2, 3), (4, 5), (1, 1, 2), (2, 2, 16)])
def test_nd_inputs(gpu_lib, lead):
    qtype, N, K = "q4_k", 80, 512
    M = int(np.prod(lead))
    w, A, R = case(qtype, M, N, K, 59, M)
    A_nd, R_nd = A.reshape(*lead, K), R.reshape(*lead, N)
    y = _host(_fc(w, qtype, N, K)(_dev(A_nd), _dev(R_nd)))
    assert y.shape == (*lead, N)
    ref = ofc.fc_ref_int8(A, w, qtype, R) if M < 8 else ofc.fc_gguf_ref(A, w, qtype, R)
    err = maxrel(y.reshape(M, N), ref) if M < 8 else relfro(y.reshape(M, N), ref)
    assert err <= (DECODE_TOL if M < 8 else PREFILL_TOL)


def test_row_count_changes_between_calls(gpu_lib):
    # one handle, M changing from call to call across both paths and the
    # split-K workspace growth
    qtype, N, K = "q6_k", 256, 4096
    fcg = None
    for i, M in enumerate([1, 9, 3, 64, 2, 200, 7, 8, 1]):
        w, A, R = case(qtype, M, N, K, 59, 1000, with_r=True)
        A = synth.normal_f16((M, K), synth.rng(59, 2000 + i, 1))
        R = synth.normal_f16((M, N), synth.rng(59, 2000 + i, 2))
        if fcg is None:
            fcg = _fc(w, qtype, N, K)
        y = _host(fcg(_dev(A), _dev(R)))
        if M < 8:
            assert maxrel(y, ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL, M
        else:
            check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))
