"""GPU parity of the grouped (MoE expert) FC against the float64 oracle.

Relative Frobenius error <= 2e-3, over the whole output and per expert, so a
bug in a 1-row expert is not hidden by the hot experts.  Covers experts
spanning several ragged tiles, N tails, shared
and per-pair activation rows, ids outside [0, E), empty experts, T = 0,
repeat calls, the 32- and 128-row tile variants (four and two workgroups
per CU), and the full-size
routed Q6_K expert FCs (128 experts, top-8, 256 tokens, Zipf 1.1 routing) on
sampled experts.  The bucketing alone is compared with the oracle's exactly:
offsets and tile list element by element, the pair list bucket by bucket as
sets (the kernel's order inside a bucket is free).
"""

import numpy as np
import pytest

from gguf_quant_block_amd import synth
from oracle import fc as ofc
from oracle import kquant as okq
from helpers import ELEM_GUARD, PREFILL_TOL, check_fro, expected_device_bytes, extreme_scales, guarded, maxrel, relfro

pytestmark = pytest.mark.gpu

QTYPES = ["q4_k", "q5_k", "q6_k"]


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _moe_case(qtype, E, N, K, T, top_k, a_per_slot, cfg, idx, s=1.1):
    w = synth.blocks(qtype, E * N, K, synth.rng(cfg, idx, synth.TAG_BLOCKS)).reshape(E, N, -1)
    shape = (T, top_k, K) if a_per_slot else (T, K)
    A = synth.normal_f16(shape, synth.rng(cfg, idx, synth.TAG_A))
    ids = synth.moe_routing(T, E, top_k, synth.rng(cfg, idx, synth.TAG_ROUTING), s=s)
    return w, A, ids


def _run(w, qtype, A, ids, a_per_slot, out=None):
    from gguf_quant_block_amd.binding import FcGguf
    E, N = w.shape[:2]
    K = A.shape[-1]
    fc = FcGguf(N, K, qtype, w, experts=E)
    return fc, fc.grouped(_dev(A), _dev(ids), a_per_slot, out=out)


def _check_experts(y, w, qtype, A, ids, a_per_slot, experts):
    """Per-expert relative Frobenius error against the oracle on `experts`."""
    worst = 0.0
    for e in experts:
        tt, jj = np.nonzero(ids == e)
        if tt.size == 0:
            continue
        W = okq.dequantize(w[e], qtype)
        rows = A[tt, jj] if a_per_slot else A[tt]
        ref = ofc.fc_ref(rows, W)
        err = relfro(y[tt, jj], ref)
        assert err <= PREFILL_TOL, f"expert {e} ({tt.size} rows): {err:.3e}"
        assert maxrel(y[tt, jj], ref) <= ELEM_GUARD, f"expert {e}: element-wise"
        worst = max(worst, err)
    return worst


@pytest.mark.parametrize("qtype", QTYPES)
@pytest.mark.parametrize("a_per_slot", [False, True])
@pytest.mark.parametrize("E,N,K,T,top_k", [
    (8, 200, 512, 37, 2),      # 32-row tiles, N tail, sparse experts
    (4, 128, 768, 64, 2),      # 128 pairs over 4 experts: full 32-row tiles
    (16, 96, 256, 90, 4),      # several ragged tiles per hot expert
    (32, 256, 512, 5, 3),      # more experts than pairs: most experts empty
    (2, 96, 1024, 100, 2),     # dense routing: 128-row tiles
])
def test_moe_small(gpu_lib, qtype, a_per_slot, E, N, K, T, top_k):
    import torch
    w, A, ids = _moe_case(qtype, E, N, K, T, top_k, a_per_slot, 40, E * 1000 + T)
    out, ok = guarded((T, top_k, N), torch.float16, seed=E + T)
    _, y = _run(w, qtype, A, ids, a_per_slot, out=out)
    ok()
    y = _host(y)
    ref = ofc.moe_ref(A, w, qtype, ids, a_per_slot)
    check_fro(y, ref)
    _check_experts(y, w, qtype, A, ids, a_per_slot, range(E))


@pytest.mark.parametrize("qtype", QTYPES)
def test_moe_extreme_scales(gpu_lib, qtype):
    E, N, K, T, top_k = 8, 128, 512, 60, 2
    w, A, ids = _moe_case(qtype, E, N, K, T, top_k, False, 45, 0)
    w = extreme_scales(w, qtype, 3)
    _, y = _run(w, qtype, A, ids, False)
    y = _host(y)
    assert np.all(np.isfinite(y))
    _check_experts(y, w, qtype, A, ids, False, range(E))


@pytest.mark.parametrize("qtype", QTYPES)
def test_moe_single_hot_expert(gpu_lib, qtype):
    # every token routed to expert 2 in slot 0: one expert spans many tiles
    E, N, K, T, top_k = 6, 160, 512, 150, 2
    w, A, ids = _moe_case(qtype, E, N, K, T, top_k, False, 41, 0)
    ids[:, 0] = 2
    ids[:, 1] = np.where(ids[:, 1] == 2, 3, ids[:, 1])
    _, y = _run(w, qtype, A, ids, False)
    y = _host(y)
    _check_experts(y, w, qtype, A, ids, False, range(E))


@pytest.mark.parametrize("qtype", QTYPES)
def test_moe_invalid_ids_give_zero_rows(gpu_lib, qtype):
    import torch
    E, N, K, T, top_k = 8, 64, 256, 20, 2
    w, A, ids = _moe_case(qtype, E, N, K, T, top_k, False, 42, 0)
    ids[3, 1] = -1
    ids[7, 0] = E
    ids[11, 1] = 1 << 30
    out = torch.full((T, top_k, N), float("nan"), dtype=torch.float16, device="cuda")
    _, y = _run(w, qtype, A, ids, False, out=out)
    y = _host(y)
    for t, j in [(3, 1), (7, 0), (11, 1)]:
        assert np.all(y[t, j] == 0)
    assert np.all(np.isfinite(y))
    _check_experts(y, w, qtype, A, ids, False, range(E))


@pytest.mark.parametrize("qtype", QTYPES)
def test_grouped_device_layout_bytes(gpu_lib, qtype):
    # grouped handles tile every expert's matrix like a single-matrix handle
    # (16 rows x 4 blocks, rows and blocks per row padded), experts one after
    # another
    from gguf_quant_block_amd.binding import FcGguf
    E, N, K = 3, 5, 768
    w = synth.blocks(qtype, E * N, K, synth.rng(44, 0, 0)).reshape(E, N, -1)
    got = _host(FcGguf(N, K, qtype, w, experts=E).debug_weights())
    exp = [expected_device_bytes(w[e], qtype, N, K) for e in range(E)]
    per = exp[0].size
    assert got.size == E * per
    for e in range(E):
        assert np.array_equal(got[e * per:(e + 1) * per], exp[e])
    if qtype == "q6_k":
        # the plane split agrees with the oracle's regroup
        planes = okq.q6k_regroup(w[0])
        assert np.array_equal(np.sort(exp[0][:16 * 4 * 128]), np.sort(np.concatenate(
            [planes[:128 * N * 3], np.zeros(128 * (64 - N * 3), np.uint8)])))


def test_moe_empty_and_repeat(gpu_lib):
    import torch
    qtype = "q6_k"
    E, N, K, T, top_k = 16, 128, 512, 48, 4
    w, A, ids = _moe_case(qtype, E, N, K, T, top_k, True, 43, 0)
    fc, y1 = _run(w, qtype, A, ids, True)
    y2 = fc.grouped(_dev(A), _dev(ids), True)
    assert torch.equal(y1, y2)                 # bit-identical whatever the pair order
    out = torch.zeros((0, top_k, N), dtype=torch.float16, device="cuda")
    fc.grouped(torch.zeros((0, top_k, K), dtype=torch.float16, device="cuda"),
               torch.zeros((0, top_k), dtype=torch.int32, device="cuda"), True, out=out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("which,a_per_slot", [("gate_up", False), ("down", True)])
def test_moe_full_size_q6k(gpu_lib, which, a_per_slot):
    """128 experts, top-8, 256 tokens, Zipf(1.1): gate/up [768, 2048] on shared
    token rows, down [2048, 768] on per-pair rows.  Checked per expert on every
    multi-tile expert, the 8 smallest non-empty ones and 8 random others."""
    m = synth.MOE
    N, K = m[which]
    E, T, top_k = m["E"], m["T"], m["top_k"]
    w, A, ids = _moe_case("q6_k", E, N, K, T, top_k, a_per_slot, 4, 0 if which == "gate_up" else 1,
                          s=m["zipf_s"])
    import torch
    out, ok = guarded((T, top_k, N), torch.float16, seed=N)
    _, y = _run(w, "q6_k", A, ids, a_per_slot, out=out)
    ok()
    y = _host(y)
    assert np.all(np.isfinite(y))
    counts = np.bincount(ids.ravel(), minlength=E)
    nonempty = np.nonzero(counts)[0]
    hot = nonempty[counts[nonempty] > 32]
    cold = nonempty[np.argsort(counts[nonempty], kind="stable")[:8]]
    g = np.random.default_rng(7)
    rest = np.setdiff1d(nonempty, np.concatenate([hot, cold]))
    sample = np.unique(np.concatenate([hot, cold, g.choice(rest, size=min(8, rest.size), replace=False)]))
    assert hot.size >= 4
    _check_experts(y, w, "q6_k", A, ids, a_per_slot, sample)


@pytest.mark.parametrize("seed", range(30))
def test_moe_random(gpu_lib, seed):
    # seeded random grouped cases: expert count, shape, tokens, top_k, routing
    # skew and row sharing drawn at random; every expert checked on its own
    g = np.random.default_rng(5000 + seed)
    qtype = QTYPES[g.integers(len(QTYPES))]
    E = int(g.integers(1, 65))
    N = int(g.integers(1, 600))
    K = 256 * int(g.integers(1, 9))
    T = int(g.integers(1, 160))
    top_k = int(g.integers(1, min(E, 8) + 1))
    a_per_slot = bool(g.integers(2))
    s = float(g.uniform(0.0, 2.0))
    w, A, ids = _moe_case(qtype, E, N, K, T, top_k, a_per_slot, 41, seed, s=s)
    import torch
    out, ok = guarded((T, top_k, N), torch.float16, seed=seed)
    _, y = _run(w, qtype, A, ids, a_per_slot, out=out)
    ok()
    y = _host(y)
    assert np.isfinite(y).all()
    check_fro(y, ofc.moe_ref(A, w, qtype, ids, a_per_slot))
    _check_experts(y, w, qtype, A, ids, a_per_slot, np.unique(ids))


@pytest.mark.parametrize("qtype", QTYPES)
def test_moe_reuse_routing(gpu_lib, qtype):
    # gate/up then down with the same routing: the down call on the gate/up
    # call's bucketing (fc_gguf_run_grouped_reuse) is bit-identical to a
    # fresh down call, including the zero rows of invalid ids
    import torch
    from gguf_quant_block_amd.binding import FcGguf
    E, T, top_k = 12, 70, 3
    (N1, K1), (N2, K2) = (192, 512), (96, 768)
    w1, A1, ids = _moe_case(qtype, E, N1, K1, T, top_k, False, 46, 0)
    w2 = synth.blocks(qtype, E * N2, K2, synth.rng(46, 1, synth.TAG_BLOCKS)).reshape(E, N2, -1)
    A2 = synth.normal_f16((T, top_k, K2), synth.rng(46, 1, synth.TAG_A))
    ids[5, 2] = -3
    ids[9, 0] = E + 1
    up = FcGguf(N1, K1, qtype, w1, experts=E)
    down = FcGguf(N2, K2, qtype, w2, experts=E)
    idd, A1d, A2d = _dev(ids), _dev(A1), _dev(A2)
    up.grouped(A1d, idd, False)
    y_reuse, ok = guarded((T, top_k, N2), torch.float16, seed=9)
    y_reuse.fill_(float("nan"))
    down.grouped(A2d, idd, True, out=y_reuse, routed=up)
    ok()
    y_fresh = down.grouped(A2d, idd, True)
    torch.cuda.synchronize()
    assert torch.equal(y_reuse, y_fresh)
    y = _host(y_reuse)
    assert np.all(y[5, 2] == 0) and np.all(y[9, 0] == 0)
    check_fro(y, ofc.moe_ref(A2, w2, qtype, ids, True))
    # a handle may reuse its own bucketing
    y_self = down.grouped(A2d, idd, True, routed=down)
    torch.cuda.synchronize()
    assert torch.equal(y_self, y_fresh)


def test_moe_reuse_checks(gpu_lib):
    import ctypes
    import torch
    from gguf_quant_block_amd.binding import FcGguf, FcGgufError, lib
    E, N, K, T, top_k = 8, 64, 256, 20, 2
    w, A, ids = _moe_case("q4_k", E, N, K, T, top_k, False, 47, 0)
    a = FcGguf(N, K, "q4_k", w, experts=E)
    b = FcGguf(N, K, "q4_k", w, experts=E)
    other = FcGguf(N, K, "q4_k", np.concatenate([w, w]).reshape(2 * E, N, -1), experts=2 * E)
    Ad, idd = _dev(A), _dev(ids)
    idd2 = idd.clone()
    Y = torch.empty((T, top_k, N), dtype=torch.float16, device="cuda")
    with pytest.raises(FcGgufError):            # a has not run yet
        b.grouped(Ad, idd, False, out=Y, routed=a)
    a.grouped(Ad, idd, False)
    b.grouped(Ad, idd, False, out=Y, routed=a)  # fine

    def reuse(h, routed, T_, ids_, k_):
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        return lib().fc_gguf_run_grouped_reuse(h.handle, routed, ctypes.c_void_p(Ad.data_ptr()), T_, 0,
                                               ctypes.c_void_p(ids_.data_ptr()), k_,
                                               ctypes.c_void_p(Y.data_ptr()), st)
    assert reuse(b, a.handle, T, idd, top_k) == 0
    assert reuse(b, a.handle, T, idd2, top_k) == -1       # another ids buffer
    assert reuse(b, a.handle, T - 1, idd, top_k) == -1    # another token count
    assert reuse(b, a.handle, T, idd, 1) == -1            # another top_k
    assert reuse(b, other.handle, T, idd, top_k) == -1    # another expert count
    assert reuse(b, None, T, idd, top_k) == -1
    a.grouped(Ad, idd2, False)                            # a's bucketing now follows idd2
    assert reuse(b, a.handle, T, idd, top_k) == -1
    assert reuse(b, a.handle, T, idd2, top_k) == 0
    torch.cuda.synchronize()


# ------------------------------------------------------------- bucketing ----

def _check_bucketing(ids, E, BM):
    from gguf_quant_block_amd.binding import debug_bucketing
    off, pairs, tiles = debug_bucketing(_dev(ids.astype(np.int32)), E, BM)
    want_off, want_pairs, want_tiles = ofc.moe_bucketing(ids, E, BM)
    assert np.array_equal(_host(off).astype(np.int64), want_off)
    got = _host(pairs).astype(np.int64)
    for b in range(E + 1):
        lo, hi = want_off[b], want_off[b + 1]
        assert np.array_equal(np.sort(got[lo:hi]), want_pairs[lo:hi]), f"bucket {b}"
    assert np.array_equal(_host(tiles).astype(np.int64).reshape(-1, 2), want_tiles)


@pytest.mark.parametrize("BM", [32, 64, 128])
def test_bucketing_benchmark_routing(gpu_lib, BM):
    m = synth.MOE
    ids = synth.moe_routing(m["T"], m["E"], m["top_k"], synth.rng(5, 0, synth.TAG_ROUTING), s=m["zipf_s"])
    _check_bucketing(ids, m["E"], BM)


@pytest.mark.parametrize("E,P,BM,seed", [
    (1, 1, 16, 0),          # one pair, one expert
    (7, 300, 32, 1),        # ids outside [0, E) as well
    (1000, 3000, 64, 2),    # more than 512 buckets: two scatter passes
    (4096, 5000, 128, 3),   # the largest E; more rounds than the ids kept in registers
    (64, 9000, 16, 4),      # long rounds loop, hot and empty buckets
])
def test_bucketing_random(gpu_lib, E, P, BM, seed):
    g = np.random.default_rng(seed)
    if seed == 4:
        ids = np.where(g.random(P) < 0.5, 3, g.integers(0, 8, size=P))
    else:
        ids = g.integers(-3, E + 3, size=P)
    _check_bucketing(ids.astype(np.int32), E, BM)
