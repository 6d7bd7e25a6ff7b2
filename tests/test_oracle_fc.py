"""Pins for the oracle's FC, activation quantisation and int8 emulation (CPU).

  * fc_ref against exact rational arithmetic (every f16 value and every
    decoded weight is a dyadic rational) and against a naive triple loop;
  * decoded weights against an exact Fraction evaluation of the formulas;
  * activation quantisation against closed-form groups and invariants;
  * int_dots against scalar brute-force loops;
  * fc_ref_int8 (explicit scale combination) against fc_ref on the
    dequantised activations, which is the same quantity in exact arithmetic;
  * a negative control: the lossy "flattened" single-level scale/zero-point
    form with a rounded zero point (the MatMulNBits mapping of the mobius
    proposal, section 7.3) gives a clearly different result from the exact
    decode (the OpenVINO PR #38696 accuracy test, adapted).
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from gguf_quant_block_amd import synth
from oracle import fc, kquant as kq


def _inputs(qtype, M, N, K, seed, with_r=True):
    w = synth.blocks(qtype, N, K, synth.rng(97, seed, 0))
    A = synth.normal_f16((M, K), synth.rng(97, seed, 1))
    R = synth.normal_f16((M, N), synth.rng(97, seed, 2)) if with_r else None
    return w, A, R


@pytest.mark.parametrize("qtype", ["q4_k", "q5_k", "q6_k"])
def test_decode_equals_exact_fraction_formula(qtype):
    w = synth.blocks(qtype, 2, 512, synth.rng(97, 11, 0))
    blk = kq.as_blocks(w, qtype)
    W = kq.dequantize(w, qtype)
    for n in range(2):
        for kb in range(2):
            b = blk[n, kb]
            for i in range(0, 256, 7):
                if qtype in ("q4_k", "q5_k"):
                    d = Fraction(float(b[0:2].view(np.float16)[0]))
                    dmin = Fraction(float(b[2:4].view(np.float16)[0]))
                    sc, m = kq.q5k_scale_min(b)
                    q = (kq.q4k_codes if qtype == "q4_k" else kq.q5k_codes)(b)[i]
                    exact = d * int(sc[i // 32]) * int(q) - dmin * int(m[i // 32])
                else:
                    d = Fraction(float(b[208:210].view(np.float16)[0]))
                    exact = d * int(kq.q6k_scales(b)[i // 16]) * (int(kq.q6k_codes(b)[i]) - 32)
                assert Fraction(float(W[n, 256 * kb + i])) == exact


@pytest.mark.parametrize("qtype", ["q4_k", "q5_k", "q6_k"])
def test_fc_ref_matches_exact_rational(qtype):
    M, N, K = 2, 3, 256
    w, A, R = _inputs(qtype, M, N, K, 12)
    W = kq.dequantize(w, qtype)
    Y = fc.fc_ref(A, W, R)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(A[m, k])) * Fraction(float(W[n, k])) for k in range(K))
            exact += Fraction(float(R[m, n]))
            # float64 BLAS rounding over 256 terms: tiny relative error bound
            scale = sum(abs(float(A[m, k]) * float(W[n, k])) for k in range(K)) + abs(float(R[m, n]))
            assert abs(float(exact) - Y[m, n]) <= 1e-13 * scale


def test_fc_naive_equals_fc_ref():
    w, A, R = _inputs("q6_k", 3, 4, 512, 13)
    W = kq.dequantize(w, "q6_k")
    assert np.allclose(fc.fc_naive(A, W, R), fc.fc_ref(A, W, R), rtol=1e-12, atol=1e-12)
    assert np.allclose(fc.fc_naive(A, W), fc.fc_ref(A, W), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------- activation quant ----

def test_quantize_closed_form_unit_amax():
    # a_k = (k-16)/16, amax = 1 exactly -> inv = 127 exactly, qa = RNE(127*a);
    # expected codes are the hand-derived fixture tests/golden/actquant_unit_amax.txt
    path = os.path.join(os.path.dirname(__file__), "golden", "actquant_unit_amax.txt")
    gold = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split(":", 1)
            gold[k.strip()] = [int(x) for x in v.split()]
    a = np.array([(k - 16) / 16 for k in range(32)], dtype=np.float16)[None]
    qa, s, T = fc.quantize_act(a)
    assert list(qa[0]) == gold["qa"]
    assert gold["qa"][8] == -64 and gold["qa"][24] == 64      # the two ties go to even
    assert s[0, 0] == np.float32(1) / np.float32(127)
    assert T[0, 0] == gold["T"][0]


def test_quantize_zero_group_and_invariants():
    g = np.random.default_rng(3)
    A = g.standard_normal((4, 256)).astype(np.float16)
    A[1, 32:64] = 0
    A[2, :32] *= np.float16(1e-3)
    qa, s, T = fc.quantize_act(A)
    assert (qa[1, 32:64] == 0).all() and s[1, 1] == 0 and T[1, 1] == 0
    assert np.abs(qa.astype(int)).max() <= 127
    a3 = A.astype(np.float32).reshape(4, 8, 32)
    q3 = qa.reshape(4, 8, 32).astype(np.float64)
    for m in range(4):
        for gi in range(8):
            if s[m, gi] == 0:
                continue
            am = np.argmax(np.abs(a3[m, gi]))
            assert abs(q3[m, gi, am]) == 127
            err = np.abs(s[m, gi] * q3[m, gi] - a3[m, gi])
            assert (err <= s[m, gi] * 0.5 * (1 + 1e-5) + 1e-7 * np.abs(a3[m, gi])).all()
    assert np.array_equal(T, qa.reshape(4, 8, 32).astype(np.int32).sum(axis=2))


def test_quantize_f32_unit_amax_matches_golden():
    # the same closed-form group as f32 values: identical codes and scale
    path = os.path.join(os.path.dirname(__file__), "golden", "actquant_unit_amax.txt")
    gold = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split(":", 1)
            gold[k.strip()] = [int(x) for x in v.split()]
    a = np.array([(k - 16) / 16 for k in range(32)], dtype=np.float32)[None]
    qa, s, T = fc.quantize_act(a)
    assert list(qa[0]) == gold["qa"] and T[0, 0] == gold["T"][0]
    assert s[0, 0] == np.float32(1) / np.float32(127)


def test_quantize_f32_groups_beyond_f16():
    g = np.random.default_rng(8)
    A = g.standard_normal((3, 128)).astype(np.float32)
    A[0, :32] *= np.float32(1e-37)          # 127/amax overflows f32: a zero group
    A[0, 32:64] = np.float32(5e-37) * np.array([(k - 16) / 16 for k in range(32)], dtype=np.float32)
    #                                         tiny but 127/amax finite: s is subnormal
    A[1, :32] *= np.float32(1e30)           # far beyond the f16 range
    A[2, 5] = np.float32(1e-40)             # an f32 subnormal inside a normal group
    qa, s, T = fc.quantize_act(A)
    assert s[0, 0] == 0 and (qa[0, :32] == 0).all() and T[0, 0] == 0
    amax = np.abs(A[0, 32:64]).max()
    assert np.isfinite(np.float32(127) / amax)
    assert s[0, 1] == amax / np.float32(127) and s[0, 1] < np.finfo(np.float32).tiny
    assert np.abs(qa[0, 32:64].astype(int)).max() == 127
    assert np.abs(qa[1, :32].astype(int)).max() == 127 and s[1, 0] == np.abs(A[1, :32]).max() / np.float32(127)
    assert qa[2, 5] == 0
    # every nonzero group: |s*q - a| <= s/2 (up to the f32 rounding of a*inv)
    a3 = A.astype(np.float64).reshape(3, 4, 32)
    q3 = qa.reshape(3, 4, 32).astype(np.float64)
    for m in range(3):
        for gi in range(4):
            if s[m, gi] == 0:
                continue
            sc = float(s[m, gi])
            assert (np.abs(sc * q3[m, gi] - a3[m, gi]) <= sc * 0.5 * (1 + 1e-5) + 1e-6 * np.abs(a3[m, gi])).all()


def test_quantize_f16_equals_f32_of_same_values():
    A = synth.normal_f16((2, 256), synth.rng(97, 40, 1))
    for x, y in zip(fc.quantize_act(A), fc.quantize_act(A.astype(np.float32))):
        assert np.array_equal(x, y)


# ------------------------------------------------------------ int dots ----

@pytest.mark.parametrize("qtype", ["q4_k", "q5_k", "q6_k"])
def test_int_dots_brute_force(qtype):
    M, N, K = 2, 3, 512
    w, A, _ = _inputs(qtype, M, N, K, 14, with_r=False)
    qa, _, _ = fc.quantize_act(A)
    S = fc.int_dots(qa, w, qtype)
    blk = kq.as_blocks(w, qtype)
    width = 16 if qtype == "q6_k" else 32
    for m in range(M):
        for n in range(N):
            for sb in range(K // width):
                acc = 0
                for k in range(sb * width, sb * width + width):
                    b = blk[n, k // 256]
                    if qtype == "q4_k":
                        q = int(kq.q4k_codes(b)[k % 256])
                    elif qtype == "q5_k":
                        q = int(kq.q5k_codes(b)[k % 256])
                    else:
                        q = int(kq.q6k_codes(b)[k % 256]) - 32
                    acc += int(qa[m, k]) * q
                assert S[m, n, sb] == acc


# ------------------------------------------------------- int8 emulation ----

@pytest.mark.parametrize("qtype", ["q4_k", "q5_k", "q6_k"])
@pytest.mark.parametrize("with_r", [False, True])
def test_int8_emulation_identity(qtype, with_r):
    M, N, K = 3, 8, 1024
    w, A, R = _inputs(qtype, M, N, K, 15, with_r)
    y_int = fc.fc_ref_int8(A, w, qtype, R)
    qa, s, _ = fc.quantize_act(A)
    y_hat = fc.fc_ref(fc.dequant_act(qa, s), kq.dequantize(w, qtype), R)
    assert np.allclose(y_int, y_hat, rtol=1e-11, atol=1e-11 * np.abs(y_hat).max())


def test_int8_emulation_close_to_unquantised():
    # int8 activations change the result by about the quantisation noise
    w, A, _ = _inputs("q6_k", 2, 64, 2048, 16, with_r=False)
    y8 = fc.fc_ref_int8(A, w, "q6_k")
    y = fc.fc_gguf_ref(A, w, "q6_k")
    rel = np.linalg.norm(y8 - y) / np.linalg.norm(y)
    assert 1e-4 < rel < 2e-2


# ----------------------------------------------------- negative control ----

def test_rounded_zero_point_is_measurably_worse():
    """Flattening Q5_K to w' = (sc*d) * (q - round(m*dmin/(sc*d))) is lossy;
    the oracle's exact decode must differ from it clearly (>= 4x error ratio
    against a float64 reference built from the fields)."""
    w, A, _ = _inputs("q5_k", 4, 64, 2048, 17, with_r=False)
    blk = kq.as_blocks(w, "q5_k")
    d = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)[..., None]
    dmin = blk[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)[..., None]
    sc, m = kq.q5k_scale_min(blk)
    q = kq.q5k_codes(blk).astype(np.float64)
    j = np.arange(256) // 32
    eff = d * sc[..., j]
    zp = np.round(np.where(eff > 0, dmin * m[..., j] / np.where(eff > 0, eff, 1), 0))
    w_flat = (eff * (q - zp)).reshape(64, 2048)
    w_fields = (d * sc[..., j] * q - dmin * m[..., j]).reshape(64, 2048)
    W = kq.dequantize(w, "q5_k")
    assert np.array_equal(W, w_fields)
    err_exact = np.linalg.norm(fc.fc_ref(A, W) - fc.fc_ref(A, w_fields))
    err_flat = np.linalg.norm(fc.fc_ref(A, w_flat) - fc.fc_ref(A, w_fields))
    assert err_flat > 0 and err_exact * 4 <= err_flat


# ------------------------------------------------------------------ MoE ----

def test_moe_ref_matches_per_pair_loop():
    E, N, K, T, top_k = 6, 8, 256, 10, 3
    we = np.stack([synth.q6k_blocks(N, K, synth.rng(97, 20 + e, 0)) for e in range(E)])
    ids = synth.moe_routing(T, E, top_k, synth.rng(97, 30, 3))
    A = synth.normal_f16((T, K), synth.rng(97, 30, 1))
    Ap = synth.normal_f16((T, top_k, K), synth.rng(97, 31, 1))
    Y = fc.moe_ref(A, we, "q6_k", ids, a_per_slot=False)
    Yp = fc.moe_ref(Ap, we, "q6_k", ids, a_per_slot=True)
    for t in range(T):
        for j in range(top_k):
            W = kq.dequantize(we[ids[t, j]], "q6_k")
            assert np.allclose(Y[t, j], W @ A[t].astype(np.float64), rtol=1e-12, atol=1e-12)
            assert np.allclose(Yp[t, j], W @ Ap[t, j].astype(np.float64), rtol=1e-12, atol=1e-12)


def test_routing_distinct_and_skewed():
    ids = synth.moe_routing(256, 128, 8, synth.rng(4, 0, 3))
    assert ids.shape == (256, 8)
    for row in ids:
        assert len(set(row.tolist())) == 8
    counts = np.bincount(ids.reshape(-1), minlength=128)
    assert counts.sum() == 2048 and counts.max() > 100 and np.median(counts) < 16


@pytest.mark.parametrize("E,BM", [(1, 16), (5, 4), (13, 32)])
def test_moe_bucketing_brute_force(E, BM):
    # the bucketing against a pair-by-pair walk: each bucket collects its
    # pairs in increasing index order, then is cut into BM-row tiles
    g = np.random.default_rng(1000 + E)
    ids = g.integers(-2, E + 2, size=(37, 3)).astype(np.int32)   # ids outside [0, E) too
    offsets, pairs, tiles = fc.moe_bucketing(ids, E, BM)
    flat = ids.reshape(-1).tolist()
    buckets = [[] for _ in range(E + 1)]
    for p, e in enumerate(flat):
        buckets[e if 0 <= e < E else E].append(p)
    want_pairs = [p for bk in buckets for p in bk]
    want_offsets = [0]
    for bk in buckets:
        want_offsets.append(want_offsets[-1] + len(bk))
    want_tiles = []
    for e, bk in enumerate(buckets):
        r0 = 0
        while r0 < len(bk):
            want_tiles.append((e, r0))
            r0 += BM
    assert pairs.tolist() == want_pairs
    assert offsets.tolist() == want_offsets
    assert [tuple(t) for t in tiles.tolist()] == want_tiles


def test_moe_bucketing_empty_buckets_and_no_invalid():
    offsets, pairs, tiles = fc.moe_bucketing(np.array([[2, 0], [2, 3]], dtype=np.int32), 4, 2)
    assert offsets.tolist() == [0, 1, 1, 3, 4, 4]
    assert pairs.tolist() == [1, 0, 2, 3]
    assert tiles.tolist() == [[0, 0], [2, 0], [3, 0]]
