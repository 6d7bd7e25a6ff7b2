"""Fully-connected reference: Y = A.W^T (+R) on GGUF Q4_K / Q5_K / Q6_K blocks.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources.
  * OpenVINO PR #39119 "FullyConnectedGGUF":
      - section Details / Implementation: the decode path quantises the
        activations per 32 values and takes int8 dot products directly
        against the Q5_K / Q6_K blocks; a same-shape residual Add is fused
        into the output store;
      - section Transformation: dynamic quantisation in groups of 32.
  * llama.cpp PR #28301 (Metal mul_mm_id), section Overview: an MoE expert
    FC multiplies each expert's routed token rows by that expert's weights.

Two references are provided:
  fc_ref       the plain definition, Y = A.W^T + R in float64 with W decoded
               exactly (used for the prefill path and for MoE);
  fc_ref_int8  an exact emulation of the int8 decode path: the activations
               are quantised per group of 32 exactly as the kernel does (f32
               arithmetic), the integer sub-block dot sums are formed in
               int64, and the scales are combined in float64.

Readings where the pages are silent (all are stated here and nowhere fixed
by the pages):
  * activation quantisation is symmetric per aligned group of 32 values of
    one row: amax = max|a| (f32), s = fl32(amax/127), inv = fl32(127/amax),
    qa = clamp(round_half_even(fl32(a*inv)), -127, 127); an all-zero group
    has s = 0 and qa = 0, and so has a group whose inverse scale 127/amax
    overflows f32 (amax < 127/FLT_MAX, reachable with f32 activations only);
  * f32 activations are quantised from their f32 values (the same steps; f16
    activations are widened to f32 exactly first);
  * the Q5_K min term uses the sum of the quantised activations,
    s_g * T_g with T_g = sum(qa over group g), so that the decode path
    computes exactly (s*qa) . W^T;
  * the residual R has the output's shape [M, N] and is added once.
"""

from __future__ import annotations

import numpy as np

from .kquant import (QK, as_blocks, dequantize, q4k_codes, q4k_scale_min, q5k_codes,
                     q5k_scale_min, q6k_codes, q6k_scales, _f16_at)

GROUP = 32


def fc_ref(A: np.ndarray, W: np.ndarray, R: np.ndarray | None = None) -> np.ndarray:
    """float64[M, N] = A.W^T + R, all operands widened to float64."""
    Y = A.astype(np.float64) @ W.astype(np.float64).T
    if R is not None:
        Y = Y + R.astype(np.float64)
    return Y


def fc_naive(A: np.ndarray, W: np.ndarray, R: np.ndarray | None = None) -> np.ndarray:
    """Triple loop in plain Python floats (tiny shapes only)."""
    M, K = A.shape
    N = W.shape[0]
    Y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(A[m, k]) * float(W[n, k])
            if R is not None:
                acc += float(R[m, n])
            Y[m, n] = acc
    return Y


def fc_gguf_ref(A, w_bytes, qtype, R=None):
    """float64 reference of the FC on raw blocks: exact decode, then fc_ref."""
    return fc_ref(A, dequantize(w_bytes, qtype), R)


# ------------------------------------------- int8 activation quantisation --

def quantize_act(A: np.ndarray):
    """Per-32 symmetric int8 quantisation of f16 or f32 activations A[M, K].

    Returns qa int8[M, K], s float32[M, K/32], T int32[M, K/32].
    All float steps are IEEE float32 (numpy float32 division and product are
    correctly rounded); np.rint rounds half to even.
    """
    M, K = A.shape
    assert K % GROUP == 0
    a = A.astype(np.float32).reshape(M, K // GROUP, GROUP)
    amax = np.abs(a).max(axis=2)
    safe = np.where(amax > 0, amax, np.float32(1))
    with np.errstate(over="ignore"):
        inv_all = (np.float32(127) / safe).astype(np.float32)
    nz = (amax > 0) & np.isfinite(inv_all)
    s = np.where(nz, safe / np.float32(127), np.float32(0)).astype(np.float32)
    inv = np.where(nz, inv_all, np.float32(0)).astype(np.float32)
    prod = (a * inv[..., None]).astype(np.float32)
    qa = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    T = qa.astype(np.int32).sum(axis=2).astype(np.int32)
    return qa.reshape(M, K), s, T


def dequant_act(qa: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float64 A_hat = s * qa (the activations the int8 path effectively uses)."""
    M, K = qa.shape
    return (qa.astype(np.float64).reshape(M, K // GROUP, GROUP)
            * s.astype(np.float64)[..., None]).reshape(M, K)


# ------------------------------------------------- integer sub-block sums --

def int_dots(qa: np.ndarray, w_bytes: np.ndarray, qtype: str) -> np.ndarray:
    """Exact integer dot sums per (m, n, sub-block).

    Q4_K, Q5_K: S[m,n,j] = sum over the 32 values of sub-block j of qa*q,
          q in [0,15] / [0,31]; shape [M, N, K/32].
    Q6_K: S[m,n,s] = sum over the 16 values of sub-block s of qa*(q-32);
          shape [M, N, K/16].
    """
    blk = as_blocks(w_bytes, qtype)
    N, nb = blk.shape[:2]
    K = nb * QK
    M = qa.shape[0]
    if qtype in ("q4_k", "q5_k"):
        codes = q4k_codes if qtype == "q4_k" else q5k_codes
        q = codes(blk).reshape(N, K)
        width = 32
    else:
        q = q6k_codes(blk).reshape(N, K) - 32
        width = 16
    qa3 = qa.astype(np.int64).reshape(M, K // width, width)
    q3 = q.astype(np.int64).reshape(N, K // width, width)
    return np.einsum("mgk,ngk->mng", qa3, q3)


def fc_ref_int8(A, w_bytes, qtype, R=None):
    """float64[M, N]: the decode path's result, combined explicitly.

    Q4_K, Q5_K: y = sum_j s_j * (d*sc_j*S_j - dmin*m_j*T_j) + R
    Q6_K: y = sum_s s_{s//2} * d*sc_s*S_s + R
    """
    qa, s, T = quantize_act(A)
    S = int_dots(qa, w_bytes, qtype).astype(np.float64)
    blk = as_blocks(w_bytes, qtype)
    N, nb = blk.shape[:2]
    M = A.shape[0]
    s64 = s.astype(np.float64)
    if qtype in ("q4_k", "q5_k"):
        d = _f16_at(blk, 0)                      # [N, nb]
        dmin = _f16_at(blk, 2)
        scale_min = q4k_scale_min if qtype == "q4_k" else q5k_scale_min
        sc, mn = scale_min(blk)                  # [N, nb, 8]
        dsc = (d[..., None] * sc).reshape(N, nb * 8)
        dmm = (dmin[..., None] * mn).reshape(N, nb * 8)
        term = (S * dsc[None]) - dmm[None] * T.astype(np.float64)[:, None, :]
        Y = (term * s64[:, None, :]).sum(axis=2)
    else:
        d = _f16_at(blk, 208)
        sc = q6k_scales(blk)                     # [N, nb, 16]
        dsc = (d[..., None] * sc).reshape(N, nb * 16)
        s16 = np.repeat(s64, 2, axis=1)          # group of sub-block s is s//2
        Y = (S * dsc[None] * s16[:, None, :]).sum(axis=2)
    if R is not None:
        Y = Y + R.astype(np.float64)
    assert Y.shape == (M, N)
    return Y


# ------------------------------------------------------------------- MoE --

def moe_bucketing(ids, E: int, BM: int):
    """Expert bucketing of the (token, slot) pairs (llama.cpp PR #28301,
    Overview: the routed rows are grouped by expert, and each expert's rows
    form row tiles).

    ids: routing ids of any shape; pair p is the p-th id in row-major order.
    Bucket e < E holds the pairs routed to expert e, bucket E those whose id
    is outside [0, E).  Returns
      offsets int64[E+2]: bucket b's pairs are pairs[offsets[b]:offsets[b+1]];
      pairs   int64[P]:   pair indices grouped by bucket, listed in
                          increasing order within a bucket (the page leaves
                          the order inside an expert open, and no result
                          depends on it: a comparison takes each bucket as a
                          set);
      tiles   int64[n, 2]: (bucket, first row within the bucket) for every BM
                          rows of every bucket, buckets in increasing order.
    """
    ids = np.asarray(ids).reshape(-1)
    b = np.where((ids >= 0) & (ids < E), ids, E)
    counts = np.bincount(b, minlength=E + 1)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    pairs = np.argsort(b, kind="stable").astype(np.int64)
    tiles = [(e, r0) for e in range(E + 1) for r0 in range(0, int(counts[e]), BM)]
    return offsets, pairs, np.array(tiles, dtype=np.int64).reshape(-1, 2)


def moe_ref(A, w_bytes_e, qtype, ids, a_per_slot: bool):
    """float64 Y[T, top_k, N]: Y[t, j] = A_row(t, j) . W_{ids[t, j]}^T.

    A is f16[T, K] (one row per token, shared by its top_k experts) or
    f16[T, top_k, K] (one row per (token, slot) pair).  w_bytes_e is
    u8[E, N, K/256*B].  No routing weights and no combine.
    """
    T, top_k = ids.shape
    E, N = w_bytes_e.shape[:2]
    Y = np.zeros((T, top_k, N))
    for e in range(E):
        tt, jj = np.nonzero(ids == e)
        if tt.size == 0:
            continue
        W = dequantize(w_bytes_e[e], qtype)
        rows = A[tt, jj] if a_per_slot else A[tt]
        Y[tt, jj] = fc_ref(rows, W)
    return Y
