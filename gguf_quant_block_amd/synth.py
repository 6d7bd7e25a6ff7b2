"""Seeded synthetic inputs for the GGUF K-quant fully-connected layer.

This module only draws random numbers and places them into the byte slots of
a block; it holds none of the layer's arithmetic (no decode, no quantisation,
no matmul).  It is the one module that both the CPU oracle tests and the HIP
path's tests and benchmark use, so that both sides see identical inputs.

Block byte slots used here (GGUF super-block structs, 256 values per block):
  Q4_K, 144 B: d f16 @0, dmin f16 @2, 12 packed scale/min bytes @4,
               qs[128] @16 (the struct printed in the onnxruntime-mobius
               GGUF proposal, section 7.3).
  Q5_K, 176 B: d f16 @0, dmin f16 @2, 12 packed scale/min bytes @4,
               qh[32] @16, qs[128] @48
               (field order as in the onnxruntime-mobius GGUF proposal,
               section 7.3, for the K-quant header d | dmin | scales).
  Q6_K, 210 B: ql[128] @0, qh[64] @128, sc[16] int8 @192, d f16 @208
               (the plane order QL | QH | SC | D of OpenVINO PR #39119,
               section Transformation).

Value distributions (all uniform unless stated):
  Q5_K: d in [1e-3, 1e-2], dmin in [0, 5e-3] (f64 draws rounded to f16 with
        round-to-nearest-even); scale/min bytes, qh and qs uniform bytes.
  Q4_K: as Q5_K, with d in [2e-3, 2e-2] (4-bit codes need twice the step
        for a similar weight range).
  Q6_K: ql, qh uniform bytes; sc uniform integers in [-32, 31]; d as Q5_K.
  Activations and residuals: f32 N(0,1) draws rounded to f16 (or kept in
  f32 for f32 activations).
  MoE routing: Zipf(s) popularity over a seeded permutation of the experts,
  top-k distinct experts per token by Gumbel-top-k (sampling without
  replacement).

Seeds: numpy PCG64 seeded with SeedSequence([2026, cfg, case, tag]), tag
0 = blocks, 1 = activations, 2 = residual, 3 = routing.
"""

from __future__ import annotations

import numpy as np

QK = 256
Q4K_BYTES = 144
Q5K_BYTES = 176
Q6K_BYTES = 210

TAG_BLOCKS, TAG_A, TAG_R, TAG_ROUTING = 0, 1, 2, 3


def rng(cfg: int, case: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, cfg, case, tag])))


def _f16_uniform(g: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return g.uniform(lo, hi, size=shape).astype(np.float16)


def q4k_blocks(N: int, K: int, g: np.random.Generator) -> np.ndarray:
    """u8[N, K/256*144]: row-major (n, kb) AoS Q4_K super-blocks."""
    assert K % QK == 0
    nb = K // QK
    raw = g.integers(0, 256, size=(N, nb, Q4K_BYTES), dtype=np.uint8)
    d = _f16_uniform(g, (N, nb), 2e-3, 2e-2)
    dmin = _f16_uniform(g, (N, nb), 0.0, 5e-3)
    raw[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
    raw[:, :, 2:4] = dmin.view(np.uint8).reshape(N, nb, 2)
    return raw.reshape(N, nb * Q4K_BYTES)


def q5k_blocks(N: int, K: int, g: np.random.Generator) -> np.ndarray:
    """u8[N, K/256*176]: row-major (n, kb) AoS Q5_K super-blocks."""
    assert K % QK == 0
    nb = K // QK
    raw = g.integers(0, 256, size=(N, nb, Q5K_BYTES), dtype=np.uint8)
    d = _f16_uniform(g, (N, nb), 1e-3, 1e-2)
    dmin = _f16_uniform(g, (N, nb), 0.0, 5e-3)
    raw[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
    raw[:, :, 2:4] = dmin.view(np.uint8).reshape(N, nb, 2)
    return raw.reshape(N, nb * Q5K_BYTES)


def q6k_blocks(N: int, K: int, g: np.random.Generator) -> np.ndarray:
    """u8[N, K/256*210]: row-major (n, kb) AoS Q6_K super-blocks."""
    assert K % QK == 0
    nb = K // QK
    raw = g.integers(0, 256, size=(N, nb, Q6K_BYTES), dtype=np.uint8)
    sc = g.integers(-32, 32, size=(N, nb, 16)).astype(np.int8)
    d = _f16_uniform(g, (N, nb), 1e-3, 1e-2)
    raw[:, :, 192:208] = sc.view(np.uint8)
    raw[:, :, 208:210] = d.view(np.uint8).reshape(N, nb, 2)
    return raw.reshape(N, nb * Q6K_BYTES)


def blocks(qtype: str, N: int, K: int, g: np.random.Generator) -> np.ndarray:
    if qtype == "q4_k":
        return q4k_blocks(N, K, g)
    if qtype == "q5_k":
        return q5k_blocks(N, K, g)
    if qtype == "q6_k":
        return q6k_blocks(N, K, g)
    raise ValueError(qtype)


def block_bytes(qtype: str) -> int:
    return {"q4_k": Q4K_BYTES, "q5_k": Q5K_BYTES, "q6_k": Q6K_BYTES}[qtype]


def normal_f16(shape, g: np.random.Generator) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32).astype(np.float16)


def normal_f32(shape, g: np.random.Generator) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


def moe_routing(T: int, E: int, top_k: int, g: np.random.Generator, s: float = 1.1) -> np.ndarray:
    """i32[T, top_k]: distinct expert ids per token, Zipf(s)-skewed popularity.

    Expert popularity p(rank r) is proportional to r**-s over a seeded
    permutation of the E expert ids; each token takes top_k distinct experts
    by the Gumbel-top-k trick (equivalent to sequential sampling without
    replacement from p).
    """
    perm = g.permutation(E)
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    logp = np.empty(E)
    logp[perm] = np.log(p / p.sum())
    gumbel = -np.log(-np.log(g.uniform(size=(T, E))))
    keys = logp[None, :] + gumbel
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :top_k]
    return ids.astype(np.int32)


# Workloads (shapes only).  Phi-3.5-mini layer shapes: hidden 3072,
# fused qkv 9216, fused gate/up 16384, down 8192 -> 3072, vocab 32064.
PHI35_LAYERS = {
    "qkv": (9216, 3072),
    "o_proj": (3072, 3072),
    "gate_up": (16384, 3072),
    "down": (3072, 8192),
}
PHI35_OUTPUT = (32064, 3072)
PREFILL_SHAPES = [(8192, 2048), (2048, 8192)]
PREFILL_MS = [8, 64, 128, 256, 512, 2048]
MOE = dict(E=128, top_k=8, T=256, gate_up=(768, 2048), down=(2048, 768), zipf_s=1.1)
