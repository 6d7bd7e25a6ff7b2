"""Shared test helpers: error metrics and seeded cases (no layer arithmetic)."""

import numpy as np

from gguf_quant_block_amd import synth


def maxrel(y, r):
    """max_i |y_i - r_i| / max(|r_i|, rms(r)): the decode-path metric."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    den = np.maximum(np.abs(r), rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(y - r) / den)) if r.size else 0.0


def relfro(y, r):
    """||y - r||_F / ||r||_F: the prefill / MoE metric."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    n = np.linalg.norm(r)
    return float(np.linalg.norm(y - r) / n) if n > 0 else float(np.linalg.norm(y))


def case(qtype, M, N, K, cfg, idx, with_r=True):
    """Seeded (blocks u8[N, K/256*B], A f16[M,K], R f16[M,N] or None)."""
    w = synth.blocks(qtype, N, K, synth.rng(cfg, idx, synth.TAG_BLOCKS))
    A = synth.normal_f16((M, K), synth.rng(cfg, idx, synth.TAG_A))
    R = synth.normal_f16((M, N), synth.rng(cfg, idx, synth.TAG_R)) if with_r else None
    return w, A, R


DECODE_TOL = 1e-3      # max relative error vs the int8-emulating oracle
PREFILL_TOL = 2e-3     # relative Frobenius error vs the float64 oracle


def extreme_scales(w, qtype, seed):
    """Blocks w with their sub-block scales pushed to the format's limits
    (Q6_K int8 scales in {-128, 127} on about half the sub-blocks, the rest
    uniform over all 256 values; Q4_K / Q5_K: all six-bit scales and mins 63
    on every other block), so that intermediate magnitudes are exercised."""
    g = np.random.default_rng(seed)
    bb = {"q4_k": 144, "q5_k": 176, "q6_k": 210}[qtype]
    blk = w.reshape(-1, bb).copy()
    if qtype == "q6_k":
        sc = g.integers(-128, 128, size=(blk.shape[0], 16))
        ext = g.random(size=sc.shape) < 0.5
        sc = np.where(ext, np.where(g.random(size=sc.shape) < 0.5, -128, 127), sc)
        blk[:, 192:208] = sc.astype(np.int8).view(np.uint8)
    else:
        blk[::2, 4:16] = 0xFF
    return blk.reshape(w.shape)
