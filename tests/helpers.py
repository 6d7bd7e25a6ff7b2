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
