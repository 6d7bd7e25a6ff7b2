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


def tile_bytes(plane, N, KB, P, fill=0):
    """Canonical plane bytes [N*KB, 16*P] (block (n, kb) at row n*KB + kb) ->
    the tiled device order: tiles of 16 rows x 4 blocks (rows padded to 16,
    blocks per row to 4), tile t = (n/16)*(KBp/4) + kb/4 stored piece-major,
    the blocks of a piece in the order (kb % 4)*16 + n % 16."""
    Np, KBp = -(-N // 16) * 16, -(-KB // 4) * 4
    x = np.full((Np, KBp, P, 16), fill, dtype=plane.dtype)
    x[:N, :KB] = plane.reshape(N, KB, P, 16)
    return x.reshape(Np // 16, 16, KBp // 4, 4, P, 16).transpose(0, 2, 4, 3, 1, 5).reshape(-1)


def _tile_d(d, N, KB):
    """Q6_K d bytes [N*KB, 2] -> tiled: 128 bytes per tile, slot (kb % 4)*16 + n % 16."""
    Np, KBp = -(-N // 16) * 16, -(-KB // 4) * 4
    x = np.zeros((Np, KBp, 2), dtype=d.dtype)
    x[:N, :KB] = d.reshape(N, KB, 2)
    return x.reshape(Np // 16, 16, KBp // 4, 4, 2).transpose(0, 2, 3, 1, 4).reshape(-1)


def expected_device_bytes(w, qtype, N, K):
    """The library's device copy of canonical blocks w[N, K/256*B] in the tiled
    layout: Q4_K / Q5_K blocks as one plane of 9 / 11 pieces; Q6_K planes
    QL | QH | SC | D (the oracle's regroup), each tiled the same way."""
    KB = K // 256
    if qtype == "q4_k":
        return tile_bytes(w.reshape(-1, 144), N, KB, 9)
    if qtype == "q5_k":
        return tile_bytes(w.reshape(-1, 176), N, KB, 11)
    from oracle import kquant as okq
    planes = okq.q6k_regroup(w)
    nblk = N * KB
    ql = planes[:128 * nblk].reshape(nblk, 128)
    qh = planes[128 * nblk:192 * nblk].reshape(nblk, 64)
    sc = planes[192 * nblk:208 * nblk].reshape(nblk, 16)
    d = planes[208 * nblk:].reshape(nblk, 2)
    return np.concatenate([tile_bytes(ql, N, KB, 8), tile_bytes(qh, N, KB, 4), tile_bytes(sc, N, KB, 1),
                           _tile_d(d, N, KB)])


ELEM_GUARD = 1e-2      # element-wise guard beside the Frobenius bar (maxrel metric)


def check_fro(y, ref, tol=PREFILL_TOL):
    """The prefill / MoE bar: relative Frobenius error <= tol, and no single
    element off by more than ELEM_GUARD of max(|ref|, rms(ref)) (one wrong
    element among many barely moves the Frobenius norm)."""
    e, g = relfro(y, ref), maxrel(y, ref)
    assert e <= tol, f"relative Frobenius error {e:.3e} > {tol}"
    assert g <= ELEM_GUARD, f"element-wise error {g:.3e} > {ELEM_GUARD}"
    return e


def stratified_cols(N, seed, tile=128, inner=2):
    """Output columns for sampled full-size checks: of every `tile`-column
    block, its first and last column and `inner` seeded ones inside."""
    g = np.random.default_rng(seed)
    cols = []
    for c0 in range(0, N, tile):
        c1 = min(N, c0 + tile)
        cols += [c0, c1 - 1]
        cols += list(g.integers(c0, c1, size=inner))
    return np.unique(np.array(cols, dtype=np.int64))


CANARY = 64            # elements of guard bytes on each side of a guarded tensor


def guarded(shape, dtype, fill=None, seed=0):
    """A CUDA tensor of `shape` inside a larger buffer with CANARY elements of
    a seeded bit pattern on each side.  Returns (tensor, check); check()
    asserts that both guard regions still hold their pattern."""
    import torch
    n = int(np.prod(shape))
    item = torch.empty((), dtype=dtype).element_size()
    pat = np.random.default_rng(seed).integers(0, 256, size=2 * CANARY * item, dtype=np.uint8)
    big = torch.empty(n * item + 2 * CANARY * item, dtype=torch.uint8, device="cuda")
    big[:CANARY * item] = torch.from_numpy(pat[:CANARY * item]).cuda()
    big[CANARY * item + n * item:] = torch.from_numpy(pat[CANARY * item:]).cuda()
    t = big[CANARY * item:CANARY * item + n * item].view(dtype).view(*shape)
    if fill is not None:
        t.copy_(torch.as_tensor(np.ascontiguousarray(fill)).to(dtype))

    def check():
        torch.cuda.synchronize()
        b = big.cpu().numpy()
        assert np.array_equal(b[:CANARY * item], pat[:CANARY * item]), "guard bytes before the tensor changed"
        assert np.array_equal(b[CANARY * item + n * item:], pat[CANARY * item:]), \
            "guard bytes after the tensor changed"

    return t, check
