"""Pins for the oracle's Q6_K plane regroup (CPU only).

OpenVINO PR #39119, section Transformation: Q6_K blocks are regrouped once
into the planes QL[nblk][128] | QH[nblk][64] | SC[nblk][16] | D[nblk] without
changing their size or contents.  Checked as a byte permutation: the inverse
restores the input, sizes and the byte multiset are preserved, and every
plane slice is the corresponding AoS field.
"""

import numpy as np

from gguf_quant_block_amd import synth
from oracle import kquant as kq


def test_regroup_round_trip_and_size():
    for N, K in ((1, 256), (3, 768), (16, 2048)):
        w = synth.q6k_blocks(N, K, synth.rng(98, N, 0))
        p = kq.q6k_regroup(w)
        assert p.size == w.size
        assert np.array_equal(np.sort(p), np.sort(w.reshape(-1)))
        assert np.array_equal(kq.q6k_ungroup(p, N, K), w)


def test_plane_slices_are_fields():
    N, K = 5, 1024
    w = synth.q6k_blocks(N, K, synth.rng(98, 7, 0))
    blk = w.reshape(-1, 210)
    nblk = blk.shape[0]
    p = kq.q6k_regroup(w)
    for b in range(nblk):
        assert np.array_equal(p[128 * b:128 * b + 128], blk[b, 0:128])
        assert np.array_equal(p[128 * nblk + 64 * b:128 * nblk + 64 * b + 64], blk[b, 128:192])
        assert np.array_equal(p[192 * nblk + 16 * b:192 * nblk + 16 * b + 16], blk[b, 192:208])
        assert np.array_equal(p[208 * nblk + 2 * b:208 * nblk + 2 * b + 2], blk[b, 208:210])


def test_plane_offsets_are_16_byte_aligned():
    # nblk = N*K/256 with K % 256 == 0 means nblk is a whole number and the
    # plane offsets 128*nblk, 192*nblk, 208*nblk are multiples of 16.
    for nblk in (1, 8, 4096, 384768):
        for off in (128 * nblk, 192 * nblk, 208 * nblk):
            assert off % 16 == 0
