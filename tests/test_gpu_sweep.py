"""Seeded random sweep: qtype, N, K, M, path (with f32 activations as a
path of its own), residual and prefill kernel (the default, or the few-row
kernel or the loader-wave tile forced) drawn at random (N up to 1499, K up
to 4096, M over the tile ladder's edges), each case checked against the oracle with its
path's bar: the int8 emulation within 1e-3 (max relative) for the decode,
f32 and int8 paths, the fp64 FC within 2e-3 (relative Frobenius) for the
prefill and dequantise-once paths."""

import numpy as np
import pytest

from oracle import fc as ofc
from helpers import DECODE_TOL, case, check_fro, maxrel

pytestmark = pytest.mark.gpu

MS = [1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 33, 64, 100, 129, 200]
PATHS = ["auto", "decode", "prefill", "int8", "scratch", "f32"]


KERNELS = [None, "skinny", "dma"]     # FC_GGUF_PREFILL_KERNEL: the default, or one forced


def _draw(seed):
    g = np.random.default_rng(seed)
    d = (["q4_k", "q5_k", "q6_k"][g.integers(3)], int(g.integers(1, 1500)),
         256 * int(g.integers(1, 17)), int(g.choice(MS)), PATHS[g.integers(len(PATHS))],
         bool(g.integers(2)))
    return d + (KERNELS[g.integers(len(KERNELS))],)


@pytest.mark.parametrize("seed", range(120))
def test_random_case(gpu_lib, monkeypatch, seed):
    import torch
    from gguf_quant_block_amd.binding import FcGguf
    qtype, N, K, M, path, with_r, kernel = _draw(1000 + seed)
    w, A, R = case(qtype, M, N, K, 700, seed, with_r=with_r)
    if path == "f32":
        A = A.astype(np.float32)
        R = None if R is None else R.astype(np.float32)
    # the prefill kernel is read when the handle is created
    if kernel:
        monkeypatch.setenv("FC_GGUF_PREFILL_KERNEL", kernel)
    else:
        monkeypatch.delenv("FC_GGUF_PREFILL_KERNEL", raising=False)
    f = FcGguf(N, K, qtype, w)
    monkeypatch.delenv("FC_GGUF_PREFILL_KERNEL", raising=False)
    if path != "f32":
        f.set_path(path)
    y = f(torch.from_numpy(A).cuda(), None if R is None else torch.from_numpy(R).cuda())
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.isfinite(y).all()
    if path in ("decode", "int8", "f32") or (path == "auto" and M < 8):
        assert maxrel(y, ofc.fc_ref_int8(A, w, qtype, R)) <= DECODE_TOL
    else:
        check_fro(y, ofc.fc_gguf_ref(A, w, qtype, R))
