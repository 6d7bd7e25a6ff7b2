"""fc_gguf_run_grouped_noalloc (static device scratch, no allocation) against
fc_gguf_run_grouped, called through the C-ABI: bit-identical outputs on two
calls in a row, the second with fewer tokens, experts and slots (the scratch
keeps the first call's contents), and the size limit."""

import ctypes

import numpy as np
import pytest

from gguf_quant_block_amd import synth

pytestmark = pytest.mark.gpu


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _case(qtype, E, N, K, T, top_k, a_per_slot, idx):
    w = synth.blocks(qtype, E * N, K, synth.rng(120, idx, synth.TAG_BLOCKS))
    A = synth.normal_f16((T, top_k, K) if a_per_slot else (T, K), synth.rng(120, idx, synth.TAG_A))
    ids = synth.moe_routing(T, E, top_k, synth.rng(120, idx, synth.TAG_ROUTING), s=1.1)
    return w, A, ids


def _call(L, fn, h, A, T, a_per_slot, ids, top_k, Y):
    import torch
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return fn(h, ctypes.c_void_p(A.data_ptr()), T, 1 if a_per_slot else 0, ctypes.c_void_p(ids.data_ptr()),
              top_k, ctypes.c_void_p(Y.data_ptr()), st)


@pytest.mark.parametrize("qtype,a_per_slot", [("q6_k", False), ("q5_k", True)])
def test_noalloc_matches_grouped_twice(gpu_lib, qtype, a_per_slot):
    import torch
    from gguf_quant_block_amd.binding import FcGguf
    L = gpu_lib
    # first call: 128 experts, top-8, 256 tokens (the MoE workload's routing
    # size); second: fewer experts routed, fewer tokens and slots
    for E, N, K, T, top_k, idx in ((128, 256, 512, 256, 8, 0), (128, 256, 512, 37, 3, 1)):
        w, A, ids = _case(qtype, E, N, K, T, top_k, a_per_slot, idx)
        fc = FcGguf(N, K, qtype, _dev(w), experts=E)
        Ad, idd = _dev(A), _dev(ids)
        ref = torch.full((T, top_k, N), float("nan"), dtype=torch.float16, device="cuda")
        got = torch.full((T, top_k, N), float("nan"), dtype=torch.float16, device="cuda")
        assert _call(L, L.fc_gguf_run_grouped, fc.handle, Ad, T, a_per_slot, idd, top_k, ref) == 0
        assert _call(L, L.fc_gguf_run_grouped_noalloc, fc.handle, Ad, T, a_per_slot, idd, top_k, got) == 0
        torch.cuda.synchronize()
        r, g = ref.cpu().numpy(), got.cpu().numpy()
        assert np.isfinite(g).all()
        assert np.array_equal(g.view(np.uint16), r.view(np.uint16))


def test_noalloc_size_limit_and_no_op(gpu_lib):
    import torch
    from gguf_quant_block_amd.binding import FcGguf
    L = gpu_lib
    E, N, K = 4096, 16, 256
    w = synth.q6k_blocks(E * N, K, synth.rng(121, 0, synth.TAG_BLOCKS))
    fc = FcGguf(N, K, "q6_k", _dev(w), experts=E)
    # T * top_k pairs whose bucketing needs more than the 512 KB scratch
    T, top_k = 32768, 8
    A = torch.zeros((T, K), dtype=torch.float16, device="cuda")
    ids = torch.zeros((T, top_k), dtype=torch.int32, device="cuda")
    Y = torch.empty((1,), dtype=torch.float16, device="cuda")
    assert _call(L, L.fc_gguf_run_grouped_noalloc, fc.handle, A, T, False, ids, top_k, Y) == -5
    # T == 0 is a no-op
    assert _call(L, L.fc_gguf_run_grouped_noalloc, fc.handle, A, 0, False, ids, top_k, Y) == 0
    torch.cuda.synchronize()
