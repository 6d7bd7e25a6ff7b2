"""The library's launches captured in HIP graphs and run on several streams.

A graph of each entry point (captured after an eager call at the same row
count, so that no workspace is allocated during capture) is replayed several
times, with other eager work and synchronisations between the replays, and
every replay is compared with the eager result bit for bit: every kernel
fixes its summation order (the grouped path too, whose row-to-tile
assignment inside a hot expert follows the order of atomic cursors but
whose per-row summation order does not depend on it).  Two handles run
concurrently on two streams (default priority) give the results they give
alone, and a handle whose workspace grows while another stream is busy
gives the result it gives alone.
"""

import numpy as np
import pytest

from gguf_quant_block_amd import synth
from helpers import case

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _dev(x):
    return _torch().from_numpy(np.ascontiguousarray(x)).cuda()


def _host(t):
    _torch().cuda.synchronize()
    return t.cpu().numpy()


def _replays(call, out, n=3, between=None):
    """Capture call() (which writes out) in a graph and replay it n times,
    with `between` (eager work) and a synchronisation before each replay;
    returns the host copy of out after each replay."""
    torch = _torch()
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    got = []
    for i in range(n):
        out.fill_(float("nan") if out.dtype.is_floating_point else 0)
        if between is not None:
            between(i)
        torch.cuda.synchronize()
        g.replay()
        got.append(_host(out))
    return got


def _fc(w, qtype, N, K, path=None):
    from gguf_quant_block_amd.binding import FcGguf
    f = FcGguf(N, K, qtype, w)
    if path:
        f.set_path(path)
    return f


# (path, M): decode at one row and at a chunked row count, prefill on the
# few-row kernel (16), the loader-wave tile with split-K partials in the
# workspace (64) and without (256), the int8 variant
CASES = [("decode", 1), ("decode", 9), ("prefill", 16), ("prefill", 64), ("prefill", 256),
         ("int8", 64)]


@pytest.mark.parametrize("qtype", ["q5_k", "q6_k"])
@pytest.mark.parametrize("path,M", CASES)
def test_graph_replay_matches_eager(gpu_lib, qtype, path, M):
    torch = _torch()
    N, K = 384, 2048
    w, A, R = case(qtype, M, N, K, 95, M)
    f = _fc(w, qtype, N, K, path)
    Ad, Rd = _dev(A), _dev(R)
    ref = _host(f(Ad, Rd))
    out = torch.empty_like(Rd)
    # eager work between the replays: another handle, another row count
    w2, A2, _ = case(qtype, 3, N, K, 96, M, with_r=False)
    f2 = _fc(w2, qtype, N, K)
    A2d = _dev(A2)
    for y in _replays(lambda: f(Ad, Rd, out=out), out, between=lambda i: f2(A2d)):
        assert np.array_equal(y.view(np.uint16), ref.view(np.uint16))


def test_graph_replay_f32_decode(gpu_lib):
    torch = _torch()
    qtype, M, N, K = "q5_k", 2, 256, 1024
    w, A, R = case(qtype, M, N, K, 97, 0)
    f = _fc(w, qtype, N, K)
    Ad = _dev(A.astype(np.float32))
    Rd = _dev(R.astype(np.float32))
    ref = _host(f(Ad, Rd))
    out = torch.empty_like(Rd)
    for y in _replays(lambda: f(Ad, Rd, out=out), out):
        assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("a_per_slot", [False, True])
def test_graph_replay_grouped(gpu_lib, a_per_slot):
    torch = _torch()
    from gguf_quant_block_amd.binding import FcGguf
    E, N, K, T, top_k = 16, 256, 1024, 48, 4
    ids = synth.moe_routing(T, E, top_k, synth.rng(98, 0, synth.TAG_ROUTING), s=1.1)
    w = synth.q6k_blocks(E * N, K, synth.rng(98, 0, synth.TAG_BLOCKS))
    f = FcGguf(N, K, "q6_k", _dev(w), experts=E)
    shape = (T, top_k, K) if a_per_slot else (T, K)
    Ad = _dev(synth.normal_f16(shape, synth.rng(98, 0, synth.TAG_A)))
    idd = _dev(ids)
    out = torch.empty((T, top_k, N), dtype=torch.float16, device="cuda")
    f.grouped(Ad, idd, a_per_slot, out=out)
    ref = _host(out)
    for y in _replays(lambda: f.grouped(Ad, idd, a_per_slot, out=out), out):
        assert np.array_equal(y.view(np.uint16), ref.view(np.uint16))


def test_two_handles_on_two_streams(gpu_lib):
    torch = _torch()
    qtype, N, K = "q5_k", 512, 2048
    wa, Aa, Ra = case(qtype, 1, N, K, 99, 0)
    wb, Ab, Rb = case(qtype, 64, N, K, 99, 1)
    fa, fb = _fc(wa, qtype, N, K), _fc(wb, qtype, N, K)
    Aad, Rad, Abd, Rbd = _dev(Aa), _dev(Ra), _dev(Ab), _dev(Rb)
    ref_a, ref_b = _host(fa(Aad, Rad)), _host(fb(Abd, Rbd))
    ya, yb = torch.empty_like(Rad), torch.empty_like(Rbd)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(sa):
            for _ in range(4):
                fa(Aad, Rad, out=ya)
        with torch.cuda.stream(sb):
            for _ in range(4):
                fb(Abd, Rbd, out=yb)
        torch.cuda.synchronize()
        assert np.array_equal(_host(ya).view(np.uint16), ref_a.view(np.uint16))
        assert np.array_equal(_host(yb).view(np.uint16), ref_b.view(np.uint16))


def test_workspace_growth_with_another_stream_busy(gpu_lib):
    # the workspace of handle b grows (split-K partials at a larger row
    # count) on stream sb while stream sa runs handle a; both results equal
    # their stand-alone results
    torch = _torch()
    qtype, N, K = "q6_k", 256, 8192
    wa, Aa, Ra = case(qtype, 512, 1024, 2048, 100, 0)
    wb, Ab, Rb = case(qtype, 512, N, K, 100, 1)
    fa, fb = _fc(wa, qtype, 1024, 2048), _fc(wb, qtype, N, K)
    Aad, Rad, Abd, Rbd = _dev(Aa), _dev(Ra), _dev(Ab), _dev(Rb)
    ref_a = _host(fa(Aad, Rad))
    fb_small = _fc(wb, qtype, N, K)
    ref_b = _host(fb_small(Abd, Rbd))
    # grow b's workspace step by step: 16 rows, then 512
    fb(Abd[:16], Rbd[:16])
    torch.cuda.synchronize()
    ya, yb = torch.empty_like(Rad), torch.empty_like(Rbd)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(sa):
        for _ in range(20):
            fa(Aad, Rad, out=ya)
    with torch.cuda.stream(sb):
        fb(Abd, Rbd, out=yb)
    torch.cuda.synchronize()
    assert np.array_equal(_host(ya).view(np.uint16), ref_a.view(np.uint16))
    assert np.array_equal(_host(yb).view(np.uint16), ref_b.view(np.uint16))
