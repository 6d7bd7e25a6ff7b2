#!/usr/bin/env python3
"""Benchmark of the GGUF K-quant FC library on one MI355X.

Metric: decode GEMV weight GB/s at M = 1 (Q5_K, Phi-3.5-mini layer set), with
prefill TFLOPS at M = 512 (Q5_K and Q6_K, [8192, 2048] and [2048, 8192]).  All
five workloads are timed in the same step, each case with its rate and its
fraction of the published peak that bounds it:
  * cfg0  one Q6_K FC [512, 2048], M = 1 (decode path) and M = 16 (prefill);
  * cfg1  Q5_K decode GEMV, Phi-3.5-mini layer set (qkv [9216, 3072], o_proj
          [3072, 3072], gate_up [16384, 3072], down [3072, 8192]) at M = 1, 2,
          4, 7, f16 residual fused;
  * cfg2  Q6_K decode GEMV, the same four shapes at M = 1, 4 with the
          residual, and the output projection [32064, 3072] at M = 1, 4
          without it;
  * cfg3  prefill, Q5_K and Q6_K on [8192, 2048] and [2048, 8192] at M = 8,
          64, 128, 256, 512, 2048, residual fused;
  * cfg4  MoE: Q6_K experts, 128 experts, top-8, 256 tokens, Zipf(1.1)
          routing: gate/up [768, 2048] (bucketing + grouped FC) then down
          [2048, 768] on the same routing's bucketing (grouped FC only);
  * the widened paths (Q4_K decode and prefill, f32 activations).
Every case is one phase of the step: a HIP graph of launches over distinct
device copies of its weights (at least 1 GiB of them per decode shape, 0.5
GiB per prefill shape, so the weights stream from HBM rather than from the
256 MB last-level cache), replayed once per step; HIP events on the replay
stream time each phase.  A case's time per launch is its phase time over
its launch count.  Weights and activations are resident in HBM before
timing.

Outside the timed steps: the measured ceilings (a plain coalesced read at
the decode shapes' byte counts and at 1 GiB, best grid; back-to-back f16 and
int8 matrix-core instructions), the dequantise-once and int8 comparison
paths, and the CPU oracle timed on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --pmc-target | --pmc-prefill-target | --pmc-prefill4-target |
                       --pmc-skinny-target | --pmc-moe-target | --pmc-int8-target
       python bench.py --traffic-summary FETCH_CSV WRITE_CSV
       python bench.py --prefill-traffic-summary FETCH_CSV WRITE_CSV
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2516.6   # MI355X dense f16 matrix cores
INT8_MFMA_PEAK_TOPS = 5033.2    # MI355X dense int8 matrix cores
ROTATE_DECODE = 1 << 30         # bytes of distinct weight copies per decode case
ROTATE_PREFILL = 1 << 29        # ... per prefill case
MOE_COPIES = 7                  # 7 x 165 MB per expert FC
CPU_LAYERS = 6                  # decode oracle sample: 6 layers of the Q5_K set
METRIC = "decode GEMV weight GB/s (M=1); prefill TFLOPS at M=512; Q5_K/Q6_K"


def gemv_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemv.hip", "quant.h", "common.h", "layout.h"):
        with open(os.path.join(ROOT, "gguf_quant_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per decode-GEMV launch from the committed counter summary,
    or None when the kernel source changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "decode_gemv_q5k_m1_traffic.json")
    try:
        with open(p) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("gemv_source_hash") != gemv_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def prefill_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("prefill.hip", "mfma_dma.h", "mfma_tile.h", "common.h", "layout.h"):
        with open(os.path.join(ROOT, "gguf_quant_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def prefill_traffic_from_profile():
    """HBM bytes per M = 512 prefill FC call from the committed counter
    summary, or None when the kernel source changed since the counters were
    taken."""
    p = os.path.join(ROOT, "profiles", "prefill_m512_traffic.json")
    try:
        with open(p) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("prefill_source_hash") != prefill_source_hash():
        return None
    return rec.get("hbm_bytes_per_call")


def moe_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("moe.hip", "mfma_tile.h", "common.h", "layout.h"):
        with open(os.path.join(ROOT, "gguf_quant_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def moe_traffic_from_profile():
    """HBM bytes per grouped (MoE) call from the committed counter summary,
    or None when the kernel source changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "moe_grouped_q6k_traffic.json")
    try:
        with open(p) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("moe_source_hash") != moe_source_hash():
        return None
    return rec.get("hbm_bytes_per_call")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except ImportError:          # pragma: no cover
        return 1


# --------------------------------------------------------------- CPU oracle --

def cpu_baselines():
    """The CPU oracle, timed on bounded samples of three workloads:
    decode (the int8-emulating oracle over CPU_LAYERS layers of the Q5_K
    layer set at M = 1; NumPy, one thread), prefill (the float64 oracle --
    exact decode to float64, then a BLAS dgemm -- on the four M = 512 prefill
    FCs) and MoE (the float64 grouped oracle on one full gate/up call)."""
    import numpy as np
    from gguf_quant_block_amd import synth
    from oracle import fc as ofc
    from oracle import kquant as okq

    cores_avail = len(os.sched_getaffinity(0))
    model = cpu_model()
    out = {}
    # decode: int8 emulation, M = 1
    inputs = []
    for i, (name, (N, K)) in enumerate(synth.PHI35_LAYERS.items()):
        inputs.append((synth.q5k_blocks(N, K, synth.rng(1, i, synth.TAG_BLOCKS)),
                       synth.normal_f16((1, K), synth.rng(1, i, synth.TAG_A)),
                       synth.normal_f16((1, N), synth.rng(1, i, synth.TAG_R))))
    total = 0
    t0 = time.perf_counter()
    for _ in range(CPU_LAYERS):
        for w, A, R in inputs:
            ofc.fc_ref_int8(A, w, "q5_k", R)
            total += w.nbytes
    dt = time.perf_counter() - t0
    out["decode"] = {"value": round(total / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                     "sample": f"{CPU_LAYERS} layers of the Q5_K Phi-3.5-mini layer set at M=1, int8-emulating "
                               f"float64 oracle (NumPy, one thread): {total / 1e6:.1f} MB of weights in {dt:.1f} s",
                     "cpu_model": model, "cores_available": cores_avail}
    # prefill: float64 oracle on the four M = 512 FCs
    flops = 0
    t_dec = t_mm = 0.0
    for q in ("q5_k", "q6_k"):
        for si, (N, K) in enumerate(synth.PREFILL_SHAPES):
            w = synth.blocks(q, N, K, synth.rng(3, 10 * si + 4, synth.TAG_BLOCKS))
            A = synth.normal_f16((512, K), synth.rng(3, 10 * si + 4, synth.TAG_A))
            R = synth.normal_f16((512, N), synth.rng(3, 10 * si + 4, synth.TAG_R))
            t0 = time.perf_counter()
            W = okq.dequantize(w, q)
            t1 = time.perf_counter()
            ofc.fc_ref(A, W, R)
            t2 = time.perf_counter()
            t_dec += t1 - t0
            t_mm += t2 - t1
            flops += 2 * 512 * N * K
    bt = blas_threads()
    out["prefill"] = {"value": round(flops / (t_dec + t_mm) / 1e9, 3), "unit": "GFLOP/s", "cores": bt,
                      "kind": "oracle",
                      "sample": "the four M=512 prefill FCs (Q5_K, Q6_K x [8192,2048], [2048,8192]) with the "
                                f"residual, float64 oracle: decode to float64 {t_dec:.2f} s (NumPy, one thread), "
                                f"dgemm {t_mm:.2f} s (BLAS, {bt} threads)",
                      "cpu_model": model, "cores_available": cores_avail}
    # MoE: one full gate/up call
    m = synth.MOE
    E, T, top_k = m["E"], m["T"], m["top_k"]
    N, K = m["gate_up"]
    ids = synth.moe_routing(T, E, top_k, synth.rng(5, 0, synth.TAG_ROUTING), s=m["zipf_s"])
    w = synth.q6k_blocks(E * N, K, synth.rng(5, 0, synth.TAG_BLOCKS)).reshape(E, N, -1)
    A = synth.normal_f16((T, K), synth.rng(5, 0, synth.TAG_A))
    t0 = time.perf_counter()
    ofc.moe_ref(A, w, "q6_k", ids, False)
    dt = time.perf_counter() - t0
    touched = int((np.bincount(ids.ravel(), minlength=E) > 0).sum()) * N * (K // 256) * 210
    out["moe"] = {"value": round(2 * T * top_k * N * K / dt / 1e9, 3), "unit": "GFLOP/s", "cores": bt,
                  "kind": "oracle",
                  "sample": f"one MoE gate/up call (128 Q6_K experts [768,2048], top-8, 256 tokens, Zipf 1.1), "
                            f"float64 grouped oracle: {dt:.2f} s, {touched / dt / 1e9:.3f} GB/s of touched weights",
                  "cpu_model": model, "cores_available": cores_avail}
    return out


# ------------------------------------------------------------ measurements --

class Ceil:
    """The measured-ceiling kernels (libfcgceil.so)."""

    def __init__(self):
        from gguf_quant_block_amd import build
        if not os.path.exists(build.CEIL_LIB):
            raise RuntimeError(f"{build.CEIL_LIB} is not built")
        L = ctypes.CDLL(build.CEIL_LIB)
        L.fc_ceiling_stream_read.restype = ctypes.c_int
        L.fc_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p]
        L.fc_ceiling_mfma.restype = ctypes.c_int
        L.fc_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        self.L = L


def _graph_time(fn, reps, stream):
    """Capture fn() once as a graph; best per-replay seconds over `reps` replays."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            fn()
    torch.cuda.synchronize()
    best = float("inf")
    with torch.cuda.stream(stream):
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1) / 1e3)
    del g
    return best


def ceilings(dev, sizes):
    """Plain coalesced read at each byte count in `sizes` (launches over
    distinct slices of a 1.1 GiB buffer, one graph per grid) and at 1 GiB,
    best of a grid sweep; and the f16 / int8 matrix-core rate."""
    import torch
    C = Ceil()
    stream = torch.cuda.Stream()
    span = (1 << 30) + (128 << 20)
    buf = torch.empty(span, dtype=torch.uint8, device=dev)
    buf.fill_(7)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    res = {"read": {}, "how": "fc_ceiling_stream_read: 256-thread workgroups, 16-byte loads, grid in "
                              "{256..8192} x unroll in {2,4,8}, best per byte count; back-to-back launches "
                              "over distinct slices covering >= 1 GiB, graph-replayed, HIP events"}
    for name, nbytes in list(sizes.items()) + [("1GiB", 1 << 30)]:
        nbytes = nbytes // 256 * 256
        stride = (nbytes + 4095) // 4096 * 4096
        copies = max(1, min((1 << 30) // max(nbytes, 1), (span - nbytes) // stride + 1))
        best = (float("inf"), None)
        for grid in (256, 512, 1024, 2048, 4096, 8192):
            for unroll in (2, 4, 8):
                def fn(grid=grid, unroll=unroll):
                    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                    for c in range(copies):
                        rc = C.L.fc_ceiling_stream_read(ctypes.c_void_p(buf.data_ptr() + c * stride), nbytes,
                                                        grid, unroll, ctypes.c_void_p(sink.data_ptr()), st)
                        assert rc == 0
                t = _graph_time(fn, 3, stream) / copies
                if t < best[0]:
                    best = (t, (grid, unroll))
        res["read"][name] = {"bytes": nbytes, "us": round(best[0] * 1e6, 3),
                             "gbps": round(nbytes / best[0] / 1e9, 1),
                             "frac_of_hbm_peak": round(nbytes / best[0] / 1e9 / HBM_PEAK_GBPS, 4),
                             "grid": best[1][0], "unroll": best[1][1], "launches": copies}
    del buf
    # matrix cores: 4 waves per workgroup, 4 independent 32x32 MFMAs per round
    mf = {}
    for dtype, name, ops_per in ((0, "f16", 32768), (1, "int8", 65536)):
        best = (0.0, None)
        for wg_per_cu in (1, 2):
            grid = 256 * wg_per_cu
            iters = 4096

            def fn(grid=grid, dtype=dtype, iters=iters):
                st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for _ in range(4):
                    assert C.L.fc_ceiling_mfma(dtype, iters, grid, ctypes.c_void_p(sink.data_ptr()), st) == 0
            t = _graph_time(fn, 3, stream) / 4
            rate = grid * 4 * iters * 4 * ops_per / t / 1e12
            if rate > best[0]:
                # one wave per SIMD issues 4 * iters MFMAs of 32 cycles each
                # (at 2.4 GHz the published peak); the implied clock follows
                clk = 4 * iters * 32 * wg_per_cu / t / 1e9
                best = (rate, {"workgroups_per_cu": wg_per_cu, "implied_clock_ghz": round(clk, 3)})
        peak = F16_MFMA_PEAK_TFLOPS if dtype == 0 else INT8_MFMA_PEAK_TOPS
        mf[name] = {"rate": round(best[0], 1), "unit": "TFLOP/s" if dtype == 0 else "TOP/s",
                    "frac_of_peak": round(best[0] / peak, 4), **best[1]}
    res["mfma"] = mf
    res["mfma_how"] = ("fc_ceiling_mfma: 4 waves per workgroup, 256 or 512 workgroups, 4096 rounds of 4 independent "
                       "v_mfma_f32_32x32x16_f16 (or v_mfma_i32_32x32x32_i8) per wave; implied clock = 32 cycles per "
                       "MFMA per SIMD")
    return res


def scratch_comparison(prefill_calls, dev, iters=10):
    """TFLOPS of the direct prefill path and of the dequantise-once path (f16
    weights + rocBLAS GEMM, the residual as beta*C) on the prefill FCs, per M."""
    import torch
    from gguf_quant_block_amd import synth

    out = {"workload": "Q5_K and Q6_K, [8192,2048] and [2048,8192], fused residual; "
                       "dequantise-once = the weights decoded to an f16 buffer on every call "
                       "(not retained), then rocBLAS gemm_ex (f16 in, f32 compute); eager launches"}
    for M in (512, 1024, 2048):
        res = {}
        for path in ("prefill", "scratch"):
            flops, calls = 0, []
            for fc in prefill_calls:
                K, N = fc.K, fc.N
                A = torch.from_numpy(synth.normal_f16((M, K), synth.rng(8, M, synth.TAG_A))).to(dev)
                R = torch.from_numpy(synth.normal_f16((M, N), synth.rng(8, M, synth.TAG_R))).to(dev)
                Y = torch.empty((M, N), dtype=torch.float16, device=dev)
                calls.append((fc, A, R, Y))
                flops += 2 * M * N * K
            for fc, *_ in calls:
                fc.set_path(path)
            for fc, A, R, Y in calls:
                fc(A, R, out=Y)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                for fc, A, R, Y in calls:
                    fc(A, R, out=Y)
            e1.record()
            torch.cuda.synchronize()
            s = e0.elapsed_time(e1) / 1e3 / iters
            res[path] = round(flops / s / 1e12, 1)
            for fc, *_ in calls:
                fc.set_path("auto")
        out[f"m{M}"] = {"direct_tflops": res["prefill"], "dequant_once_tflops": res["scratch"]}
    return out


def int8_comparison(prefill_calls, dev, iters=10):
    """The int8 matrix-core prefill variant against the f16 prefill path on the
    prefill FCs at M = 512, eager launches; int8 multiply-adds count 2 ops."""
    import torch
    from gguf_quant_block_amd import synth

    M = 512
    out = {"workload": "Q5_K and Q6_K, [8192,2048] and [2048,8192], M=512, fused residual; "
                       "the variant's quantisation pass included; eager launches",
           "peak_int8_tops": INT8_MFMA_PEAK_TOPS}
    for path in ("prefill", "int8"):
        ops, calls = 0, []
        for fc in prefill_calls:
            K, N = fc.K, fc.N
            A = torch.from_numpy(synth.normal_f16((M, K), synth.rng(9, M, synth.TAG_A))).to(dev)
            R = torch.from_numpy(synth.normal_f16((M, N), synth.rng(9, M, synth.TAG_R))).to(dev)
            Y = torch.empty((M, N), dtype=torch.float16, device=dev)
            calls.append((fc, A, R, Y))
            ops += 2 * M * N * K
        for fc, *_ in calls:
            fc.set_path(path)
        for fc, A, R, Y in calls:
            fc(A, R, out=Y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            for fc, A, R, Y in calls:
                fc(A, R, out=Y)
        e1.record()
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) / 1e3 / iters
        key = "f16_prefill" if path == "prefill" else "int8_mfma"
        out[key + "_tops"] = round(ops / s / 1e12, 1)
        out[key + "_us_per_fc"] = round(s * 1e6 / len(calls), 2)
        for fc, *_ in calls:
            fc.set_path("auto")
    out["int8_frac_of_int8_peak"] = round(out["int8_mfma_tops"] / INT8_MFMA_PEAK_TOPS, 4)
    return out


# ------------------------------------------------------- counter targets ----

def pmc_target(dev):
    """Counter-collection target: the decode GEMVs of the Q5_K layer set at
    M = 1, plus a plain device copy of 256 MiB whose FETCH_SIZE / WRITE_SIZE
    readings give the counters' scale factors."""
    import torch
    from gguf_quant_block_amd import synth
    from gguf_quant_block_amd.binding import FcGguf
    fcs = []
    for i, (name, (N, K)) in enumerate(synth.PHI35_LAYERS.items()):
        w = torch.from_numpy(synth.q5k_blocks(N, K, synth.rng(1, i, synth.TAG_BLOCKS))).to(dev)
        A = torch.from_numpy(synth.normal_f16((1, K), synth.rng(1, i, synth.TAG_A))).to(dev)
        R = torch.from_numpy(synth.normal_f16((1, N), synth.rng(1, i, synth.TAG_R))).to(dev)
        Y = torch.empty((1, N), dtype=torch.float16, device=dev)
        for _ in range(4):
            fcs.append((FcGguf(N, K, "q5_k", w), A, R, Y))
    for _ in range(3):
        for fc, A, R, Y in fcs:
            fc(A, R, out=Y)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("pmc target done", flush=True)


def pmc_prefill_target(dev):
    """Counter-collection target for the prefill kernel: the Q5_K FC on
    [8192, 2048] at M = 512, ten eager launches, then a 256 MiB device copy."""
    import torch
    from gguf_quant_block_amd import synth
    from gguf_quant_block_amd.binding import FcGguf
    N, K = synth.PREFILL_SHAPES[0]
    M = 512
    w = torch.from_numpy(synth.q5k_blocks(N, K, synth.rng(2, 0, synth.TAG_BLOCKS))).to(dev)
    A = torch.from_numpy(synth.normal_f16((M, K), synth.rng(2, 0, synth.TAG_A))).to(dev)
    R = torch.from_numpy(synth.normal_f16((M, N), synth.rng(2, 0, synth.TAG_R))).to(dev)
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    fc = FcGguf(N, K, "q5_k", w)
    for _ in range(10):
        fc(A, R, out=Y)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("pmc prefill target done", flush=True)


def pmc_skinny_target(dev):
    """Counter-collection target for the few-row prefill kernel: the Q5_K
    FC on [8192, 2048] at M = 8 (one row tile per workgroup, two
    workgroups per CU), ten eager launches, then three 256 MiB device
    copies."""
    import torch
    from gguf_quant_block_amd import synth
    from gguf_quant_block_amd.binding import FcGguf
    N, K = synth.PREFILL_SHAPES[0]
    M = 8
    w = torch.from_numpy(synth.q5k_blocks(N, K, synth.rng(2, 7, synth.TAG_BLOCKS))).to(dev)
    A = torch.from_numpy(synth.normal_f16((M, K), synth.rng(2, 7, synth.TAG_A))).to(dev)
    R = torch.from_numpy(synth.normal_f16((M, N), synth.rng(2, 7, synth.TAG_R))).to(dev)
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    fc = FcGguf(N, K, "q5_k", w)
    for _ in range(10):
        fc(A, R, out=Y)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("pmc skinny target done", flush=True)


PREFILL4_CALLS = 3      # eager calls of each of the four M = 512 FCs in --pmc-prefill4-target


def prefill4_fcs():
    """The four M = 512 prefill FCs of the benchmark, in target order."""
    from gguf_quant_block_amd import synth
    return [(q, N, K) for q in ("q5_k", "q6_k") for (N, K) in synth.PREFILL_SHAPES]


def pmc_prefill4_target(dev):
    """Counter-collection target for the prefill FC traffic: the four M = 512
    FCs (Q5_K, Q6_K x [8192, 2048], [2048, 8192]) with the residual,
    PREFILL4_CALLS eager calls each, then three 256 MiB device copies."""
    import torch
    from gguf_quant_block_amd import synth
    from gguf_quant_block_amd.binding import FcGguf
    M = 512
    for i, (q, N, K) in enumerate(prefill4_fcs()):
        w = torch.from_numpy(synth.blocks(q, N, K, synth.rng(2, i, synth.TAG_BLOCKS))).to(dev)
        A = torch.from_numpy(synth.normal_f16((M, K), synth.rng(2, i, synth.TAG_A))).to(dev)
        R = torch.from_numpy(synth.normal_f16((M, N), synth.rng(2, i, synth.TAG_R))).to(dev)
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
        fc = FcGguf(N, K, q, w)
        fc(A, R, out=Y)                       # the workspace grows here, before the counted calls
        torch.cuda.synchronize()
        for _ in range(PREFILL4_CALLS):
            fc(A, R, out=Y)
        torch.cuda.synchronize()
        del fc, w
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("pmc prefill4 target done", flush=True)


def pmc_moe_target(dev):
    """Counter-collection target for the grouped path: the benchmark's first
    routing and weight copy, gate/up then down (on gate/up's bucketing),
    three eager rounds."""
    import torch
    from gguf_quant_block_amd import synth
    from gguf_quant_block_amd.binding import FcGguf
    m = synth.MOE
    E, T, top_k = m["E"], m["T"], m["top_k"]
    ids = torch.from_numpy(synth.moe_routing(T, E, top_k, synth.rng(5, 0, synth.TAG_ROUTING),
                                             s=m["zipf_s"])).to(dev)
    fcs = []
    for fi, (which, per_slot) in enumerate((("gate_up", False), ("down", True))):
        N, K = m[which]
        w = torch.from_numpy(synth.q6k_blocks(E * N, K, synth.rng(5, fi, synth.TAG_BLOCKS))).to(dev)
        fcs.append((FcGguf(N, K, "q6_k", w, experts=E), per_slot, N, K))
    calls = []
    for fc, per_slot, N, K in fcs:
        shape = (T, top_k, K) if per_slot else (T, K)
        A = torch.from_numpy(synth.normal_f16(shape, synth.rng(5, len(calls), synth.TAG_A))).to(dev)
        calls.append((fc, A, per_slot, torch.empty((T, top_k, N), dtype=torch.float16, device=dev)))
    for _ in range(3):
        # gate/up sorts the routing; down runs on its bucketing
        (up, A0, p0, Y0), (down, A1, p1, Y1) = calls
        up.grouped(A0, ids, p0, out=Y0)
        down.grouped(A1, ids, p1, out=Y1, routed=up)
    torch.cuda.synchronize()
    print("pmc moe target done", flush=True)


def pmc_int8_target(dev):
    """Counter-collection target for the int8 matrix-core prefill variant:
    the Q5_K FC on [8192, 2048] at M = 512 on the int8 path, ten eager
    launches (each: quant_i8_kernel, then prefill_i8_kernel)."""
    import torch
    from gguf_quant_block_amd import synth
    from gguf_quant_block_amd.binding import FcGguf
    N, K = synth.PREFILL_SHAPES[0]
    M = 512
    w = torch.from_numpy(synth.q5k_blocks(N, K, synth.rng(2, 0, synth.TAG_BLOCKS))).to(dev)
    A = torch.from_numpy(synth.normal_f16((M, K), synth.rng(2, 0, synth.TAG_A))).to(dev)
    R = torch.from_numpy(synth.normal_f16((M, N), synth.rng(2, 0, synth.TAG_R))).to(dev)
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    fc = FcGguf(N, K, "q5_k", w)
    fc.set_path("int8")
    for _ in range(10):
        fc(A, R, out=Y)
    torch.cuda.synchronize()
    print("pmc int8 target done", flush=True)


CALIB_BYTES = 256 << 20


def traffic_summary(fetch_csv, write_csv):
    """Turn the two counter passes over --pmc-target into HBM bytes per decode
    GEMV launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled
    by what they read for the 256 MiB device copy, then averaged over the GEMV
    dispatches (an equal mix of the four shapes)."""
    import csv
    from gguf_quant_block_amd import synth

    def read(path, counter):
        gemv, calib = [], []
        with open(path) as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r.get("Dispatch_Id") or 0))
        for r in rows:
            v = float(r["Counter_Value"]) * 1024.0
            if "gemv_kernel" in r["Kernel_Name"]:
                gemv.append((len(gemv), v))
            elif "copyBuffer" in r["Kernel_Name"]:
                calib.append(v)
        return gemv, calib

    fg, fc = read(fetch_csv, "FETCH_SIZE")
    wg, wc = read(write_csv, "WRITE_SIZE")
    # the calibration copies are the last three device copies of the run
    f_factor = CALIB_BYTES / (sum(fc[-3:]) / 3)
    w_factor = CALIB_BYTES / (sum(wc[-3:]) / 3)
    fetch = sum(v for _, v in fg) / len(fg) * f_factor
    write = sum(v for _, v in wg) / len(wg) * w_factor
    alg = sum(N * (K // 256) * 176 + 2 * K + 4 * N for N, K in synth.PHI35_LAYERS.values()) / len(synth.PHI35_LAYERS)
    # --pmc-target dispatches, per pass, 4 launches of each shape in layer order
    names = list(synth.PHI35_LAYERS)
    per_shape = {}
    for (i, fv), (_, wv) in zip(fg, wg):
        per_shape.setdefault(names[(i % (4 * len(names))) // 4], []).append(fv * f_factor + wv * w_factor)
    rec = {
        "kernel": "gemv_kernel<Q5_K, M=1>",
        "workload": "Q5_K decode GEMV at M=1 over the Phi-3.5-mini layer set, equal mix of the four shapes",
        "gemv_source_hash": gemv_source_hash(),
        "gemv_dispatches": len(fg),
        "fetch_factor": round(f_factor, 4),
        "write_factor": round(w_factor, 4),
        "hbm_fetch_bytes_per_launch": round(fetch),
        "hbm_write_bytes_per_launch": round(write),
        "hbm_bytes_per_launch": round(fetch + write),
        "algorithmic_bytes_per_launch": round(alg),
        "traffic_over_algorithmic": round((fetch + write) / alg, 4),
        "hbm_bytes_per_launch_by_shape": {k: round(sum(v) / len(v)) for k, v in per_shape.items()},
    }
    out = os.path.join(ROOT, "profiles", "decode_gemv_q5k_m1_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def prefill_traffic_summary(fetch_csv, write_csv):
    """Turn the two counter passes over --pmc-prefill4-target into HBM bytes
    per prefill FC call (the loader-wave tile plus, for a split-K grid, its
    reduction): each counter scaled by what it reads for the 256 MiB device
    copy; per FC, the dispatches of its counted calls (the first call of each
    FC, which grows the workspace, is left out) over the call count."""
    import csv

    def read(path, counter):
        with open(path) as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r.get("Dispatch_Id") or 0))
        fcs, calib, cur = [], [], None
        for r in rows:
            name = r["Kernel_Name"]
            v = float(r["Counter_Value"]) * 1024.0
            if "copyBuffer" in name:
                calib.append(v)
            elif "prefill_dma_kernel" in name:
                cur = [v]
                fcs.append(cur)
            elif "splitk_reduce_kernel" in name and cur is not None:
                cur.append(v)
        return [sum(c) for c in fcs], calib

    fcalls, fc = read(fetch_csv, "FETCH_SIZE")
    wcalls, wc = read(write_csv, "WRITE_SIZE")
    per = PREFILL4_CALLS + 1
    assert len(fcalls) == len(wcalls) == 4 * per, (len(fcalls), len(wcalls))
    f_factor = CALIB_BYTES / (sum(fc[-3:]) / 3)
    w_factor = CALIB_BYTES / (sum(wc[-3:]) / 3)
    M = 512
    bb = {"q4_k": 144, "q5_k": 176, "q6_k": 210}
    by_fc, alg_by_fc = {}, {}
    for i, (q, N, K) in enumerate(prefill4_fcs()):
        calls = range(i * per + 1, (i + 1) * per)
        b = sum(fcalls[j] * f_factor + wcalls[j] * w_factor for j in calls) / PREFILL4_CALLS
        key = f"{q}_{N}x{K}"
        by_fc[key] = round(b)
        alg_by_fc[key] = N * (K // 256) * bb[q] + 2 * M * K + 4 * M * N
    hbm = sum(by_fc.values()) / 4
    alg = sum(alg_by_fc.values()) / 4
    rec = {
        "kernel": "prefill_dma_kernel (+ splitk_reduce_kernel where K is split)",
        "workload": "the four M = 512 prefill FCs (Q5_K, Q6_K x [8192, 2048], [2048, 8192]) "
                    "with the residual, equal mix",
        "prefill_source_hash": prefill_source_hash(),
        "fc_calls_counted": 4 * PREFILL4_CALLS,
        "fetch_factor": round(f_factor, 4),
        "write_factor": round(w_factor, 4),
        "hbm_bytes_per_call": round(hbm),
        "algorithmic_bytes_per_call": round(alg),
        "traffic_over_algorithmic": round(hbm / alg, 4),
        "hbm_bytes_per_call_by_fc": by_fc,
        "algorithmic_bytes_per_call_by_fc": alg_by_fc,
    }
    out = os.path.join(ROOT, "profiles", "prefill_m512_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def moe_traffic_summary(fetch_csv, write_csv):
    """Turn the two counter passes over --pmc-moe-target into HBM bytes per
    grouped call: gate/up (bucketing + grouped FC) and down (grouped FC on
    gate/up's bucketing), three rounds each, the counters scaled by the
    factors the decode record measured on the 256 MiB device copy."""
    import csv

    import numpy as np
    from gguf_quant_block_amd import synth

    with open(os.path.join(ROOT, "profiles", "decode_gemv_q5k_m1_traffic.json")) as f:
        dec = json.load(f)
    f_factor, w_factor = dec["fetch_factor"], dec["write_factor"]

    def read(path, counter):
        with open(path) as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r.get("Dispatch_Id") or 0))
        calls, cur = [], 0.0
        for r in rows:
            v = float(r["Counter_Value"]) * 1024.0
            if "moe_bucket_kernel" in r["Kernel_Name"]:
                cur += v
            elif "moe_grouped_kernel" in r["Kernel_Name"]:
                calls.append(cur + v)
                cur = 0.0
        return calls

    fc, wc = read(fetch_csv, "FETCH_SIZE"), read(write_csv, "WRITE_SIZE")
    assert len(fc) == len(wc) == 6, (len(fc), len(wc))
    per = [fc[i] * f_factor + wc[i] * w_factor for i in range(6)]
    m = synth.MOE
    E, T, top_k = m["E"], m["T"], m["top_k"]
    ids = synth.moe_routing(T, E, top_k, synth.rng(5, 0, synth.TAG_ROUTING), s=m["zipf_s"])
    nonempty = int((np.bincount(ids.ravel(), minlength=E) > 0).sum())
    alg = {}
    for which, per_slot in (("gate_up", False), ("down", True)):
        N, K = m[which]
        a_elems = T * top_k * K if per_slot else T * K
        alg[which] = nonempty * N * (K // 256) * 210 + 2 * a_elems + 2 * T * top_k * N
    hbm = {"gate_up": sum(per[0::2]) / 3, "down": sum(per[1::2]) / 3}
    rec = {
        "kernel": "moe_bucket_kernel + moe_grouped_kernel (Q6_K)",
        "workload": "128 experts, top-8, 256 tokens, Zipf(1.1): gate/up [768, 2048] on token rows "
                    "(bucketing + grouped FC), down [2048, 768] on pair rows (grouped FC on gate/up's "
                    "bucketing); the benchmark's first routing and weight copy",
        "moe_source_hash": moe_source_hash(),
        "calls_counted": 6,
        "fetch_factor": f_factor,
        "write_factor": w_factor,
        "hbm_bytes_per_call": round((hbm["gate_up"] + hbm["down"]) / 2),
        "algorithmic_bytes_per_call": round((alg["gate_up"] + alg["down"]) / 2),
        "traffic_over_algorithmic": round((hbm["gate_up"] + hbm["down"]) / (alg["gate_up"] + alg["down"]), 4),
        "hbm_bytes_per_call_by_fc": {k: round(v) for k, v in hbm.items()},
        "algorithmic_bytes_per_call_by_fc": alg,
    }
    out = os.path.join(ROOT, "profiles", "moe_grouped_q6k_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


# ----------------------------------------------------------------- main ----

class Case:
    """One timed phase: `calls` (fc, A, R, Y) run in order as one graph."""

    def __init__(self, key, calls, *, kind, weight_bytes=0, alg_bytes=0, flops=0, grouped=False, info=None):
        self.key, self.calls, self.kind = key, calls, kind
        self.weight_bytes, self.alg_bytes, self.flops = weight_bytes, alg_bytes, flops
        self.grouped = grouped
        self.info = info or {}
        self.times = []

    def run(self):
        if self.grouped:
            for fc, A, ids, per_slot, Y, routed in self.calls:
                fc.grouped(A, ids, per_slot, out=Y, routed=routed)
        else:
            for fc, A, R, Y in self.calls:
                fc(A, R, out=Y)

    @property
    def launches(self):
        return len(self.calls)

    def seconds(self):
        return sum(self.times) / len(self.times)

    def summary(self):
        s = self.seconds()
        d = {"us_per_launch": round(s * 1e6 / self.launches, 3), "launches": self.launches}
        if self.weight_bytes:
            gb = self.weight_bytes / s / 1e9
            d["weight_gbps"] = round(gb, 1)
        if self.alg_bytes:
            a = self.alg_bytes / s / 1e9
            d["alg_gbps"] = round(a, 1)
            d["frac_of_hbm_peak"] = round(a / HBM_PEAK_GBPS, 4)
        if self.flops:
            tf = self.flops / s / 1e12
            d["tflops"] = round(tf, 2)
            d["frac_of_f16_peak"] = round(tf / F16_MFMA_PEAK_TFLOPS, 4)
        d.update(self.info)
        return d


def copies_for(nbytes, budget):
    return max(4, math.ceil(budget / nbytes))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the ceilings and the comparison paths (outside the timed steps)")
    ap.add_argument("--pmc-target", action="store_true",
                    help="run the decode GEMVs eagerly (4 shapes x 4 weight copies x 3 passes) and a "
                         "256 MiB device copy of known size, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--pmc-prefill-target", action="store_true",
                    help="run the Q5_K [8192, 2048] prefill FC at M = 512 ten times eagerly, for "
                         "rocprofv3 --pmc counter passes over the prefill kernel")
    ap.add_argument("--pmc-moe-target", action="store_true",
                    help="run the benchmark's Q6_K grouped calls (gate/up, down) three times each "
                         "eagerly, for rocprofv3 --pmc counter passes over the grouped kernel")
    ap.add_argument("--pmc-int8-target", action="store_true",
                    help="run the int8 prefill variant (Q5_K [8192, 2048], M = 512) ten times eagerly, "
                         "for rocprofv3 --pmc counter passes")
    ap.add_argument("--pmc-prefill4-target", action="store_true",
                    help="run the four M = 512 prefill FCs eagerly and a 256 MiB device copy of "
                         "known size, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--pmc-skinny-target", action="store_true",
                    help="run the few-row prefill kernel (Q5_K [8192, 2048], M = 8) ten times "
                         "eagerly and a 256 MiB device copy, for rocprofv3 --pmc counter passes")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic record from the two counter passes over --pmc-target")
    ap.add_argument("--moe-traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/moe_grouped_q6k_traffic.json from two --pmc-moe-target counter passes")
    ap.add_argument("--prefill-traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the prefill HBM traffic record from the two counter passes over "
                         "--pmc-prefill4-target")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.prefill_traffic_summary:
        prefill_traffic_summary(*args.prefill_traffic_summary)
        return
    if args.moe_traffic_summary:
        moe_traffic_summary(*args.moe_traffic_summary)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU (across GPUs the FC would shard along N, each GPU "
              "computing its own output columns with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from gguf_quant_block_amd import synth
    from gguf_quant_block_amd.binding import FcGguf

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.pmc_target:
        pmc_target(dev)
        return
    if args.pmc_prefill_target:
        pmc_prefill_target(dev)
        return
    if args.pmc_prefill4_target:
        pmc_prefill4_target(dev)
        return
    if args.pmc_skinny_target:
        pmc_skinny_target(dev)
        return
    if args.pmc_moe_target:
        pmc_moe_target(dev)
        return
    if args.pmc_int8_target:
        pmc_int8_target(dev)
        return

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    def todev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    cases = []
    bb = {"q4_k": 144, "q5_k": 176, "q6_k": 210}

    # ---- decode (cfg1 Q5_K at M = 1, 2, 4, 7; cfg2 Q6_K at M = 1, 4 + output) ----
    def decode_cases(qtype, cfg, shapes, Ms, tag, r_for=lambda name: True, budget=ROTATE_DECODE):
        out = []
        for i, (name, (N, K)) in enumerate(shapes):
            base = todev(synth.blocks(qtype, N, K, synth.rng(cfg, i, synth.TAG_BLOCKS)))
            wb = N * (K // 256) * bb[qtype]
            n_copies = copies_for(wb, budget)
            handles = [FcGguf(N, K, qtype, base) for _ in range(n_copies)]
            del base
            for M in Ms:
                A = todev(synth.normal_f16((M, K), synth.rng(cfg, 100 * M + i, synth.TAG_A)))
                R = todev(synth.normal_f16((M, N), synth.rng(cfg, 100 * M + i, synth.TAG_R))) if r_for(name) else None
                Y = torch.empty((M, N), dtype=torch.float16, device=dev)
                alg = wb + 2 * M * K + 2 * M * N * (2 if R is not None else 1)
                out.append(Case(f"{tag}_{name}_m{M}", [(h, A, R, Y) for h in handles], kind="decode",
                                weight_bytes=wb * n_copies, alg_bytes=alg * n_copies,
                                info={"qtype": qtype, "N": N, "K": K, "M": M, "residual": R is not None}))
        return out

    log("building decode cases")
    cfg1 = decode_cases("q5_k", 1, list(synth.PHI35_LAYERS.items()), (1, 2, 4, 7), "cfg1_q5k")
    cfg2 = decode_cases("q6_k", 2, list(synth.PHI35_LAYERS.items()), (1, 4), "cfg2_q6k")
    cfg2 += decode_cases("q6_k", 2, [("output", synth.PHI35_OUTPUT)], (1, 4), "cfg2_q6k",
                         r_for=lambda name: False)
    cases += cfg1 + cfg2

    # ---- cfg0: one Q6_K FC [512, 2048], M = 1 and 16, no residual ----
    log("building cfg0 and prefill cases")
    N0, K0 = 512, 2048
    base0 = todev(synth.q6k_blocks(N0, K0, synth.rng(0, 0, synth.TAG_BLOCKS)))
    h0 = [FcGguf(N0, K0, "q6_k", base0) for _ in range(64)]
    wb0 = N0 * (K0 // 256) * 210
    for M in (1, 16):
        A = todev(synth.normal_f16((M, K0), synth.rng(0, M, synth.TAG_A)))
        Y = torch.empty((M, N0), dtype=torch.float16, device=dev)
        cases.append(Case(f"cfg0_q6k_m{M}", [(h, A, None, Y) for h in h0],
                          kind="decode" if M < 8 else "prefill", weight_bytes=wb0 * len(h0),
                          alg_bytes=(wb0 + 2 * M * K0 + 2 * M * N0) * len(h0),
                          flops=2 * M * N0 * K0 * len(h0) if M >= 8 else 0,
                          info={"qtype": "q6_k", "N": N0, "K": K0, "M": M, "residual": False,
                                "note": "0.86 MB of weights: 64 copies (55 MB) stay in the last-level cache"}))

    # ---- cfg3: prefill sweep ----
    prefill_first = []        # one handle per (qtype, shape) for the comparison paths
    pre512 = []
    for q in ("q5_k", "q6_k"):
        for si, (N, K) in enumerate(synth.PREFILL_SHAPES):
            base = todev(synth.blocks(q, N, K, synth.rng(3, 10 * si + 4, synth.TAG_BLOCKS)))
            wb = N * (K // 256) * bb[q]
            n_copies = copies_for(wb, ROTATE_PREFILL)
            handles = [FcGguf(N, K, q, base) for _ in range(n_copies)]
            del base
            prefill_first.append(handles[0])
            for M in synth.PREFILL_MS:
                A = todev(synth.normal_f16((M, K), synth.rng(3, 10 * si + M, synth.TAG_A)))
                R = todev(synth.normal_f16((M, N), synth.rng(3, 10 * si + M, synth.TAG_R)))
                Y = torch.empty((M, N), dtype=torch.float16, device=dev)
                c = Case(f"cfg3_{q.replace('_', '')}_{N}x{K}_m{M}", [(h, A, R, Y) for h in handles],
                         kind="prefill", weight_bytes=wb * n_copies,
                         alg_bytes=(wb + 2 * M * K + 4 * M * N) * n_copies,
                         flops=2 * M * N * K * n_copies,
                         info={"qtype": q, "N": N, "K": K, "M": M, "residual": True})
                cases.append(c)
                if M == 512:
                    pre512.append(c)

    # ---- cfg4: MoE ----
    log("building MoE and widened-path cases")
    m = synth.MOE
    E, T, top_k = m["E"], m["T"], m["top_k"]
    moe_calls, moe_touched, moe_alg, moe_flops = [], 0, 0, 0
    for c in range(MOE_COPIES):
        ids_np = synth.moe_routing(T, E, top_k, synth.rng(5, c, synth.TAG_ROUTING), s=m["zipf_s"])
        ids = todev(ids_np)
        nonempty = int((np.bincount(ids_np.ravel(), minlength=E) > 0).sum())
        up = None
        for fi, (which, per_slot) in enumerate((("gate_up", False), ("down", True))):
            N, K = m[which]
            w = todev(synth.q6k_blocks(E * N, K, synth.rng(5, 10 * c + fi, synth.TAG_BLOCKS)))
            fc = FcGguf(N, K, "q6_k", w, experts=E)
            del w
            shape = (T, top_k, K) if per_slot else (T, K)
            A = todev(synth.normal_f16(shape, synth.rng(5, 10 * c + fi, synth.TAG_A)))
            Y = torch.empty((T, top_k, N), dtype=torch.float16, device=dev)
            # down runs on gate/up's bucketing of the same routing
            moe_calls.append((fc, A, ids, per_slot, Y, up))
            up = fc
            eb = N * (K // 256) * 210
            moe_touched += nonempty * eb
            moe_alg += nonempty * eb + A.numel() * 2 + Y.numel() * 2
            moe_flops += 2 * T * top_k * N * K
    moe_case = Case("cfg4_moe_q6k", moe_calls, kind="moe", weight_bytes=moe_touched, alg_bytes=moe_alg,
                    flops=moe_flops, grouped=True,
                    info={"note": "gate/up [768,2048] on token rows + down [2048,768] on pair rows, "
                                  f"{MOE_COPIES} weight copies and routings in rotation; launches = calls "
                                  "(gate/up: bucketing + grouped FC; down: grouped FC on gate/up's "
                                  "bucketing, fc_gguf_run_grouped_reuse)"})
    cases.append(moe_case)

    # ---- widened paths: Q4_K decode (M = 1) and prefill (M = 512); f32 decode ----
    q4 = decode_cases("q4_k", 6, list(synth.PHI35_LAYERS.items()), (1,), "wide_q4k", budget=ROTATE_DECODE // 2)
    cases += q4
    for si, (N, K) in enumerate(synth.PREFILL_SHAPES):
        base = todev(synth.q4k_blocks(N, K, synth.rng(6, 10 + si, synth.TAG_BLOCKS)))
        wb = N * (K // 256) * 144
        handles = [FcGguf(N, K, "q4_k", base) for _ in range(copies_for(wb, ROTATE_PREFILL // 2))]
        del base
        A = todev(synth.normal_f16((512, K), synth.rng(6, 10 + si, synth.TAG_A)))
        R = todev(synth.normal_f16((512, N), synth.rng(6, 10 + si, synth.TAG_R)))
        Y = torch.empty((512, N), dtype=torch.float16, device=dev)
        cases.append(Case(f"wide_q4k_{N}x{K}_m512", [(h, A, R, Y) for h in handles], kind="prefill",
                          weight_bytes=wb * len(handles), flops=2 * 512 * N * K * len(handles),
                          info={"qtype": "q4_k", "N": N, "K": K, "M": 512, "residual": True}))
    f32_calls, f32_bytes = [], 0
    for name, (N, K) in synth.PHI35_LAYERS.items():
        src = next(c for c in cfg1 if c.key == f"cfg1_q5k_{name}_m1")
        hs = [h for h, *_ in src.calls][:8]
        i = list(synth.PHI35_LAYERS).index(name)
        A = todev(synth.normal_f32((1, K), synth.rng(7, i, synth.TAG_A)))
        R = todev(synth.normal_f32((1, N), synth.rng(7, i, synth.TAG_R)))
        Y = torch.empty((1, N), dtype=torch.float32, device=dev)
        f32_calls += [(h, A, R, Y) for h in hs]
        f32_bytes += N * (K // 256) * 176 * len(hs)
    cases.append(Case("wide_f32_q5k_m1", f32_calls, kind="decode", weight_bytes=f32_bytes,
                      info={"note": "Q5_K decode GEMV on f32 A, R and Y over the layer set, 8 copies each"}))

    # ---- eager warm-up, graph capture ----
    log(f"{len(cases)} cases; warm-up and capture")
    for c in cases:
        c.run()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graphs = {}
    for c in cases:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                c.run()
        graphs[c.key] = g
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        for c in cases:
            graphs[c.key].replay()
    torch.cuda.synchronize()

    # ---- timed steps ----
    log("timed steps")
    ev = {c.key: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)] for c in cases}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    with torch.cuda.stream(stream):
        for s in range(args.steps):
            for c in cases:
                e0, e1 = ev[c.key][s]
                e0.record(stream)
                graphs[c.key].replay()
                e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    for c in cases:
        c.times = [e0.elapsed_time(e1) / 1e3 for e0, e1 in ev[c.key]]
    step_s = sum(c.seconds() for c in cases)
    byk = {c.key: c for c in cases}

    # headline: Q5_K decode at M = 1 over the layer set (one launch per shape)
    def layer_rate(prefix, M, which="weight"):
        w = a = t = 0.0
        for name, (N, K) in synth.PHI35_LAYERS.items():
            c = byk[f"{prefix}_{name}_m{M}"]
            t += c.seconds() / c.launches
            w += c.weight_bytes / c.launches
            a += c.alg_bytes / c.launches
        return w / t / 1e9, a / t / 1e9, t / len(synth.PHI35_LAYERS)

    value, achieved, us_launch = layer_rate("cfg1_q5k", 1)
    pre_flops = sum(c.flops for c in pre512)
    pre_s = sum(c.seconds() for c in pre512)
    prefill_tflops = pre_flops / pre_s / 1e12
    pre_us = sum(c.seconds() / c.launches for c in pre512) / len(pre512)
    traffic = traffic_from_profile()

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 dot products (decode); f16 in, f32 accumulate (prefill)",
        "data": "synthetic (seeded blocks; distinct device copies of each weight matrix in rotation)",
        "config": {
            "workload": "Q5_K decode GEMV, Phi-3.5-mini layer set (qkv 9216x3072, o_proj 3072x3072, "
                        "gate_up 16384x3072, down 3072x8192), M=1, fused f16 residual; one launch per shape, "
                        ">= 1 GiB of weight copies per shape in rotation",
            "cases_per_step": len(cases),
            "launches_per_step": sum(c.launches for c in cases),
        },
        "decode_us_per_launch": round(us_launch * 1e6, 3),
        "prefill_tflops_m512": round(prefill_tflops, 1),
        "prefill_us_per_launch_m512": round(pre_us * 1e6, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_kernel (decode, Q5_K, M=1)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "roofline_prefill": {
            "bound": "mfma",
            "kernel": "prefill kernel (M=512, Q5_K and Q6_K, both shapes)",
            "achieved": round(prefill_tflops, 1),
            "peak": F16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(prefill_tflops / F16_MFMA_PEAK_TFLOPS, 4),
            "traffic": prefill_traffic_from_profile(),
        },
        "roofline_moe": {
            "bound": "hbm",
            "kernel": "moe_bucket_kernel + moe_grouped_kernel (Q6_K)",
            "achieved": round(moe_alg / moe_case.seconds() / 1e9, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(moe_alg / moe_case.seconds() / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": moe_traffic_from_profile(),
        },
        "layer_sets": {
            f"{p}_m{M}": {"weight_gbps": round(layer_rate(p, M)[0], 1),
                          "frac_of_hbm_peak": round(layer_rate(p, M)[1] / HBM_PEAK_GBPS, 4),
                          "us_per_launch": round(layer_rate(p, M)[2] * 1e6, 3)}
            for p, Ms in (("cfg1_q5k", (1, 2, 4, 7)), ("cfg2_q6k", (1, 4)), ("wide_q4k", (1,)))
            for M in Ms
        },
        "cases": {c.key: c.summary() for c in cases},
        "wall_s": round(wall, 3),
    }
    log("timed steps done")
    if not args.no_extras:
        sizes = {name: N * (K // 256) * 176 for name, (N, K) in synth.PHI35_LAYERS.items()}
        ceil = ceilings(dev, sizes)
        line["ceilings"] = ceil
        # the decode layer set against the plain read of the same bytes
        t_read = sum(ceil["read"][n]["us"] for n in sizes) / 1e6
        line["ceilings"]["q5k_layer_read_gbps"] = round(sum(sizes.values()) / t_read / 1e9, 1)
        line["ceilings"]["decode_m1_frac_of_read_ceiling"] = round(
            value / (sum(sizes.values()) / t_read / 1e9), 4)
        line["ceilings"]["prefill_m512_frac_of_mfma_ceiling"] = round(
            prefill_tflops / ceil["mfma"]["f16"]["rate"], 4)
        log("ceilings done")
        line["scratch_comparison"] = scratch_comparison(prefill_first, dev)
        line["int8_comparison"] = int8_comparison(prefill_first, dev)
        log("comparisons done")
    if not args.no_cpu_baseline:
        log("CPU oracle")
        cb = cpu_baselines()
        line["cpu_baseline"] = cb["decode"]
        line["cpu_baseline_prefill"] = cb["prefill"]
        line["cpu_baseline_moe"] = cb["moe"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
