#!/usr/bin/env python3
"""Benchmark of the GGUF K-quant FC library on one MI355X.

Metric: decode GEMV weight GB/s at M = 1 (Q5_K, Phi-3.5-mini layer set), with
the prefill TFLOPS at M = 512 (Q5_K and Q6_K, [8192, 2048] and [2048, 8192])
and the MoE grouped-FC rates reported beside it.

One step = one pass of the hot path over one batch of synthetic input:
  * decode: a 32-layer decode sweep, each layer running its four FCs (fused
    qkv [9216, 3072], o_proj [3072, 3072], fused gate_up [16384, 3072], down
    [3072, 8192]) on M = 1 f16 activations with the f16 residual fused into
    the store; per-32 int8 activation quantisation + int8 GEMV.  Every layer
    has its own copy of the weights in HBM (2.49 GB), so the weights stream
    from HBM rather than from the 256 MB last-level cache.
  * prefill: the four prefill FCs at M = 512 (f16 matrix-core path).
  * moe: the routed Q6_K expert FCs (128 experts, top-8, 256 tokens, Zipf 1.1
    routing): expert bucketing + one grouped launch for gate/up [768, 2048]
    and for down [2048, 768], over 7 weight copies with 7 routings so that
    the touched expert weights stream from HBM.
  * the widened paths, reported beside the headline: Q4_K decode (the same
    layer set, 8 layers of weights) and Q4_K prefill at M = 512, and the f32
    activation path (Q5_K decode GEMV on f32 A, R and Y, 8 layers).
After the timed steps (outside them), the dequantise-once comparison path
(weights decoded to f16, then a rocBLAS GEMM) is timed against the direct
prefill path on the four prefill FCs at M = 512, 1024 and 2048, eagerly with
HIP events on the current stream.
Each phase is captured once as a HIP graph and replayed; HIP events on the
replay stream time the phases.  `value` is the decode phase's weight bytes /
decode time.  Weights and activations are resident in HBM before timing.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --pmc-target            (counter-collection target)
       python bench.py --traffic-summary FETCH_CSV WRITE_CSV
"""

from __future__ import annotations

import argparse
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
LAYERS = 32
MOE_COPIES = 7               # 7 x 165 MB per expert FC: the weights stream from HBM
CPU_LAYERS = 6               # oracle sample: about 10-30 s on one core


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


def cpu_baseline():
    """The CPU oracle (int8-emulating decode reference) on a bounded sample:
    CPU_LAYERS layers of the Q5_K Phi-3.5-mini layer set at M = 1 (the same
    weights each layer, as in the GPU sweep), single-threaded NumPy."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:          # pragma: no cover
        threadpool_limits = None
    import numpy as np  # noqa: F401
    from gguf_quant_block_amd import synth
    from oracle import fc as ofc

    import contextlib
    ctx = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    total_bytes = 0
    with ctx:
        inputs = []
        for i, (name, (N, K)) in enumerate(synth.PHI35_LAYERS.items()):
            inputs.append((synth.q5k_blocks(N, K, synth.rng(1, i, synth.TAG_BLOCKS)),
                           synth.normal_f16((1, K), synth.rng(1, i, synth.TAG_A)),
                           synth.normal_f16((1, N), synth.rng(1, i, synth.TAG_R))))
        t0 = time.perf_counter()
        for _ in range(CPU_LAYERS):
            for w, A, R in inputs:
                ofc.fc_ref_int8(A, w, "q5_k", R)
                total_bytes += w.nbytes
        dt = time.perf_counter() - t0
    return {"value": round(total_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{CPU_LAYERS} layers of the Q5_K Phi-3.5-mini layer set (qkv, o_proj, gate_up, down) at M=1, "
                      f"int8-emulating float64 oracle, {total_bytes / 1e6:.1f} MB of weights in {dt:.1f} s"}


def scratch_comparison(prefill, dev, iters=10):
    """TFLOPS of the direct prefill path and of the dequantise-once path (f16
    weights + rocBLAS GEMM, the residual as beta*C) on the prefill FCs, per M."""
    import torch
    from gguf_quant_block_amd import synth

    out = {"workload": "Q5_K and Q6_K, [8192,2048] and [2048,8192], fused residual; "
                       "dequantise-once = the weights decoded to an f16 buffer on every call "
                       "(not retained), then rocBLAS gemm_ex (f16 in, f32 compute)"}
    for M in (512, 1024, 2048):
        res = {}
        for path in ("prefill", "scratch"):
            flops, calls = 0, []
            for fc, _, _, _ in prefill:
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
            res[path + "_tflops"] = round(flops / s / 1e12, 1)
            for fc, *_ in calls:
                fc.set_path("auto")
        out[f"m{M}"] = {"direct_tflops": res["prefill_tflops"], "dequant_once_tflops": res["scratch_tflops"]}
    return out


def int8_comparison(prefill, dev, iters=10):
    """The int8 matrix-core prefill variant (FC_GGUF_PATH_INT8: per-32 int8
    activations, integer MFMA per group, f32 scale algebra) against the f16
    prefill path on the same prefill FCs at M = 512, eager launches timed with
    HIP events; int8 multiply-adds counted as 2 ops."""
    import torch
    from gguf_quant_block_amd import synth

    M = 512
    out = {"workload": "Q5_K and Q6_K, [8192,2048] and [2048,8192], M=512, fused residual; "
                       "the variant's quantisation pass included",
           "peak_int8_tops": INT8_MFMA_PEAK_TOPS}
    for path in ("prefill", "int8"):
        ops, calls = 0, []
        for fc, _, _, _ in prefill:
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


def pmc_target(dev):
    """Counter-collection target: the decode GEMVs the benchmark times, plus a
    plain device copy of 256 MiB whose FETCH_SIZE / WRITE_SIZE readings give
    the counters' scale factors."""
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
    [8192, 2048] at M = 512 (one workgroup per CU, no split-K), ten eager
    launches."""
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
    torch.cuda.synchronize()
    print("pmc prefill target done", flush=True)


def pmc_moe_target(dev):
    """Counter-collection target for the grouped path: the benchmark's first
    routing and weight copy, gate/up then down, three eager calls each."""
    import torch
    from gguf_quant_block_amd import synth
    from gguf_quant_block_amd.binding import FcGguf
    m = synth.MOE
    E, T, top_k = m["E"], m["T"], m["top_k"]
    ids = torch.from_numpy(synth.moe_routing(T, E, top_k, synth.rng(5, 0, synth.TAG_ROUTING),
                                             s=m["zipf_s"])).to(dev)
    for fi, (which, per_slot) in enumerate((("gate_up", False), ("down", True))):
        N, K = m[which]
        w = torch.from_numpy(synth.q6k_blocks(E * N, K, synth.rng(5, fi, synth.TAG_BLOCKS))).to(dev)
        fc = FcGguf(N, K, "q6_k", w, experts=E)
        shape = (T, top_k, K) if per_slot else (T, K)
        A = torch.from_numpy(synth.normal_f16(shape, synth.rng(5, fi, synth.TAG_A))).to(dev)
        Y = torch.empty((T, top_k, N), dtype=torch.float16, device=dev)
        for _ in range(3):
            fc.grouped(A, ids, per_slot, out=Y)
        torch.cuda.synchronize()
    print("pmc moe target done", flush=True)


CALIB_BYTES = 256 << 20


def traffic_summary(fetch_csv, write_csv):
    """Turn the two counter passes over --pmc-target into HBM bytes per decode
    GEMV launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled
    by what they read for the 256 MiB device copy, then averaged over the GEMV
    dispatches (the same equal mix of the four shapes that the timed sweep runs)."""
    import csv
    from gguf_quant_block_amd import synth

    def read(path, counter):
        gemv, calib = [], []
        with open(path) as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        for r in rows:
            v = float(r["Counter_Value"]) * 1024.0
            if "gemv_kernel" in r["Kernel_Name"]:
                gemv.append((int(r["Grid_Size"]), v))
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
    alg = sum(w_bytes + 2 * K + 4 * N for (N, K), w_bytes in
              (((N, K), N * (K // 256) * 176) for N, K in synth.PHI35_LAYERS.values())) / len(synth.PHI35_LAYERS)
    per_grid = {}
    for (g, fv), (_, wv) in zip(fg, wg):
        per_grid.setdefault(g, []).append(fv * f_factor + wv * w_factor)
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
        "hbm_bytes_per_launch_by_grid": {str(g): round(sum(v) / len(v)) for g, v in sorted(per_grid.items())},
    }
    out = os.path.join(ROOT, "profiles", "decode_gemv_q5k_m1_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-target", action="store_true",
                    help="run the decode sweep eagerly (4 shapes x 4 weight copies x 3 passes) and a "
                         "256 MiB device copy of known size, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--pmc-prefill-target", action="store_true",
                    help="run the Q5_K [8192, 2048] prefill FC at M = 512 ten times eagerly, for "
                         "rocprofv3 --pmc counter passes over the prefill kernel")
    ap.add_argument("--pmc-moe-target", action="store_true",
                    help="run the benchmark's Q6_K grouped calls (gate/up, down) three times each "
                         "eagerly, for rocprofv3 --pmc counter passes over the grouped kernel")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic record from the two counter passes over --pmc-target")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
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
    if args.pmc_moe_target:
        pmc_moe_target(dev)
        return

    # ---- decode workload: 32 layers x 4 FCs, Q5_K, M = 1, residual fused ----
    shapes = list(synth.PHI35_LAYERS.items())
    layer_sets = []
    decode_weight_bytes = 0
    decode_alg_bytes = 0
    base = {}
    for i, (name, (N, K)) in enumerate(shapes):
        base[name] = torch.from_numpy(synth.q5k_blocks(N, K, synth.rng(1, i, synth.TAG_BLOCKS))).to(dev)
    acts = {}
    for i, (name, (N, K)) in enumerate(shapes):
        A = torch.from_numpy(synth.normal_f16((1, K), synth.rng(1, i, synth.TAG_A))).to(dev)
        R = torch.from_numpy(synth.normal_f16((1, N), synth.rng(1, i, synth.TAG_R))).to(dev)
        Y = torch.empty((1, N), dtype=torch.float16, device=dev)
        acts[name] = (A, R, Y)
    for layer in range(LAYERS):
        fcs = {}
        for name, (N, K) in shapes:
            fcs[name] = FcGguf(N, K, "q5_k", base[name])
            w_bytes = N * (K // 256) * 176                                    # the Q5_K blocks
            decode_weight_bytes += w_bytes
            decode_alg_bytes += w_bytes + 2 * K + 2 * 2 * N                   # weights + A + R + Y
        layer_sets.append(fcs)
    decode_launches = LAYERS * len(shapes)

    def decode_pass():
        for fcs in layer_sets:
            for name, _ in shapes:
                A, R, Y = acts[name]
                fcs[name](A, R, out=Y)

    # ---- prefill workload: M = 512, Q5_K and Q6_K, both weight shapes ----
    Mp = 512
    prefill = []
    prefill_flops = 0
    for qi, q in enumerate(("q5_k", "q6_k")):
        for si, (N, K) in enumerate(synth.PREFILL_SHAPES):
            w = torch.from_numpy(synth.blocks(q, N, K, synth.rng(3, 10 * si + 4, synth.TAG_BLOCKS))).to(dev)
            fc = FcGguf(N, K, q, w)
            A = torch.from_numpy(synth.normal_f16((Mp, K), synth.rng(3, 10 * si + 4, synth.TAG_A))).to(dev)
            R = torch.from_numpy(synth.normal_f16((Mp, N), synth.rng(3, 10 * si + 4, synth.TAG_R))).to(dev)
            Y = torch.empty((Mp, N), dtype=torch.float16, device=dev)
            prefill.append((fc, A, R, Y))
            prefill_flops += 2 * Mp * N * K

    def prefill_pass():
        for fc, A, R, Y in prefill:
            fc(A, R, out=Y)

    # ---- MoE workload: Q6_K experts, 128 experts, top-8, 256 tokens, Zipf 1.1 ----
    m = synth.MOE
    E, T, top_k = m["E"], m["T"], m["top_k"]
    moe = []
    moe_touched = moe_alg = moe_flops = 0
    for c in range(MOE_COPIES):
        ids_np = synth.moe_routing(T, E, top_k, synth.rng(5, c, synth.TAG_ROUTING), s=m["zipf_s"])
        ids = torch.from_numpy(ids_np).to(dev)
        nonempty = int((np.bincount(ids_np.ravel(), minlength=E) > 0).sum())
        for fi, (which, per_slot) in enumerate((("gate_up", False), ("down", True))):
            N, K = m[which]
            w = torch.from_numpy(synth.q6k_blocks(E * N, K, synth.rng(5, 10 * c + fi, synth.TAG_BLOCKS))).to(dev)
            fc = FcGguf(N, K, "q6_k", w, experts=E)
            del w
            shape = (T, top_k, K) if per_slot else (T, K)
            A = torch.from_numpy(synth.normal_f16(shape, synth.rng(5, 10 * c + fi, synth.TAG_A))).to(dev)
            Y = torch.empty((T, top_k, N), dtype=torch.float16, device=dev)
            moe.append((fc, A, ids, per_slot, Y))
            expert_bytes = N * (K // 256) * 210
            moe_touched += nonempty * expert_bytes
            moe_alg += nonempty * expert_bytes + A.numel() * 2 + Y.numel() * 2
            moe_flops += 2 * T * top_k * N * K

    def moe_pass():
        for fc, A, ids, per_slot, Y in moe:
            fc.grouped(A, ids, per_slot, out=Y)

    # ---- widened paths: Q4_K decode and prefill; f32 activations ----
    WIDE_LAYERS = 8
    q4_dec, q4_dec_bytes = [], 0
    q4_base = {}
    for i, (name, (N, K)) in enumerate(shapes):
        q4_base[name] = torch.from_numpy(synth.q4k_blocks(N, K, synth.rng(6, i, synth.TAG_BLOCKS))).to(dev)
    for layer in range(WIDE_LAYERS):
        for name, (N, K) in shapes:
            A, R, Y = acts[name]
            q4_dec.append((FcGguf(N, K, "q4_k", q4_base[name]), A, R, Y))
            q4_dec_bytes += N * (K // 256) * 144
    q4_pre, q4_pre_flops = [], 0
    for si, (N, K) in enumerate(synth.PREFILL_SHAPES):
        w = torch.from_numpy(synth.q4k_blocks(N, K, synth.rng(6, 10 + si, synth.TAG_BLOCKS))).to(dev)
        A = torch.from_numpy(synth.normal_f16((Mp, K), synth.rng(6, 10 + si, synth.TAG_A))).to(dev)
        R = torch.from_numpy(synth.normal_f16((Mp, N), synth.rng(6, 10 + si, synth.TAG_R))).to(dev)
        q4_pre.append((FcGguf(N, K, "q4_k", w), A, R, torch.empty((Mp, N), dtype=torch.float16, device=dev)))
        q4_pre_flops += 2 * Mp * N * K
    f32_dec, f32_bytes = [], 0
    acts32 = {}
    for i, (name, (N, K)) in enumerate(shapes):
        acts32[name] = (torch.from_numpy(synth.normal_f32((1, K), synth.rng(7, i, synth.TAG_A))).to(dev),
                        torch.from_numpy(synth.normal_f32((1, N), synth.rng(7, i, synth.TAG_R))).to(dev),
                        torch.empty((1, N), dtype=torch.float32, device=dev))
    for fcs in layer_sets[:WIDE_LAYERS]:
        for name, (N, K) in shapes:
            f32_dec.append((fcs[name], *acts32[name]))
            f32_bytes += N * (K // 256) * 176

    def run_list(lst):
        def f():
            for fc, A, R, Y in lst:
                fc(A, R, out=Y)
        return f

    # eager warm-up (sets kernel attributes, allocates split-K workspaces)
    phases = (("decode", decode_pass), ("prefill", prefill_pass), ("moe", moe_pass),
              ("q4k_decode", run_list(q4_dec)), ("q4k_prefill", run_list(q4_pre)),
              ("f32_decode", run_list(f32_dec)))
    for _, fn in phases:
        fn()
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    graphs = {}
    for key, fn in phases:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                fn()
        graphs[key] = g
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for key, _ in phases:
            graphs[key].replay()
    torch.cuda.synchronize()

    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for k, _ in phases}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    with torch.cuda.stream(stream):
        for s in range(args.steps):
            for k, _ in phases:
                e0, e1 = ev[k][s]
                e0.record(stream)
                graphs[k].replay()
                e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    def phase_s(k):
        return sum(e0.elapsed_time(e1) for e0, e1 in ev[k]) / 1e3 / args.steps

    dec_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev["decode"])
    pre_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev["prefill"])
    moe_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev["moe"])
    step_ms = sum(phase_s(k) for k, _ in phases) * 1e3
    q4d_s, q4p_s, f32_s = phase_s("q4k_decode"), phase_s("q4k_prefill"), phase_s("f32_decode")
    moe_s = moe_ms / 1e3 / args.steps
    dec_s = dec_ms / 1e3 / args.steps
    pre_s = pre_ms / 1e3 / args.steps
    value = decode_weight_bytes / dec_s / 1e9
    achieved = decode_alg_bytes / dec_s / 1e9
    prefill_tflops = prefill_flops / pre_s / 1e12
    traffic = traffic_from_profile()

    line = {
        "metric": "decode GEMV weight GB/s (M=1); prefill TFLOPS at M=512; Q5_K/Q6_K",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 dot products (decode); f16 in, f32 accumulate (prefill)",
        "data": "synthetic (seeded blocks; 32 device copies of one Q5_K layer set)",
        "config": {
            "workload": "Q5_K decode GEMV, Phi-3.5-mini layer set (qkv 9216x3072, o_proj 3072x3072, "
                        "gate_up 16384x3072, down 3072x8192), M=1, fused f16 residual, 32-layer sweep",
            "decode_weight_bytes_per_step": decode_weight_bytes,
            "decode_launches_per_step": decode_launches,
            "prefill": "Q5_K and Q6_K, [8192,2048] and [2048,8192], M=512, fused residual",
        },
        "decode_us_per_launch": round(dec_s * 1e6 / decode_launches, 3),
        "prefill_tflops_m512": round(prefill_tflops, 1),
        "prefill_us_per_launch": round(pre_s * 1e6 / len(prefill), 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_kernel (decode, Q5_K, M=1)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "moe": {
            "workload": "Q6_K experts, 128 experts, top-8, 256 tokens, Zipf(1.1) routing: gate/up [768,2048] "
                        f"on token rows + down [2048,768] on pair rows, {MOE_COPIES} weight copies and routings "
                        "in rotation",
            "touched_weight_gbps": round(moe_touched / moe_s / 1e9, 1),
            "tflops": round(moe_flops / moe_s / 1e12, 2),
            "us_per_call": round(moe_s * 1e6 / len(moe), 2),
        },
        "roofline_moe": {
            "bound": "hbm",
            "kernel": "moe_bucket_kernel + moe_grouped_kernel (Q6_K)",
            "achieved": round(moe_alg / moe_s / 1e9, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(moe_alg / moe_s / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": None,
        },
        "roofline_prefill": {
            "bound": "mfma",
            "kernel": "prefill_dma_kernel (M=512)",
            "achieved": round(prefill_tflops, 1),
            "peak": F16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(prefill_tflops / F16_MFMA_PEAK_TFLOPS, 4),
            "traffic": None,
        },
        "q4k": {
            "workload": f"Q4_K decode GEMV over the same layer set ({WIDE_LAYERS} layers of weights, M=1, fused "
                        "residual) and Q4_K prefill at M=512 on [8192,2048] and [2048,8192]",
            "decode_weight_gbps": round(q4_dec_bytes / q4d_s / 1e9, 1),
            "decode_us_per_launch": round(q4d_s * 1e6 / len(q4_dec), 3),
            "decode_frac_of_hbm_peak": round(q4_dec_bytes / q4d_s / 1e9 / HBM_PEAK_GBPS, 4),
            "prefill_tflops_m512": round(q4_pre_flops / q4p_s / 1e12, 1),
            "prefill_frac_of_f16_peak": round(q4_pre_flops / q4p_s / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
        },
        "f32_decode": {
            "workload": f"Q5_K decode GEMV on f32 activations, residual and output, M=1, {WIDE_LAYERS} layers",
            "weight_gbps": round(f32_bytes / f32_s / 1e9, 1),
            "us_per_launch": round(f32_s * 1e6 / len(f32_dec), 3),
        },
        "wall_s": round(wall, 3),
    }
    line["scratch_comparison"] = scratch_comparison(prefill, dev)
    line["int8_comparison"] = int8_comparison(prefill, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
