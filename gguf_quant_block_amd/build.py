"""Build the HIP libraries in-tree for gfx950 (hipcc).

Usage: python -m gguf_quant_block_amd.build [--jobs N]
Each translation unit under csrc/ is compiled to an object in _build/; the FC
library's objects are linked into gguf_quant_block_amd/libfcgguf.so, and the
benchmark's ceiling kernels (csrc/ceilings.hip) into libfcgceil.so.  Always
rebuilds.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfcgguf.so")
CEIL_LIB = os.path.join(PKG, "libfcgceil.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed-FP32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]
SOURCES = ["fc_gguf_api.cpp", "layout.hip", "gemv.hip", "prefill.hip", "skinny.hip", "prefill_i8.hip",
           "moe.hip", "dequant.hip"]
CEIL_SOURCES = ["ceilings.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def _link(objs, out, libs):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, *libs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"link of {os.path.basename(out)} failed")
    os.replace(tmp, out)


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, 8))) as ex:
        objs = list(ex.map(_compile, SOURCES + CEIL_SOURCES))
    n = len(SOURCES)
    # rocBLAS serves only the dequantise-once comparison path
    _link(objs[:n], LIB, ["-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"])
    _link(objs[n:], CEIL_LIB, [])
    if verbose:
        print(f"built {LIB} and {CEIL_LIB}")
    return LIB


# Host-side sanitizer build of the C-ABI layer (argument validation, handle
# and workspace management): fc_gguf_api.cpp's host code with AddressSanitizer
# and UndefinedBehaviorSanitizer, linked with the regular kernel objects.  The
# GPU code is built as usual (each sanitizer flag applies to the host pass
# only).  Loaded by a process that preloads ASAN_RUNTIME.
SAN_LIB = os.path.join(BUILD, "san", "libfcgguf_san.so")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime() -> str:
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "amdclang++")
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    return r.stdout.strip()


def build_sanitized() -> str:
    """The host-sanitized library (after build(), whose kernel objects it reuses)."""
    san = os.path.dirname(SAN_LIB)
    os.makedirs(san, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "fc_gguf_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build()
    api = os.path.join(san, "fc_gguf_api.o")
    cmd = [HIPCC, "-x", "hip", *CFLAGS, "-g", *SAN_HOST, "-c", os.path.join(CSRC, "fc_gguf_api.cpp"),
           "-o", api]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on the sanitized fc_gguf_api.cpp")
    _link([api, *objs], SAN_LIB, [*SAN_HOST, "-shared-libsan", "-L/opt/rocm/lib", "-lrocblas",
                                  "-Wl,-rpath,/opt/rocm/lib"])
    return SAN_LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    a = ap.parse_args()
    build(a.jobs, verbose=True)
