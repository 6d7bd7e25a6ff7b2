"""ctypes binding of libfcgguf.so (the C-ABI declared in include/fc_gguf.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is not built, or no GPU is visible,
calls raise.
"""

from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
# FC_GGUF_LIB names another build of the library (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("FC_GGUF_LIB") or os.path.join(PKG, "libfcgguf.so")

Q4_K, Q5_K, Q6_K = 4, 5, 6
QTYPES = {"q4_k": Q4_K, "q5_k": Q5_K, "q6_k": Q6_K}
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q6_K: 210}
PATHS = {"auto": 0, "decode": 1, "prefill": 2, "scratch": 3, "int8": 4}

_lib = None
_lock = threading.Lock()

_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_SIGS = {
    "fc_gguf_create": (ctypes.c_int, [_c_i64, _c_i64, ctypes.c_int, _vp, ctypes.c_int, ctypes.POINTER(_vp)]),
    "fc_gguf_create_grouped": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, ctypes.c_int, _vp, ctypes.c_int,
                                              ctypes.POINTER(_vp)]),
    "fc_gguf_run": (ctypes.c_int, [_vp, _vp, _c_i64, _vp, _vp, _vp]),
    "fc_gguf_run_f32": (ctypes.c_int, [_vp, _vp, _c_i64, _vp, _vp, _vp]),
    "fc_gguf_run_grouped": (ctypes.c_int, [_vp, _vp, _c_i64, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp]),
    "fc_gguf_run_grouped_noalloc": (ctypes.c_int, [_vp, _vp, _c_i64, ctypes.c_int, _vp, ctypes.c_int, _vp,
                                                   _vp]),
    "fc_gguf_run_grouped_reuse": (ctypes.c_int, [_vp, _vp, _vp, _c_i64, ctypes.c_int, _vp, ctypes.c_int,
                                                 _vp, _vp]),
    "fc_gguf_set_path": (ctypes.c_int, [_vp, ctypes.c_int]),
    "fc_gguf_destroy": (ctypes.c_int, [_vp]),
    "fc_gguf_info": (ctypes.c_int, [_vp, ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i64),
                                    ctypes.POINTER(ctypes.c_int), ctypes.POINTER(_c_i64)]),
    "fc_gguf_debug_quantize": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp]),
    "fc_gguf_debug_quantize_f32": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp]),
    "fc_gguf_debug_bucketing": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp]),
    "fc_gguf_debug_int_dots": (ctypes.c_int, [_vp, _vp, _c_i64, _vp, _vp]),
    "fc_gguf_debug_weights": (ctypes.c_int, [_vp, _vp, _vp]),
    "fc_gguf_strerror": (ctypes.c_char_p, [ctypes.c_int]),
}


class FcGgufError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run `python -m gguf_quant_block_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().fc_gguf_strerror(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise FcGgufError(code, what)


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible: the FC library has no CPU path")
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _blocks_arg(blocks):
    """(pointer, on_device, keepalive) for a numpy or torch uint8 array."""
    import numpy as np
    if isinstance(blocks, np.ndarray):
        arr = np.ascontiguousarray(blocks, dtype=np.uint8)
        return ctypes.c_void_p(arr.ctypes.data), 0, arr
    torch = _torch()
    assert blocks.dtype == torch.uint8
    t = blocks.contiguous()
    return ctypes.c_void_p(t.data_ptr()), (1 if t.is_cuda else 0), t


class FcGguf:
    """One weight matrix W[N, K] in GGUF Q4_K, Q5_K or Q6_K blocks, resident on the GPU.

    y = fc(A, R=None, out=None): A [..., K] on cuda, f16 or f32 (any number
    of leading dims, flattened to M rows; M may change from call to call);
    R [..., N] of A's dtype or None; the output has A's dtype.  f32
    activations always take the int8 GEMV path.
    """

    def __init__(self, N: int, K: int, qtype: str, blocks, *, experts: int | None = None):
        self.N, self.K, self.qtype = int(N), int(K), qtype
        self.experts = experts
        ptr, on_dev, keep = _blocks_arg(blocks)
        h = ctypes.c_void_p()
        if experts is None:
            _check(lib().fc_gguf_create(self.N, self.K, QTYPES[qtype], ptr, on_dev, ctypes.byref(h)),
                   "fc_gguf_create")
        else:
            _check(lib().fc_gguf_create_grouped(int(experts), self.N, self.K, QTYPES[qtype], ptr, on_dev,
                                                ctypes.byref(h)), "fc_gguf_create_grouped")
        del keep
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().fc_gguf_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_path(self, path: str):
        _check(lib().fc_gguf_set_path(self._h, PATHS[path]), "fc_gguf_set_path")

    @property
    def weight_bytes(self) -> int:
        wb = ctypes.c_int64()
        _check(lib().fc_gguf_info(self._h, None, None, None, ctypes.byref(wb)), "fc_gguf_info")
        return wb.value

    def __call__(self, A, R=None, out=None):
        torch = _torch()
        dt = A.dtype
        assert dt in (torch.float16, torch.float32) and A.is_cuda and A.shape[-1] == self.K
        lead = A.shape[:-1]
        A2 = A.reshape(-1, self.K).contiguous()
        M = A2.shape[0]
        if R is not None:
            assert R.dtype == dt and R.shape == (*lead, self.N)
            R = R.reshape(M, self.N).contiguous()
        if out is None:
            out = torch.empty((*lead, self.N), dtype=dt, device=A.device)
        assert out.is_contiguous() and out.dtype == dt and out.shape == (*lead, self.N)
        run = lib().fc_gguf_run if dt == torch.float16 else lib().fc_gguf_run_f32
        _check(run(self._h, _ptr(A2), M, _ptr(R), _ptr(out), _stream()), "fc_gguf_run")
        return out

    def grouped(self, A, ids, a_per_slot: bool, out=None, noalloc: bool = False, routed=None):
        """MoE: Y[t, j] = A_row(t, j) . W_{ids[t, j]}^T; A f16 [T, K] or [T, top_k, K].
        noalloc: fc_gguf_run_grouped_noalloc (the library's static scratch, no allocation).
        routed: a grouped FcGguf whose last grouped() call had this same ids tensor:
        fc_gguf_run_grouped_reuse (its expert bucketing, not sorted again)."""
        torch = _torch()
        assert self.experts is not None, "grouped() needs a handle made with experts=E"
        T, top_k = ids.shape
        assert ids.is_cuda and A.is_cuda and A.dtype == torch.float16
        assert A.shape == ((T, top_k, self.K) if a_per_slot else (T, self.K))
        if routed is not None:
            # the same ids memory as the routed call's: no conversion copy
            assert ids.dtype == torch.int32 and ids.is_contiguous(), "ids: contiguous int32"
        ids = ids.to(torch.int32).contiguous()
        A = A.contiguous()
        if out is None:
            out = torch.empty((T, top_k, self.N), dtype=torch.float16, device=A.device)
        assert out.is_contiguous() and out.dtype == torch.float16 and out.shape == (T, top_k, self.N)
        if routed is not None:
            assert not noalloc
            _check(lib().fc_gguf_run_grouped_reuse(self._h, routed.handle, _ptr(A), T, 1 if a_per_slot else 0,
                                                   _ptr(ids), top_k, _ptr(out), _stream()),
                   "fc_gguf_run_grouped_reuse")
            return out
        run = lib().fc_gguf_run_grouped_noalloc if noalloc else lib().fc_gguf_run_grouped
        _check(run(self._h, _ptr(A), T, 1 if a_per_slot else 0, _ptr(ids), top_k, _ptr(out), _stream()),
               "fc_gguf_run_grouped_noalloc" if noalloc else "fc_gguf_run_grouped")
        return out

    # ---- test exports ----
    def debug_int_dots(self, qa):
        torch = _torch()
        M = qa.shape[0]
        ns = self.K // (16 if self.qtype == "q6_k" else 32)
        S = torch.empty((M, self.N, ns), dtype=torch.int32, device=qa.device)
        _check(lib().fc_gguf_debug_int_dots(self._h, _ptr(qa.contiguous()), M, _ptr(S), _stream()),
               "fc_gguf_debug_int_dots")
        return S

    def debug_weights(self):
        torch = _torch()
        out = torch.empty(self.weight_bytes, dtype=torch.uint8, device="cuda")
        _check(lib().fc_gguf_debug_weights(self._h, _ptr(out), _stream()), "fc_gguf_debug_weights")
        return out


def debug_quantize(A):
    """The decode path's per-32 int8 quantisation of f16 or f32 A[M, K]:
    (qa i8[M,K], s f32[M,K/32], T i32[M,K/32], H i32[M,K/16]); H holds the
    code sums of the groups' 16-value halves."""
    torch = _torch()
    M, K = A.shape
    assert A.dtype in (torch.float16, torch.float32)
    qa = torch.empty((M, K), dtype=torch.int8, device=A.device)
    s = torch.empty((M, K // 32), dtype=torch.float32, device=A.device)
    T = torch.empty((M, K // 32), dtype=torch.int32, device=A.device)
    H = torch.empty((M, K // 16), dtype=torch.int32, device=A.device)
    f = lib().fc_gguf_debug_quantize if A.dtype == torch.float16 else lib().fc_gguf_debug_quantize_f32
    _check(f(_ptr(A.contiguous()), M, K, _ptr(qa), _ptr(s), _ptr(T), _ptr(H), _stream()),
           "fc_gguf_debug_quantize")
    return qa, s, T, H


def debug_bucketing(ids, E: int, BM: int):
    """The grouped path's expert bucketing of device i32 routing ids (any
    shape, pairs in row-major order): (offsets i32[E+2], pairs i32[P] grouped
    by bucket, in no fixed order within a bucket, tiles i32[n, 2])."""
    torch = _torch()
    ids = ids.contiguous().reshape(-1)
    assert ids.dtype == torch.int32
    P = ids.numel()
    cap = -(-P // BM) + min(E + 1, P)
    offsets = torch.empty(E + 2, dtype=torch.int32, device=ids.device)
    pairs = torch.empty(max(P, 1), dtype=torch.int32, device=ids.device)
    tiles = torch.empty((max(cap, 1), 2), dtype=torch.int32, device=ids.device)
    n = torch.zeros(1, dtype=torch.int32, device=ids.device)
    _check(lib().fc_gguf_debug_bucketing(_ptr(ids), P, E, BM, _ptr(offsets), _ptr(pairs), _ptr(tiles),
                                         _ptr(n), _stream()), "fc_gguf_debug_bucketing")
    return offsets, pairs[:P], tiles[:int(n.item())]
