// C-ABI of the GGUF K-quant FC library (declarations and contracts in
// include/fc_gguf.h).  Host logic only: argument checks, weight upload and
// Q6_K regroup, path selection from the row count, launch configuration and
// the split-K workspace.  Every step of the computation runs in the HIP
// kernels of this library.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <new>

#include <rocblas/rocblas.h>

#include "fc_gguf.h"
#include "internal.h"

struct fc_gguf {
  int64_t E = 1, N = 0, K = 0;
  int qtype = 0;
  uint8_t* w = nullptr;         // device weights (Q4_K / Q5_K blocks; Q6_K planes; per expert)
  size_t expert_bytes = 0;      // bytes of one [N, K] matrix
  int path = FC_GGUF_PATH_AUTO;
  int decode_rows = 8;                // AUTO: M < decode_rows -> decode path
  int prefill_kernel = 0;             // fcg::PREFILL_KERNEL_*: which prefill kernel
  int tile_mt = 0, tile_splits = 0;   // FC_GGUF_TILE: forced loader-wave tile (0: by M)
  int device = 0;
  int num_cu = 256;
  void* ws = nullptr;           // device workspace (split-K partials, MoE bucketing, the
                                // dequantised f16 weights of the scratch path, the int8
                                // path's quantised activations)
  size_t ws_bytes = 0;
  // the routing whose bucketing the workspace holds (set by a completed
  // fc_gguf_run_grouped launch; read by fc_gguf_run_grouped_reuse)
  const int32_t* routed_ids = nullptr;
  int64_t routed_T = 0;
  int routed_top_k = 0;
  rocblas_handle blas = nullptr;  // created on the first scratch-path call
  hipError_t last = hipSuccess;
};

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr size_t kScratchBytes = 512 * 1024;   // fc_gguf_run_grouped_noalloc's scratch per device
constexpr int kMaxDevices = 64;

int block_bytes(int qtype) {
  switch (qtype) {
    case FC_GGUF_Q4_K: return 144;
    case FC_GGUF_Q5_K: return 176;
    case FC_GGUF_Q6_K: return 210;
    default: return 0;
  }
}

int hip_fail(fc_gguf* h, hipError_t e) {
  if (h) h->last = e;
  return FC_GGUF_EHIP;
}

int default_path() {
  const char* p = getenv("FC_GGUF_PATH");
  if (!p) return FC_GGUF_PATH_AUTO;
  if (!strcmp(p, "decode")) return FC_GGUF_PATH_DECODE;
  if (!strcmp(p, "prefill")) return FC_GGUF_PATH_PREFILL;
  if (!strcmp(p, "scratch")) return FC_GGUF_PATH_SCRATCH;
  if (!strcmp(p, "int8")) return FC_GGUF_PATH_INT8;
  return FC_GGUF_PATH_AUTO;
}

// AUTO's row threshold: FC_GGUF_DECODE_ROWS if it holds an integer in
// [0, 2^20], else the page's 8.
int default_decode_rows() {
  const char* p = getenv("FC_GGUF_DECODE_ROWS");
  if (!p || !*p) return 8;
  char* end = nullptr;
  const long v = strtol(p, &end, 10);
  if (*end != '\0' || v < 0 || v > (1L << 20)) return 8;
  return (int)v;
}

// FC_GGUF_PREFILL_KERNEL=dma|lds|skinny forces one of the prefill kernels
// (testing; skinny only where its rows fit, else the row count decides);
// anything else leaves the choice to the row count.
int default_prefill_kernel() {
  const char* p = getenv("FC_GGUF_PREFILL_KERNEL");
  if (p && !strcmp(p, "dma")) return fcg::PREFILL_KERNEL_DMA;
  if (p && !strcmp(p, "lds")) return fcg::PREFILL_KERNEL_LDS;
  if (p && !strcmp(p, "skinny")) return fcg::PREFILL_KERNEL_SKINNY;
  return fcg::PREFILL_KERNEL_AUTO;
}

// FC_GGUF_TILE=<mt>,<splits> forces the loader-wave prefill tile (tuning):
// 16*mt activation rows (mt = 1, 2, 4 or 8) and K in `splits` parts (a power
// of two from 1 to 64).  Read when a handle is created; anything else, and a
// split count that would leave a part of K empty for the call's K, leaves
// the choice to the row count.
void default_tile(int* mt, int* splits) {
  *mt = *splits = 0;
  const char* p = getenv("FC_GGUF_TILE");
  if (!p || !*p) return;
  char* end = nullptr;
  const long m = strtol(p, &end, 10);
  if (*end != ',') return;
  const long s = strtol(end + 1, &end, 10);
  if (*end != '\0') return;
  if ((m != 1 && m != 2 && m != 4 && m != 8) || s < 1 || s > 64 || (s & (s - 1))) return;
  *mt = (int)m;
  *splits = (int)s;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// FC_GGUF_TEST_FAIL_ALLOC names allocations that fail on purpose, so that
// tests can reach the FC_GGUF_ENOMEM paths: "create" (the weights of a new
// handle), "workspace" (growing a handle's workspace) or "all".  Read at
// every allocation.
bool fail_alloc(const char* what) {
  const char* p = getenv("FC_GGUF_TEST_FAIL_ALLOC");
  if (!p || !*p) return false;
  return !strcmp(p, "all") || !strcmp(p, what);
}

// Grow the handle's workspace to `bytes` on the call's stream.  The old
// buffer is released and the new one taken from the device's stream-ordered
// pool (hipFreeAsync / hipMallocAsync on `st`), so the growth waits only for
// the work already queued on that stream (the last user of the old buffer:
// a handle is never run on two streams at once) and no other stream stalls.
int ensure_ws(fc_gguf* h, size_t bytes, hipStream_t st) {
  if (bytes <= h->ws_bytes) return FC_GGUF_OK;
  if (fail_alloc("workspace")) return FC_GGUF_ENOMEM;
  if (h->ws) {
    const hipError_t e = hipFreeAsync(h->ws, st);
    h->ws = nullptr;
    h->ws_bytes = 0;
    if (e != hipSuccess) return hip_fail(h, e);
  }
  hipError_t e = hipMallocAsync(&h->ws, bytes, st);
  if (e != hipSuccess) {
    h->ws = nullptr;
    h->last = e;
    return FC_GGUF_ENOMEM;
  }
  h->ws_bytes = bytes;
  return FC_GGUF_OK;
}

int create_impl(int64_t E, int64_t N, int64_t K, int qtype, const void* blocks, int on_device,
                int grouped, fc_gguf_t* out) {
  if (!out) return FC_GGUF_EINVAL;
  *out = nullptr;
  if (!blocks || E <= 0 || N <= 0 || K <= 0 || (K % 256) != 0) return FC_GGUF_EINVAL;
  const int bb = block_bytes(qtype);
  if (!bb) return FC_GGUF_EUNSUPPORTED;
  if (N > kMaxDim || K > kMaxDim || E > 65536) return FC_GGUF_ERANGE;
  const size_t nblk = (size_t)N * (size_t)(K / 256);
  if (nblk > ((size_t)1 << 31) / 256) return FC_GGUF_ERANGE;
  const size_t src_bytes = nblk * (size_t)bb;                        // one canonical matrix
  // one device matrix in the tiled layout (grouped handles: one per expert)
  const size_t expert_bytes = fcg::layout_bytes(qtype, (int)N, (int)K);

  fc_gguf* h = new (std::nothrow) fc_gguf();
  if (!h) return FC_GGUF_ENOMEM;
  h->E = E;
  h->N = N;
  h->K = K;
  h->qtype = qtype;
  h->expert_bytes = expert_bytes;
  h->path = default_path();
  h->decode_rows = default_decode_rows();
  h->prefill_kernel = default_prefill_kernel();
  default_tile(&h->tile_mt, &h->tile_splits);
  hipError_t e = hipGetDevice(&h->device);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&h->num_cu, hipDeviceAttributeMultiprocessorCount, h->device);
  if (e != hipSuccess) {
    delete h;
    return FC_GGUF_EHIP;
  }
  const size_t total = expert_bytes * (size_t)E;
  e = fail_alloc("create") ? hipErrorOutOfMemory : hipMalloc(&h->w, total);
  if (e != hipSuccess) {
    delete h;
    return FC_GGUF_ENOMEM;
  }
  // canonical blocks (staged on the device when they come from the host) ->
  // the device layout, one matrix at a time
  const uint8_t* src = (const uint8_t*)blocks;
  uint8_t* staging = nullptr;
  if (!on_device) {
    e = hipMalloc(&staging, src_bytes * (size_t)E);
    if (e == hipSuccess)
      e = hipMemcpy(staging, blocks, src_bytes * (size_t)E, hipMemcpyHostToDevice);
    src = staging;
  }
  for (int64_t x = 0; e == hipSuccess && x < E; ++x)
    e = fcg::launch_weight_layout(qtype, src + x * src_bytes,
                                  h->w + x * expert_bytes, (int)N, (int)K, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (staging) (void)hipFree(staging);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(h->w);
    delete h;
    return FC_GGUF_EHIP;
  }
  *out = h;
  return FC_GGUF_OK;
}

// The dequantise-once comparison path: the weights decoded to f16 in the
// handle's workspace, then one rocBLAS GEMM with the residual as beta * C.
// Row-major Y[M,N] = A[M,K] . W16[N,K]^T is, column-major, Y^T = W16^T^T . A^T:
// op(A) = transpose of the K x N column-major W16, op(B) = the K x M A.
int run_scratch(fc_gguf* h, const fcg::f16* a, const fcg::f16* r, fcg::f16* y, int64_t M,
                hipStream_t st) {
  const int N = (int)h->N, K = (int)h->K;
  int rc = ensure_ws(h, (size_t)N * K * sizeof(fcg::f16), st);
  if (rc != FC_GGUF_OK) return rc;
  if (!h->blas && rocblas_create_handle(&h->blas) != rocblas_status_success) {
    h->blas = nullptr;
    return FC_GGUF_EHIP;
  }
  hipError_t e = fcg::launch_dequant_f16(h->qtype, h->w, (fcg::f16*)h->ws, N, K, st);
  if (e != hipSuccess) return hip_fail(h, e);
  if (rocblas_set_stream(h->blas, st) != rocblas_status_success) return FC_GGUF_EHIP;
  const float alpha = 1.f, beta = r ? 1.f : 0.f;
  const void* c = r ? (const void*)r : (const void*)y;
  const rocblas_status s = rocblas_gemm_ex(
      h->blas, rocblas_operation_transpose, rocblas_operation_none, N, (rocblas_int)M, K, &alpha,
      h->ws, rocblas_datatype_f16_r, K, a, rocblas_datatype_f16_r, K, &beta, c,
      rocblas_datatype_f16_r, N, y, rocblas_datatype_f16_r, N, rocblas_datatype_f32_r,
      rocblas_gemm_algo_standard, 0, 0);
  return s == rocblas_status_success ? FC_GGUF_OK : FC_GGUF_EHIP;
}

// Validation shared by fc_gguf_run and fc_gguf_run_f32 (element size es).
// FC_GGUF_OK when the current device is the handle's (its weights, workspace
// and launches all live there).
int check_device(fc_gguf_t h) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FC_GGUF_EHIP;
  return dev == h->device ? FC_GGUF_OK : FC_GGUF_EDEVICE;
}

int check_run(fc_gguf_t h, const void* A, int64_t M, const void* R, const void* Y, size_t es) {
  if (!h || M < 0) return FC_GGUF_EINVAL;
  if (const int rc = check_device(h); rc != FC_GGUF_OK) return rc;
  if (h->E != 1) return FC_GGUF_EINVAL;            // grouped handles use run_grouped
  if (M == 0) return FC_GGUF_OK;
  if (!A || !Y) return FC_GGUF_EINVAL;
  if (M > kMaxDim || M * h->N > ((int64_t)1 << 31) || M * h->K > ((int64_t)1 << 31))
    return FC_GGUF_ERANGE;
  const size_t ya = es == 2 ? 8 : 4;
  if (!aligned(A, 16) || !aligned(Y, ya) || (R && !aligned(R, ya))) return FC_GGUF_EINVAL;
  return FC_GGUF_OK;
}

// The decode path over M rows: chunks of at most 7 rows (one launch each),
// smaller when the quantised activations of a chunk would not fit in one CU's
// LDS.  At most one or two workgroups per CU: past that, workgroups take
// several row tiles each, streaming the next one's weights under this one's
// arithmetic.
template <class AT>
hipError_t run_decode(fc_gguf_t h, const AT* a, const AT* r, AT* y, int64_t M, hipStream_t st,
                      int* rc) {
  const int N = (int)h->N, K = (int)h->K;
  int cap = 7;
  while (cap > 1 && fcg::gemv_lds_bytes(h->qtype, cap, K) > 160 * 1024) --cap;
  if (fcg::gemv_lds_bytes(h->qtype, cap, K) > 160 * 1024) {
    *rc = FC_GGUF_ERANGE;
    return hipSuccess;
  }
  hipError_t e = hipSuccess;
  for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += cap) {
    const int mc = (int)(M - m0 < cap ? M - m0 : cap);
    // measured: one or two activation rows stream best with two workgroups
    // per CU (two rows: Q5_K layer set 7.29 -> 7.04 us per launch), four and
    // more (more arithmetic per weight byte) with one (two per CU: Q6_K
    // qkv at four rows 9.26 -> 11.07 us, Q5_K at seven rows +26-29 %)
    const int max_wgs = (mc <= 2 ? 2 : 1) * h->num_cu;
    if constexpr (sizeof(AT) == 2)
      e = fcg::launch_gemv(h->qtype, h->w, a + m0 * K, r ? r + m0 * N : nullptr, y + m0 * N, mc, N,
                           K, max_wgs, st);
    else
      e = fcg::launch_gemv_f32(h->qtype, h->w, a + m0 * K, r ? r + m0 * N : nullptr, y + m0 * N, mc,
                               N, K, max_wgs, st);
  }
  *rc = FC_GGUF_OK;
  return e;
}

// Argument checks of the grouped calls (FC_GGUF_OK also for T == 0).
int check_grouped(fc_gguf_t h, const void* A, int64_t T, int a_per_slot, const int32_t* ids,
                  int top_k, const void* Y) {
  if (!h || T < 0) return FC_GGUF_EINVAL;
  if (const int rc = check_device(h); rc != FC_GGUF_OK) return rc;
  if (T == 0) return FC_GGUF_OK;
  if (!A || !ids || !Y || top_k <= 0 || top_k > h->E || (a_per_slot != 0 && a_per_slot != 1))
    return FC_GGUF_EINVAL;
  if (T * top_k > ((int64_t)1 << 24) || T * top_k * h->K > ((int64_t)1 << 31) ||
      T * top_k * h->N > ((int64_t)1 << 31))
    return FC_GGUF_ERANGE;
  if (!aligned(A, 16) || !aligned(Y, 8) || !aligned(ids, 4)) return FC_GGUF_EINVAL;
  return FC_GGUF_OK;
}

// The bucketing (if `bucket`) and grouped-FC launches with the bucketing
// workspace `ws`.
int launch_grouped(fc_gguf_t h, const void* A, int64_t T, int a_per_slot, const int32_t* ids,
                   int top_k, void* Y, void* ws, bool bucket, hipStream_t st) {
  hipError_t e = fcg::launch_moe(h->qtype, h->w, h->expert_bytes, (int)h->E, (int)h->N, (int)h->K,
                                 (const fcg::f16*)A, (int)T, a_per_slot, ids, top_k, (fcg::f16*)Y,
                                 ws, bucket, st);
  if (e == hipErrorNotSupported) return FC_GGUF_EUNSUPPORTED;
  if (e != hipSuccess) return hip_fail(h, e);
  return FC_GGUF_OK;
}

}  // namespace

// Scratch of fc_gguf_run_grouped_noalloc: the bucketing workspace (tile list,
// expert offsets, pair list, tile count) in a static device array, so that
// the call allocates nothing.  Each GPU holds its own copy for the life of
// the process.  In host code `fcg_noalloc_scratch` names a host-side stand-in,
// not the device memory: its device address is taken with
// hipGetSymbolAddress on the device's first call and kept per device.  The
// bucketing kernel writes every word the grouped kernel then reads, so
// nothing needs clearing between calls.
static __device__ __align__(256) uint8_t fcg_noalloc_scratch[kScratchBytes];

namespace {
std::atomic<void*> g_scratch[kMaxDevices];

int scratch_ptr(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return FC_GGUF_ERANGE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // the handle's device is current (checked by the caller)
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(fcg_noalloc_scratch));
    if (e != hipSuccess || !p) return FC_GGUF_EHIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FC_GGUF_OK;
}
}  // namespace

extern "C" {

int fc_gguf_create(int64_t N, int64_t K, int qtype, const void* blocks, int blocks_on_device,
                   fc_gguf_t* out) {
  return create_impl(1, N, K, qtype, blocks, blocks_on_device, 0, out);
}

int fc_gguf_create_grouped(int64_t E, int64_t N, int64_t K, int qtype, const void* blocks,
                           int blocks_on_device, fc_gguf_t* out) {
  if (out) *out = nullptr;
  if (E > fcg::MOE_MAX_E) return FC_GGUF_ERANGE;
  return create_impl(E, N, K, qtype, blocks, blocks_on_device, 1, out);
}

int fc_gguf_destroy(fc_gguf_t h) {
  if (!h) return FC_GGUF_OK;
  // the handle's device, whichever is current: its work must end before the
  // memory is freed
  int cur = -1;
  const bool switched = hipGetDevice(&cur) == hipSuccess && cur != h->device &&
                        hipSetDevice(h->device) == hipSuccess;
  (void)hipDeviceSynchronize();                    // best effort: the handle goes anyway
  if (h->w) (void)hipFree(h->w);
  if (h->ws) {                                     // from the stream-ordered pool
    (void)hipFreeAsync(h->ws, nullptr);
    (void)hipStreamSynchronize(nullptr);
  }
  if (h->blas) rocblas_destroy_handle(h->blas);
  if (switched) (void)hipSetDevice(cur);
  delete h;
  return FC_GGUF_OK;
}

int fc_gguf_set_path(fc_gguf_t h, int path) {
  if (!h) return FC_GGUF_EINVAL;
  if (path < FC_GGUF_PATH_AUTO || path > FC_GGUF_PATH_INT8) return FC_GGUF_EUNSUPPORTED;
  h->path = path;
  return FC_GGUF_OK;
}

int fc_gguf_info(fc_gguf_t h, int64_t* N, int64_t* K, int* qtype, int64_t* weight_bytes) {
  if (!h) return FC_GGUF_EINVAL;
  if (N) *N = h->N;
  if (K) *K = h->K;
  if (qtype) *qtype = h->qtype;
  if (weight_bytes) *weight_bytes = (int64_t)(h->expert_bytes * (size_t)h->E);
  return FC_GGUF_OK;
}

int fc_gguf_run(fc_gguf_t h, const void* A, int64_t M, const void* R, void* Y, void* stream) {
  int rc = check_run(h, A, M, R, Y, 2);
  if (rc != FC_GGUF_OK || M == 0) return rc;
  const int N = (int)h->N, K = (int)h->K;
  hipStream_t st = (hipStream_t)stream;
  int path = h->path;
  if (path == FC_GGUF_PATH_AUTO)
    path = M < h->decode_rows ? FC_GGUF_PATH_DECODE : FC_GGUF_PATH_PREFILL;
  const fcg::f16* a = (const fcg::f16*)A;
  const fcg::f16* r = (const fcg::f16*)R;
  fcg::f16* y = (fcg::f16*)Y;
  hipError_t e = hipSuccess;
  if (path == FC_GGUF_PATH_DECODE) {
    e = run_decode(h, a, r, y, M, st, &rc);
    if (rc != FC_GGUF_OK) return rc;
  } else if (path == FC_GGUF_PATH_SCRATCH) {
    return run_scratch(h, a, r, y, M, st);
  } else if (path == FC_GGUF_PATH_INT8) {
    int mt, nt, splits;
    fcg::prefill_choose(h->qtype, (int)M, N, K, h->num_cu, &mt, &nt, &splits);
    rc = ensure_ws(h, fcg::prefill_i8_workspace_bytes((int)M, N, K, splits), st);
    if (rc != FC_GGUF_OK) return rc;
    e = fcg::launch_prefill_i8(h->qtype, h->w, a, r, y, h->ws, (int)M, N, K, mt, splits, st);
  } else {
    // a forced loader-wave tile (FC_GGUF_TILE) also forces that kernel
    const int kernel = h->tile_mt && h->prefill_kernel == fcg::PREFILL_KERNEL_AUTO
                           ? fcg::PREFILL_KERNEL_DMA
                           : h->prefill_kernel;
    fcg::PrefillPlan plan = fcg::prefill_plan(h->qtype, (int)M, N, K, h->num_cu, kernel);
    if (plan.kind == fcg::PREFILL_KERNEL_DMA && h->tile_mt) {
      // the forced tile, when every part of K keeps at least one stage
      const int S_total = K / fcg::PREFILL_KSTAGE;
      const int per = (S_total + h->tile_splits - 1) / h->tile_splits;
      if ((h->tile_splits - 1) * per < S_total) {
        plan.mt = h->tile_mt;
        plan.splits = h->tile_splits;
      }
    }
    const size_t need = fcg::prefill_workspace_bytes((int)M, N, plan.splits);
    if (need) {
      rc = ensure_ws(h, need, st);
      if (rc != FC_GGUF_OK) return rc;
    }
    e = fcg::launch_prefill(plan, h->qtype, h->w, a, r, y, (float*)h->ws, (int)M, N, K, st);
  }
  if (e != hipSuccess) return hip_fail(h, e);
  return FC_GGUF_OK;
}

int fc_gguf_run_f32(fc_gguf_t h, const float* A, int64_t M, const float* R, float* Y,
                    void* stream) {
  int rc = check_run(h, A, M, R, Y, 4);
  if (rc != FC_GGUF_OK || M == 0) return rc;
  const hipError_t e = run_decode(h, A, R, Y, M, (hipStream_t)stream, &rc);
  if (rc != FC_GGUF_OK) return rc;
  if (e != hipSuccess) return hip_fail(h, e);
  return FC_GGUF_OK;
}

int fc_gguf_run_grouped(fc_gguf_t h, const void* A, int64_t T, int a_per_slot, const int32_t* ids,
                        int top_k, void* Y, void* stream) {
  int rc = check_grouped(h, A, T, a_per_slot, ids, top_k, Y);
  if (rc != FC_GGUF_OK || T == 0) return rc;
  h->routed_ids = nullptr;                          // the workspace is about to change
  const size_t need = fcg::moe_workspace_bytes((int)h->E, (int)T, top_k);
  rc = ensure_ws(h, need, (hipStream_t)stream);
  if (rc != FC_GGUF_OK) return rc;
  rc = launch_grouped(h, A, T, a_per_slot, ids, top_k, Y, h->ws, true, (hipStream_t)stream);
  if (rc == FC_GGUF_OK) {
    h->routed_ids = ids;
    h->routed_T = T;
    h->routed_top_k = top_k;
  }
  return rc;
}

int fc_gguf_run_grouped_reuse(fc_gguf_t h, fc_gguf_t routed, const void* A, int64_t T,
                              int a_per_slot, const int32_t* ids, int top_k, void* Y,
                              void* stream) {
  int rc = check_grouped(h, A, T, a_per_slot, ids, top_k, Y);
  if (rc != FC_GGUF_OK || T == 0) return rc;
  if (!routed || routed->E != h->E || routed->device != h->device || routed->routed_ids != ids ||
      routed->routed_T != T || routed->routed_top_k != top_k)
    return FC_GGUF_EINVAL;
  return launch_grouped(h, A, T, a_per_slot, ids, top_k, Y, routed->ws, false, (hipStream_t)stream);
}

int fc_gguf_run_grouped_noalloc(fc_gguf_t h, const void* A, int64_t T, int a_per_slot,
                                const int32_t* ids, int top_k, void* Y, void* stream) {
  int rc = check_grouped(h, A, T, a_per_slot, ids, top_k, Y);
  if (rc != FC_GGUF_OK || T == 0) return rc;
  if (fcg::moe_workspace_bytes((int)h->E, (int)T, top_k) > kScratchBytes) return FC_GGUF_ERANGE;
  void* ws = nullptr;
  rc = scratch_ptr(h->device, &ws);
  if (rc != FC_GGUF_OK) return rc;
  return launch_grouped(h, A, T, a_per_slot, ids, top_k, Y, ws, true, (hipStream_t)stream);
}

int fc_gguf_debug_quantize(const void* A, int64_t M, int64_t K, int8_t* qa, float* s, int32_t* T,
                           int32_t* H, void* stream) {
  if (M < 0 || K <= 0 || (K % 32) != 0) return FC_GGUF_EINVAL;
  if (M == 0) return FC_GGUF_OK;
  if (!A || !qa || !s || !T || !aligned(A, 16) || !aligned(qa, 16)) return FC_GGUF_EINVAL;
  if (M * K > ((int64_t)1 << 31)) return FC_GGUF_ERANGE;
  hipError_t e = fcg::launch_debug_quantize(A, false, (int)M, (int)K, qa, s, T, H, (hipStream_t)stream);
  return e == hipSuccess ? FC_GGUF_OK : FC_GGUF_EHIP;
}

int fc_gguf_debug_quantize_f32(const float* A, int64_t M, int64_t K, int8_t* qa, float* s,
                               int32_t* T, int32_t* H, void* stream) {
  if (M < 0 || K <= 0 || (K % 32) != 0) return FC_GGUF_EINVAL;
  if (M == 0) return FC_GGUF_OK;
  if (!A || !qa || !s || !T || !aligned(A, 16) || !aligned(qa, 16)) return FC_GGUF_EINVAL;
  if (M * K > ((int64_t)1 << 31)) return FC_GGUF_ERANGE;
  hipError_t e = fcg::launch_debug_quantize(A, true, (int)M, (int)K, qa, s, T, H, (hipStream_t)stream);
  return e == hipSuccess ? FC_GGUF_OK : FC_GGUF_EHIP;
}

int fc_gguf_debug_int_dots(fc_gguf_t h, const int8_t* qa, int64_t M, int32_t* S, void* stream) {
  if (!h || M < 0 || h->E != 1) return FC_GGUF_EINVAL;
  if (const int rc = check_device(h); rc != FC_GGUF_OK) return rc;
  if (M == 0) return FC_GGUF_OK;
  if (!qa || !S || !aligned(qa, 16)) return FC_GGUF_EINVAL;
  const int ns = (int)(h->K / (h->qtype == FC_GGUF_Q6_K ? 16 : 32));
  if (M * h->N * ns > ((int64_t)1 << 31)) return FC_GGUF_ERANGE;
  hipError_t e = fcg::launch_debug_int_dots(h->qtype, h->w, qa, (int)M, (int)h->N, (int)h->K, S,
                                            (hipStream_t)stream);
  return e == hipSuccess ? FC_GGUF_OK : hip_fail(h, e);
}

int fc_gguf_debug_bucketing(const int32_t* ids, int64_t P, int64_t E, int64_t BM, int32_t* offsets,
                            int32_t* pairs, int32_t* tiles, int32_t* ntiles, void* stream) {
  if (P < 0 || E < 1 || BM < 1 || BM > 4096) return FC_GGUF_EINVAL;
  if (E > fcg::MOE_MAX_E || P > ((int64_t)1 << 30)) return FC_GGUF_ERANGE;
  if (P == 0) return FC_GGUF_OK;
  if (!ids || !offsets || !pairs || !tiles || !ntiles || !aligned(tiles, 8)) return FC_GGUF_EINVAL;
  hipError_t e = fcg::launch_debug_bucketing(ids, (int)P, (int)E, (int)BM, offsets, pairs, tiles,
                                             ntiles, (hipStream_t)stream);
  return e == hipSuccess ? FC_GGUF_OK : FC_GGUF_EHIP;
}

int fc_gguf_debug_weights(fc_gguf_t h, void* dst, void* stream) {
  if (!h || !dst) return FC_GGUF_EINVAL;
  if (const int rc = check_device(h); rc != FC_GGUF_OK) return rc;
  hipError_t e = hipMemcpyAsync(dst, h->w, h->expert_bytes * (size_t)h->E, hipMemcpyDeviceToDevice,
                                (hipStream_t)stream);
  return e == hipSuccess ? FC_GGUF_OK : hip_fail(h, e);
}

const char* fc_gguf_strerror(int code) {
  switch (code) {
    case FC_GGUF_OK: return "ok";
    case FC_GGUF_EINVAL: return "invalid argument";
    case FC_GGUF_EUNSUPPORTED: return "unsupported qtype or path";
    case FC_GGUF_ENOMEM: return "device allocation failed";
    case FC_GGUF_EHIP: return "HIP runtime or launch error";
    case FC_GGUF_ERANGE: return "size exceeds an internal limit";
    case FC_GGUF_EDEVICE: return "the current device is not the handle's device";
    default: return "unknown error";
  }
}

}  // extern "C"
