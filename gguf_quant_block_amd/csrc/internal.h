// Launchers shared between the kernel translation units and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>
#include <stdint.h>

namespace fcg {
typedef _Float16 f16;

// Raises kern's dynamic-LDS limit to `bytes` on the current device, once per
// device: the limit is an attribute of the function on each device.  `done`
// (one per kernel instantiation) holds a bit per device id; ids past 63 are
// set on every call.
inline hipError_t raise_lds_limit(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// canonical AoS blocks of an [N, K] matrix -> the tiled device layout of
// layout.h (the destination holds layout_bytes(...) bytes)
size_t layout_bytes(int qtype, int N, int K);
hipError_t launch_weight_layout(int qtype, const uint8_t* src, uint8_t* dst, int N, int K,
                                hipStream_t st);

// decode path (M in 1..7); A, R, Y all f16, or all f32
size_t gemv_lds_bytes(int qtype, int M, int K);
// max_wgs: the most workgroups the launch uses (one per row tile up to it;
// each then takes every max_wgs-th row tile)
hipError_t launch_gemv(int qtype, const uint8_t* W, const f16* A, const f16* R, f16* Y, int M,
                       int N, int K, int max_wgs, hipStream_t st);
hipError_t launch_gemv_f32(int qtype, const uint8_t* W, const float* A, const float* R, float* Y,
                           int M, int N, int K, int max_wgs, hipStream_t st);
// A is f32 if f32, else f16; H (16-value half sums) may be null
hipError_t launch_debug_quantize(const void* A, bool f32, int M, int K, int8_t* qa, float* s, int* T,
                                 int* H, hipStream_t st);
hipError_t launch_debug_int_dots(int qtype, const uint8_t* W, const int8_t* qa, int M, int N, int K,
                                 int* S, hipStream_t st);

// dequantise-once comparison path: tiled weights -> row-major f16 W16[N, K]
hipError_t launch_dequant_f16(int qtype, const uint8_t* W, f16* out, int N, int K, hipStream_t st);

// prefill path: three kernels, the loader-wave tile (16 .. 128 activation
// rows, weights decoded in the compute waves' registers), the decode-once
// tile (128 x 128, weights decoded once into an f16 LDS tile by producer
// waves) and the few-row kernel (skinny.hip: the GEMV's work layout on the
// matrix cores, no K split); prefill_plan takes the few-row kernel where
// M <= 32 rows fit its LDS, else the loader-wave tile, and
// FC_GGUF_PREFILL_KERNEL=dma|lds|skinny forces one
constexpr int PREFILL_KSTAGE = 128;   // values of K per loader-wave stage (half a super-block)
constexpr int PREFILL_KERNEL_AUTO = 0;
constexpr int PREFILL_KERNEL_DMA = 1;
constexpr int PREFILL_KERNEL_LDS = 2;
constexpr int PREFILL_KERNEL_SKINNY = 3;
struct PrefillPlan {
  int kind;       // PREFILL_KERNEL_DMA, _LDS or _SKINNY
  int mt;         // activation rows per tile / 16
  int splits;     // K splits (f32 partials + reduction when > 1)
  int sb_per;     // super-blocks per split (decode-once tile)
  int wgs;        // most workgroups of the launch (skinny kernel)
};
void prefill_choose(int qtype, int M, int N, int K, int num_cu, int* mt, int* nt, int* splits);
PrefillPlan prefill_plan(int qtype, int M, int N, int K, int num_cu, int kernel);
size_t prefill_workspace_bytes(int M, int N, int splits);
hipError_t launch_prefill(const PrefillPlan& p, int qtype, const uint8_t* W, const f16* A,
                          const f16* R, f16* Y, float* P, int M, int N, int K, hipStream_t st);
// the few-row prefill kernel (skinny.hip): M <= 32 rows whose f16 copy fits
// the LDS next to the partial sums; max_wgs as for the GEMV
bool skinny_fits(int M, int K);
int skinny_max_wgs(int M, int K, int num_cu);
hipError_t launch_skinny(int qtype, const uint8_t* W, const f16* A, const f16* R, f16* Y, int M,
                         int N, int K, int max_wgs, hipStream_t st);
// Y = sum over splits of P[split][M*N] + R, one f16 rounding
hipError_t launch_splitk_reduce(const float* P, const f16* R, f16* Y, long long MN, int splits,
                                hipStream_t st);

// int8 matrix-core prefill variant (tile and splits from prefill_choose); ws
// holds prefill_i8_workspace_bytes(M, N, K, splits) bytes
size_t prefill_i8_workspace_bytes(int M, int N, int K, int splits);
hipError_t launch_prefill_i8(int qtype, const uint8_t* W, const f16* A, const f16* R, f16* Y,
                             void* ws, int M, int N, int K, int mt, int splits, hipStream_t st);

// grouped (MoE) path
constexpr int MOE_MAX_E = 4096;   // experts per grouped handle (bucketing counts live in LDS)
size_t moe_workspace_bytes(int E, int T, int top_k);
// bucket: run the bucketing into ws first; false: ws already holds the
// bucketing of the same routing (E, T, top_k, ids)
hipError_t launch_moe(int qtype, const uint8_t* W, size_t expert_bytes, int E, int N, int K,
                      const f16* A, int T, int a_per_slot, const int32_t* ids, int top_k, f16* Y,
                      void* ws, bool bucket, hipStream_t st);
// the grouped path's bucketing alone, into caller buffers (test export)
hipError_t launch_debug_bucketing(const int32_t* ids, int P, int E, int BM, int* offsets, int* pairs,
                                  int* tiles, int* ntiles, hipStream_t st);
}  // namespace fcg
