// Measured ceilings of this chip for the FC kernels: a plain coalesced read
// of a buffer (the most any kernel that reads the weight bytes once per
// launch can reach), and back-to-back matrix-core instructions (the f16 and
// int8 MFMA rate under sustained load, with the clock the chip holds then).
// Not part of the FC: the benchmark reports the kernels' rates against these
// beside the published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fc_gguf_ceilings.h"

namespace {

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx16 __attribute__((ext_vector_type(16)));

// Every thread reads U 16-byte words per round, rounds strided over the
// grid, and folds them into one word; the fold is stored only if it equals a
// value no input produces in practice, so the loads cannot be dropped and
// nothing is written.
template <int U>
__global__ void __launch_bounds__(256) stream_read_kernel(const uint4* __restrict__ src,
                                                          long long n16, uint32_t* sink) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Each wave issues `iters` rounds of four independent 32x32x16 f16 MFMAs.
__global__ void __launch_bounds__(256) mfma_f16_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  half8v a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(0.001f * (float)(lane + j));
    b[j] = (_Float16)(0.002f * (float)(lane - j));
  }
  floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  if (s == 1234.5f) sink[0] = s;
}

// The same with 32x32x32 int8 MFMAs.
__global__ void __launch_bounds__(256) mfma_i8_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  typedef int int4v __attribute__((ext_vector_type(4)));
  int4v a, b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = 0x01020304 * (lane + j + 1);
    b[j] = 0x05060708 ^ (lane * 131 + j);
  }
  intx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] ^ c1[j] ^ c2[j] ^ c3[j];
  if (s == 0x7654321) sink[0] = (float)s;
}

}  // namespace

extern "C" {

int fc_ceiling_stream_read(const void* src, int64_t bytes, int grid, int unroll, void* sink,
                           void* stream) {
  if (!src || !sink || bytes < 0 || (bytes % 16) != 0 || grid <= 0 ||
      ((uintptr_t)src % 16) != 0)
    return -1;
  const long long n16 = bytes / 16;
  hipStream_t st = (hipStream_t)stream;
  switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(grid), dim3(256), 0, st,
                               (const uint4*)src, n16, (uint32_t*)sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(grid), dim3(256), 0, st,
                               (const uint4*)src, n16, (uint32_t*)sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(256), 0, st,
                               (const uint4*)src, n16, (uint32_t*)sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(256), 0, st,
                               (const uint4*)src, n16, (uint32_t*)sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int fc_ceiling_mfma(int dtype, int iters, int grid, void* sink, void* stream) {
  if (!sink || iters <= 0 || grid <= 0 || (dtype != 0 && dtype != 1)) return -1;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == 0)
    hipLaunchKernelGGL(mfma_f16_kernel, dim3(grid), dim3(256), 0, st, iters, (float*)sink);
  else
    hipLaunchKernelGGL(mfma_i8_kernel, dim3(grid), dim3(256), 0, st, iters, (float*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
