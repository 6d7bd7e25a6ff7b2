// Q6_K plane regroup, run once when a handle is created.
//
// OpenVINO PR #39119, section Transformation: Q6_K blocks are regrouped into
// aligned planes QL[nblk][128] | QH[nblk][64] | SC[nblk][16] | D[nblk]; the
// size and contents are unchanged.  Blocks are taken in row-major (n, kb)
// order.  One thread per destination byte (a one-time byte permutation).
#include "common.h"
#include "internal.h"

namespace fcg {

__global__ void q6k_regroup_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                   size_t nblk) {
  const size_t total = (size_t)Q6K_BYTES * nblk;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (size_t)gridDim.x * blockDim.x) {
    size_t b, f;
    if (o < 128 * nblk) {
      b = o / 128; f = o % 128;
    } else if (o < 192 * nblk) {
      const size_t r = o - 128 * nblk; b = r / 64; f = 128 + r % 64;
    } else if (o < 208 * nblk) {
      const size_t r = o - 192 * nblk; b = r / 16; f = 192 + r % 16;
    } else {
      const size_t r = o - 208 * nblk; b = r / 2; f = 208 + r % 2;
    }
    dst[o] = src[b * Q6K_BYTES + f];
  }
}

hipError_t launch_q6k_regroup(const uint8_t* src, uint8_t* dst, size_t nblk, hipStream_t st) {
  const size_t total = (size_t)Q6K_BYTES * nblk;
  size_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(q6k_regroup_kernel, dim3((unsigned)grid), dim3(256), 0, st, src, dst, nblk);
  return hipGetLastError();
}

}  // namespace fcg
