// Weight layout transform, run once when a handle is created: canonical GGUF
// blocks (array of structures, row-major) -> the device layout of layout.h.
//
// OpenVINO PR #39119, section Transformation: Q6_K blocks are regrouped into
// the planes QL | QH | SC | D with unchanged size and contents; here every
// plane (and the single Q5_K plane) is additionally piece-interleaved over
// groups of 64 blocks so that a wave reads 64 whole blocks with coalesced
// accesses.  One thread per destination byte (a one-time byte permutation).
#include "common.h"
#include "internal.h"
#include "layout.h"

namespace fcg {

// source (block b, byte f of the block) of destination byte o
__device__ __forceinline__ void q5k_src(size_t o, size_t& b, int& f) {
  const size_t g = o / (11 * 1024);
  const int r = (int)(o % (11 * 1024));
  const int p = r >> 10, l = (r >> 4) & 63;
  b = g * 64 + l;
  f = 16 * p + (r & 15);
}

__device__ __forceinline__ void q6k_src(size_t o, size_t nbp, size_t& b, int& f) {
  if (o < q6k_qh_base(nbp)) {                       // QL, 8 pieces
    const size_t g = o / (8 * 1024);
    const int r = (int)(o % (8 * 1024));
    b = g * 64 + ((r >> 4) & 63);
    f = 16 * (r >> 10) + (r & 15);
  } else if (o < q6k_sc_base(nbp)) {                // QH, 4 pieces
    const size_t q = o - q6k_qh_base(nbp);
    const size_t g = q / (4 * 1024);
    const int r = (int)(q % (4 * 1024));
    b = g * 64 + ((r >> 4) & 63);
    f = 128 + 16 * (r >> 10) + (r & 15);
  } else if (o < q6k_d_base(nbp)) {                 // SC, block order
    const size_t q = o - q6k_sc_base(nbp);
    b = q / 16;
    f = 192 + (int)(q % 16);
  } else {                                          // D, block order
    const size_t q = o - q6k_d_base(nbp);
    b = q / 2;
    f = 208 + (int)(q % 2);
  }
}

template <int QT>
__global__ void weight_layout_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                     size_t nblk) {
  const size_t nbp = padded_blocks(nblk);
  constexpr int BB = QT == QT_Q5K ? Q5K_BYTES : Q6K_BYTES;
  const size_t total = (size_t)BB * nbp;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (size_t)gridDim.x * blockDim.x) {
    size_t b;
    int f;
    if constexpr (QT == QT_Q5K) q5k_src(o, b, f); else q6k_src(o, nbp, b, f);
    dst[o] = b < nblk ? src[b * BB + f] : (uint8_t)0;
  }
}

size_t layout_bytes(int qtype, size_t nblk) {
  return (size_t)(qtype == QT_Q5K ? Q5K_BYTES : Q6K_BYTES) * padded_blocks(nblk);
}

hipError_t launch_weight_layout(int qtype, const uint8_t* src, uint8_t* dst, size_t nblk,
                                hipStream_t st) {
  const size_t total = layout_bytes(qtype, nblk);
  size_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  if (qtype == QT_Q5K)
    hipLaunchKernelGGL(weight_layout_kernel<QT_Q5K>, dim3((unsigned)grid), dim3(256), 0, st, src,
                       dst, nblk);
  else
    hipLaunchKernelGGL(weight_layout_kernel<QT_Q6K>, dim3((unsigned)grid), dim3(256), 0, st, src,
                       dst, nblk);
  return hipGetLastError();
}

}  // namespace fcg
