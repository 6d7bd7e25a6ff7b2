// Weight layout transform, run once when a handle is created: canonical GGUF
// blocks (array of structures, row-major) -> the device layout of layout.h
// (piece-interleaved, for single-matrix handles) or the canonical device
// layout (Q4_K / Q5_K blocks in order, Q6_K row-major planes; for grouped handles,
// whose expert tiles read rows rather than runs of consecutive blocks).
//
// OpenVINO PR #39119, section Transformation: Q6_K blocks are regrouped into
// the planes QL | QH | SC | D with unchanged size and contents; here every
// plane (and the single Q4_K / Q5_K plane) is additionally piece-interleaved over
// groups of 64 blocks so that a wave reads 64 whole blocks with coalesced
// accesses.  One thread per destination byte (a one-time byte permutation).
#include "common.h"
#include "internal.h"
#include "layout.h"

namespace fcg {

// source (block b, byte f of the block) of destination byte o of a
// single-plane format (Q4_K, Q5_K) of BB = 16*P bytes per block
template <int BB, bool IL>
__device__ __forceinline__ void aos_src(size_t o, size_t& b, int& f) {
  constexpr int P = BB / 16;
  if constexpr (IL) {
    const size_t g = o / (P * 1024);
    const int r = (int)(o % (P * 1024));
    b = g * 64 + ((r >> 4) & 63);
    f = 16 * (r >> 10) + (r & 15);
  } else {
    b = o / BB;
    f = (int)(o % BB);
  }
}

// piece-interleaved plane of P pieces: (block, byte within the plane's part)
__device__ __forceinline__ void il_src(size_t q, int P, size_t& b, int& f) {
  const size_t g = q / ((size_t)P * 1024);
  const int r = (int)(q % ((size_t)P * 1024));
  b = g * 64 + ((r >> 4) & 63);
  f = 16 * (r >> 10) + (r & 15);
}

template <bool IL>
__device__ __forceinline__ void q6k_src(size_t o, size_t nbp, size_t& b, int& f) {
  if (o < q6k_qh_base(nbp)) {                       // QL, 8 pieces
    if constexpr (IL) il_src(o, 8, b, f);
    else { b = o / 128; f = (int)(o % 128); }
  } else if (o < q6k_sc_base(nbp)) {                // QH, 4 pieces
    const size_t q = o - q6k_qh_base(nbp);
    if constexpr (IL) il_src(q, 4, b, f);
    else { b = q / 64; f = (int)(q % 64); }
    f += 128;
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

template <int QT, bool IL>
__global__ void weight_layout_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                     size_t nblk) {
  const size_t nbp = padded_blocks(nblk);
  constexpr int BB = block_bytes_of(QT);
  const size_t total = (size_t)BB * nbp;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (size_t)gridDim.x * blockDim.x) {
    size_t b;
    int f;
    if constexpr (QT == QT_Q6K) q6k_src<IL>(o, nbp, b, f); else aos_src<BB, IL>(o, b, f);
    dst[o] = b < nblk ? src[b * BB + f] : (uint8_t)0;
  }
}

size_t layout_bytes(int qtype, size_t nblk) {
  return (size_t)block_bytes_of(qtype) * padded_blocks(nblk);
}

hipError_t launch_weight_layout(int qtype, bool interleaved, const uint8_t* src, uint8_t* dst,
                                size_t nblk, hipStream_t st) {
  const size_t total = layout_bytes(qtype, nblk);
  size_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  const dim3 g((unsigned)grid), b(256);
  if (qtype == QT_Q4K) {
    if (interleaved) hipLaunchKernelGGL((weight_layout_kernel<QT_Q4K, true>), g, b, 0, st, src, dst, nblk);
    else hipLaunchKernelGGL((weight_layout_kernel<QT_Q4K, false>), g, b, 0, st, src, dst, nblk);
  } else if (qtype == QT_Q5K) {
    if (interleaved) hipLaunchKernelGGL((weight_layout_kernel<QT_Q5K, true>), g, b, 0, st, src, dst, nblk);
    else hipLaunchKernelGGL((weight_layout_kernel<QT_Q5K, false>), g, b, 0, st, src, dst, nblk);
  } else {
    if (interleaved) hipLaunchKernelGGL((weight_layout_kernel<QT_Q6K, true>), g, b, 0, st, src, dst, nblk);
    else hipLaunchKernelGGL((weight_layout_kernel<QT_Q6K, false>), g, b, 0, st, src, dst, nblk);
  }
  return hipGetLastError();
}

}  // namespace fcg
