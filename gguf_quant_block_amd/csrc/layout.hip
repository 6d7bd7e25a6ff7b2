// Weight layout transform, run once when a handle is created: canonical GGUF
// blocks (array of structures, row-major) -> the tiled device layout of
// layout.h (every handle; grouped handles per expert).
//
// OpenVINO PR #39119, section Transformation: Q6_K blocks are regrouped into
// the planes QL | QH | SC | D with unchanged size and contents; here every
// plane (and the single Q4_K / Q5_K plane) is additionally cut into tiles of
// 16 rows x 4 blocks stored piece-major, so that both the GEMV waves and the
// matrix-core tiles read their blocks with coalesced accesses.  One thread
// per destination byte (a one-time byte permutation).
#include "common.h"
#include "internal.h"
#include "layout.h"

namespace fcg {

// source (row n, block kb, byte f of the block) of destination byte o;
// false for padding
template <int QT>
__device__ __forceinline__ bool layout_src(size_t o, const WMap& L, int& n, int& kb, int& f) {
  constexpr int BB = block_bytes_of(QT);
  // position inside a plane of P pieces per block -> (block, byte of the plane's part)
  auto from_plane = [&](size_t q, int P) {
    const size_t t = q / ((size_t)P * 1024);
    const int r = (int)(q % ((size_t)P * 1024));
    const int l = (r >> 4) & 63;
    const int tiles_k = L.KBp / TILE_KB;
    n = (int)(t / tiles_k) * TILE_ROWS + (l % TILE_ROWS);
    kb = (int)(t % tiles_k) * TILE_KB + l / TILE_ROWS;
    f = 16 * (r >> 10) + (r & 15);
  };
  if constexpr (QT != QT_Q6K) {
    from_plane(o, BB / 16);
  } else if (o < L.qh_base()) {                       // QL, 8 pieces
    from_plane(o, 8);
  } else if (o < L.sc_base()) {                       // QH, 4 pieces
    from_plane(o - L.qh_base(), 4);
    f += 128;
  } else if (o < L.d_base()) {                        // SC, 1 piece
    from_plane(o - L.sc_base(), 1);
    f += 192;
  } else {                                            // D, 2 bytes per block
    const size_t q = o - L.d_base();
    const size_t t = q / 128;
    const int l = (int)(q % 128) / 2;
    const int tiles_k = L.KBp / TILE_KB;
    n = (int)(t / tiles_k) * TILE_ROWS + (l % TILE_ROWS);
    kb = (int)(t % tiles_k) * TILE_KB + l / TILE_ROWS;
    f = 208 + (int)(q % 2);
  }
  return kb < L.KB;                                   // (rows past N are checked by the caller)
}

template <int QT>
__global__ void weight_layout_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                     int N, int K) {
  constexpr int BB = block_bytes_of(QT);
  const WMap L(N, K);
  const size_t total = (size_t)BB * L.nbt;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (size_t)gridDim.x * blockDim.x) {
    int n, kb, f;
    const bool in = layout_src<QT>(o, L, n, kb, f) && n < N;
    dst[o] = in ? src[((size_t)n * L.KB + kb) * BB + f] : (uint8_t)0;
  }
}

size_t layout_bytes(int qtype, int N, int K) {
  return (size_t)block_bytes_of(qtype) * WMap(N, K).nbt;
}

hipError_t launch_weight_layout(int qtype, const uint8_t* src, uint8_t* dst, int N, int K,
                                hipStream_t st) {
  const size_t total = layout_bytes(qtype, N, K);
  size_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  const dim3 g((unsigned)grid);
  if (qtype == QT_Q4K)
    hipLaunchKernelGGL(weight_layout_kernel<QT_Q4K>, g, dim3(256), 0, st, src, dst, N, K);
  else if (qtype == QT_Q5K)
    hipLaunchKernelGGL(weight_layout_kernel<QT_Q5K>, g, dim3(256), 0, st, src, dst, N, K);
  else
    hipLaunchKernelGGL(weight_layout_kernel<QT_Q6K>, g, dim3(256), 0, st, src, dst, N, K);
  return hipGetLastError();
}

}  // namespace fcg
