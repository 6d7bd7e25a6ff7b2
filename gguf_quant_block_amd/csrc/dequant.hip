// Dequantise-once comparison path: the tiled device weights -> a row-major f16
// matrix W16[N, K], which a vendor GEMM then multiplies.
//
// OpenVINO PR #39119, sections Details and Implementation (and the ROCm
// llama.cpp PR #37, one-time f16 dequantisation for prefill GEMMs, section
// How it works): devices without
// the decode-once matrix kernel decode the weights to a pooled f16 scratch
// buffer and run a library MatMul (the residual Add as its post-op); the
// testing option can force this path.  Here it is kept as a comparison
// against the direct prefill path (where the two cross over), and forced
// with FC_GGUF_PATH_SCRATCH.
//
// One thread per 8 consecutive values of a row (one 16-byte store; the 32
// threads of a block write its 512 bytes contiguously).  Weights are decoded
// in f32 from the formulas and rounded once to f16:
//   Q4_K / Q5_K  w = d * sc_j * q - dmin * m_j   (j = i / 32)
//   Q6_K         w = d * sc_s * (q - 32)         (s = i / 16)
#include "common.h"
#include "internal.h"
#include "layout.h"

namespace fcg {

__device__ __forceinline__ uint64_t ld8(const uint8_t* p) { return *(const uint64_t*)p; }

template <int QT>
__global__ void __launch_bounds__(256)
dequant_f16_kernel(const uint8_t* __restrict__ W, f16* __restrict__ out, int N, int K) {
  const WMap L(N, K);
  const int KB = L.KB;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)N * KB * 32) return;
  const int c = (int)(gid & 31);                    // 8-value chunk of the block
  const long long b = gid >> 5;
  const int n = (int)(b / KB), kb = (int)(b % KB);
  float w[8];
  if constexpr (QT != QT_Q6K) {
    constexpr int P = block_bytes_of(QT) / 16;
    auto byte_at = [&](int f) { return W + L.piece(n, kb, P, f >> 4) + (f & 15); };
    const uint4 hdr = *(const uint4*)byte_at(0);
    const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
    const int j = c >> 2;                           // sub-block of values 8c .. 8c+7
    const uint32_t hw[4] = {hdr.x, hdr.y, hdr.z, hdr.w};
    auto sb = [&](int k) { return (int)((hw[(4 + k) >> 2] >> (8 * ((4 + k) & 3))) & 0xFF); };   // scale byte k
    int sc, mn;
    if (j < 4) {
      sc = sb(j) & 63;
      mn = sb(j + 4) & 63;
    } else {
      sc = (sb(j + 4) & 15) | ((sb(j - 4) >> 6) << 4);
      mn = (sb(j + 4) >> 4) | ((sb(j) >> 6) << 4);
    }
    const int qs0 = QT == QT_Q5K ? 48 : 16;         // byte offset of qs in the block
    // values 8c .. 8c+7: bytes qs[32*(c/8) + 8*(c%4) ..], low nibbles if c%8 < 4
    const uint64_t qs = ld8(byte_at(qs0 + 32 * (c >> 3) + 8 * (c & 3)));
    const int hi = (c & 7) >= 4 ? 4 : 0;
    uint64_t qh = 0;
    if constexpr (QT == QT_Q5K) qh = ld8(byte_at(16 + 8 * (c & 3)));   // qh[i % 32]
    const float dsc = d * (float)sc, dmm = dmin * (float)mn;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int q = (int)((qs >> (8 * e + hi)) & 15);
      if constexpr (QT == QT_Q5K) q |= (int)((qh >> (8 * e + j)) & 1) << 4;
      w[e] = dsc * (float)q - dmm;
    }
  } else {
    // value i = 8c + e: h = c / 16, g = (c % 16) / 4, l = 8 (c % 4) + e
    const int h = c >> 4, g = (c & 15) >> 2;
    const uint64_t ql = ld8(W + L.piece(n, kb, 8, (64 * h + 32 * (g & 1) + 8 * (c & 3)) >> 4) +
                            ((8 * (c & 3)) & 15));
    const uint64_t qh = ld8(W + L.qh_base() + L.piece(n, kb, 4, (32 * h + 8 * (c & 3)) >> 4) +
                            ((8 * (c & 3)) & 15));
    const int sc = (int)(int8_t)W[L.sc(n, kb) + (c >> 1)];
    const float d = h2f(*(const uint16_t*)(W + L.d(n, kb)));
    const float dsc = d * (float)sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = (int)((ql >> (8 * e + 4 * (g >> 1))) & 15) | ((int)((qh >> (8 * e + 2 * g)) & 3) << 4);
      w[e] = dsc * (float)(q - 32);
    }
  }
  uint4 o;
  o.x = (uint32_t)f2h_bits(w[0]) | ((uint32_t)f2h_bits(w[1]) << 16);
  o.y = (uint32_t)f2h_bits(w[2]) | ((uint32_t)f2h_bits(w[3]) << 16);
  o.z = (uint32_t)f2h_bits(w[4]) | ((uint32_t)f2h_bits(w[5]) << 16);
  o.w = (uint32_t)f2h_bits(w[6]) | ((uint32_t)f2h_bits(w[7]) << 16);
  *(uint4*)(out + (size_t)n * K + (size_t)kb * QK + 8 * c) = o;
}

hipError_t launch_dequant_f16(int qtype, const uint8_t* W, f16* out, int N, int K,
                              hipStream_t st) {
  const long long threads = (long long)N * (K / QK) * 32;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (qtype == QT_Q4K)
    hipLaunchKernelGGL(dequant_f16_kernel<QT_Q4K>, dim3(grid), dim3(256), 0, st, W, out, N, K);
  else if (qtype == QT_Q5K)
    hipLaunchKernelGGL(dequant_f16_kernel<QT_Q5K>, dim3(grid), dim3(256), 0, st, W, out, N, K);
  else
    hipLaunchKernelGGL(dequant_f16_kernel<QT_Q6K>, dim3(grid), dim3(256), 0, st, W, out, N, K);
  return hipGetLastError();
}

}  // namespace fcg
