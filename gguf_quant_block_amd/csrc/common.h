// Shared device helpers for the GGUF K-quant FC kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fcg {

typedef _Float16 f16;
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16-byte register chunk

constexpr int QK = 256;          // values per super-block
constexpr int Q4K_BYTES = 144;   // d, dmin, scales[12], qs[128]
constexpr int Q5K_BYTES = 176;   // d, dmin, scales[12], qh[32], qs[128]
constexpr int Q6K_BYTES = 210;   // ql[128], qh[64], sc[16], d
constexpr int QT_Q4K = 4;
constexpr int QT_Q5K = 5;
constexpr int QT_Q6K = 6;

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(f16, (uint16_t)(bits16 & 0xFFFFu));
}

__device__ __forceinline__ uint16_t f2h_bits(float x) {
  return __builtin_bit_cast(uint16_t, (f16)x);   // round to nearest even
}

// signed 8-bit x 4 dot product accumulated into c (v_dot4_i32_i8)
__device__ __forceinline__ int dot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

__device__ __forceinline__ int sext8(uint32_t x) { return (int)(int8_t)(x & 0xFF); }

// bytes per super-block and 16-byte pieces per block (Q6_K: the sum over its planes)
__host__ __device__ constexpr int block_bytes_of(int qt) {
  return qt == QT_Q4K ? Q4K_BYTES : (qt == QT_Q5K ? Q5K_BYTES : Q6K_BYTES);
}

}  // namespace fcg
