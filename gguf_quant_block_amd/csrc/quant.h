// Per-32 int8 activation quantisation shared by the decode GEMV (fused into
// its launch), the int8 matrix-core prefill (a pass of its own) and the
// debug export: the one routine, so every path sees bit-identical codes and
// scales.
#pragma once

#include <type_traits>

#include "common.h"

namespace fcg {

constexpr float RNE_MAGIC = 12582912.0f;   // 1.5 * 2^23: x + magic rounds x to an integer, ties to even

// ------------------------------------------------ activation quantisation --
// Per-32 int8 quantisation (OpenVINO PR #39119, sections Transformation and
// Implementation: dynamic quantisation in groups of 32 for the int8 GEMV;
// f16 activations, and f32 activations at any row count, take this path).
// Symmetric: s = amax/127, inv = 127/amax (IEEE-correct f32 divisions),
// code = round-half-even(fl32(a * inv)); |fl32(a * inv)| <= 127.5 so no clamp
// is needed.  An all-zero group, or an f32 group so small that 127/amax
// overflows (amax < 127/FLT_MAX), gives s = 0 and codes 0.
//
// The lanes of a group share it: each lane holds one 16-byte chunk of the
// group's values (8 f16 values, the group on 4 consecutive lanes; or 4 f32
// values, on 8 lanes), so that a wave's loads of consecutive chunks are
// contiguous; the group's lanes exchange their maxima and sums over DPP.  round-half-even(fl32(a * inv)) lands in the low byte of the
// result.  The product is rounded to f32 first and only then rounded to an
// integer (adding 1.5*2^23 rounds to the nearest integer, ties to even, for
// |x| < 2^22); the empty asm keeps the compiler from fusing the two into one
// fma, which would round the exact product once and differ on ties.
__device__ __forceinline__ uint32_t rne_code(float a, float inv) {
  float p = a * inv;
  asm volatile("" : "+v"(p));
  return __builtin_bit_cast(uint32_t, p + RNE_MAGIC);
}

// Lane exchanges inside the 4 or 8 lanes of a group, on the DPP crossbar
// (an operand modifier of the consuming instruction; no LDS round trip):
// xor 1 and xor 2 within an aligned quad, and the mirror of an aligned
// 8-lane half row (lane i <-> 7 - i), which pairs each lane of one quad with
// one of the other.  Every lane of the group must be active.
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;  // row_half_mirror
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true); }
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}

template <class AT>
constexpr int chunk_vals() { return 16 / (int)sizeof(AT); }       // values per 16-byte chunk
template <class AT>
constexpr int group_lanes() { return 32 / chunk_vals<AT>(); }     // lanes per 32-value group

// Quantise the lane's chunk: raw = its 16 bytes; the group starts at a lane
// index that is a multiple of group_lanes<AT>(), and every lane of the wave
// takes part (cross-lane shuffles).  Out:
//   q[0 .. chunk_vals/4):  packed int8 codes of the chunk's values
//   s:                     the group's scale (every lane of the group)
//   tsum:                  sum of the group's 32 codes (every lane)
//   thalf:                 sum of the 16 codes of the lane's half of the group
template <class AT>
__device__ __forceinline__ void quant_chunk(uint4 raw, uint32_t* q, float& s, int& tsum,
                                            int& thalf) {
  constexpr int GL = group_lanes<AT>();
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  auto value = [&](int i) -> float {
    if constexpr (std::is_same<AT, f16>::value) return h2f(w[i >> 1] >> (16 * (i & 1)));
    else return __builtin_bit_cast(float, w[i]);
  };
  float amax;
  if constexpr (std::is_same<AT, f16>::value) {
    half2v m2 = {(f16)0.f, (f16)0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(half2v, w[j] & 0x7FFF7FFFu));
    amax = fmaxf((float)m2[0], (float)m2[1]);
  } else {
    amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, __builtin_bit_cast(float, w[j] & 0x7FFFFFFFu));
  }
  amax = fmaxf(amax, dpp_f<DPP_XOR1>(amax));
  amax = fmaxf(amax, dpp_f<DPP_XOR2>(amax));
  if constexpr (GL == 8) amax = fmaxf(amax, dpp_f<DPP_HALF_MIRROR>(amax));
  float inv = 0.f;
  s = 0.f;
  if (amax > 0.f) {
    inv = __fdiv_rn(127.0f, amax);
    if (inv <= 3.402823466e38f) s = __fdiv_rn(amax, 127.0f);   // inv finite
    else inv = 0.f;
  }
  int p = 0;
#pragma unroll
  for (int c = 0; c < chunk_vals<AT>() / 4; ++c) {
    // four values -> four rounded floats -> the low byte of each is the code
    const uint32_t r0 = rne_code(value(4 * c), inv);
    const uint32_t r1 = rne_code(value(4 * c + 1), inv);
    const uint32_t r2 = rne_code(value(4 * c + 2), inv);
    const uint32_t r3 = rne_code(value(4 * c + 3), inv);
    const uint32_t lo = __builtin_amdgcn_perm(r1, r0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(r3, r2, 0x0c0c0400u);
    q[c] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    p = dot4((int)q[c], 0x01010101, p);
  }
  // code sums: over the lanes of the half (2 or 4 lanes), then of the group
  p += dpp_i<DPP_XOR1>(p);
  if constexpr (GL == 8) p += dpp_i<DPP_XOR2>(p);
  thalf = p;
  if constexpr (GL == 8) tsum = p + dpp_i<DPP_HALF_MIRROR>(p);
  else tsum = p + dpp_i<DPP_XOR2>(p);
}

}  // namespace fcg
