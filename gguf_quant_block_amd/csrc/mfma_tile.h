// Matrix-core tile machinery shared by the dense prefill FC and the grouped
// (MoE expert) FC: raw K-quant block loads, exact decode of a half
// super-block into v_mfma_f32_16x16x32_f16 operand registers, and the
// double-buffered main loop over K.
//
// OpenVINO PR #39119, section Implementation: every weight value is decoded
// once per workgroup and reused across all the activation rows of the tile.
//
// Tile: one workgroup = 4 waves; BM = 16*MT activation rows, BN = 64*NT
// weight rows, K walked in half super-blocks of 128 values.
//   * The activation tile [BM x 128] f16 is staged global -> registers -> LDS,
//     double-buffered: the next stage's loads are in flight while the current
//     stage runs on the matrix cores.  Rows are addressed through per-thread
//     row pointers, so the caller decides which rows form the tile (a dense
//     range, or the gathered rows of one expert).
//   * Each wave owns 16*NT weight rows.  Its lanes load those rows' raw block
//     bytes one stage ahead and decode them straight into the MFMA operand
//     registers (Q45Half / Q6Half): a byte permute builds the magic f16
//     (1024 + q); Q4_K / Q5_K: fma(1024+q, sc, -1024*sc) = sc*q exactly, then
//     w = (sc*q)*d - dmin*m with one rounding; Q6_K: w = (q - 32)*(sc*d).
//   * Only the first MTA 16-row halves of the tile are staged and run on the
//     matrix cores: a tile whose rows end early skips its empty halves
//     (llama.cpp PR #28301, section Overview, skips the empty upper half of
//     under-filled expert tiles the same way).
#pragma once

#include <type_traits>

#include "common.h"
#include "layout.h"

namespace fcg {

constexpr int KSTAGE = 128;          // values of K per half super-block
// A stage covers SH half super-blocks (SH = 1 or 2); its LDS activation
// tile has a row stride of astr(SH) halves (16 bytes of padding per row).
__host__ __device__ constexpr int astr(int SH) { return KSTAGE * SH + 8; }
constexpr int ASTR = astr(1);

struct RawQ5 {  // one lane, one row, one half-block
  uint4 hdr;    // d | dmin, scales[0..3], scales[4..7], scales[8..11]
  uint2 qsA;    // qs[64hb + 8kq .. +8]      : sub-blocks 4hb+0 (lo), 4hb+1 (hi)
  uint2 qsB;    // qs[64hb + 32 + 8kq .. +8] : sub-blocks 4hb+2 (lo), 4hb+3 (hi)
  uint2 qh;     // qh[8kq .. +8]
};
struct RawQ4 {  // one lane, one row, one half-block
  uint4 hdr;    // d | dmin, scales[0..3], scales[4..7], scales[8..11]
  uint2 qsA;    // qs[64hb + 8kq .. +8]      : sub-blocks 4hb+0 (lo), 4hb+1 (hi)
  uint2 qsB;    // qs[64hb + 32 + 8kq .. +8] : sub-blocks 4hb+2 (lo), 4hb+3 (hi)
};
struct RawQ6 {
  uint2 qlA;    // ql[64hb + 8kq .. +8]      : groups g=0 (lo), g=2 (hi)
  uint2 qlB;    // ql[64hb + 32 + 8kq .. +8] : groups g=1 (lo), g=3 (hi)
  uint2 qh;     // qh[32hb + 8kq .. +8]
  uint2 sc;     // sc[8hb .. 8hb+7]
  uint32_t d;   // f16 bits
};

__device__ __forceinline__ half2v magic_pair(uint32_t codes, uint32_t sel) {
  // bytes {code, 0x64, code', 0x64} -> f16 (1024 + code, 1024 + code')
  return __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, codes, sel));
}

__device__ __forceinline__ half8v make_frag(half2v a, half2v b, half2v c, half2v d) {
  half8v f;
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
  return f;
}

// Codes (packed bytes, 8 values) -> 8 f16 weights: w = d*(sc*q) - dmm.
__device__ __forceinline__ half8v decode8(uint32_t c0, uint32_t c1, half2v sc2, half2v bias2,
                                          half2v d2, half2v negdmm2) {
  half2v p0 = magic_pair(c0, 0x04010400u), p1 = magic_pair(c0, 0x04030402u);
  half2v p2 = magic_pair(c1, 0x04010400u), p3 = magic_pair(c1, 0x04030402u);
  p0 = __builtin_elementwise_fma(p0, sc2, bias2);
  p1 = __builtin_elementwise_fma(p1, sc2, bias2);
  p2 = __builtin_elementwise_fma(p2, sc2, bias2);
  p3 = __builtin_elementwise_fma(p3, sc2, bias2);
  p0 = __builtin_elementwise_fma(p0, d2, negdmm2);
  p1 = __builtin_elementwise_fma(p1, d2, negdmm2);
  p2 = __builtin_elementwise_fma(p2, d2, negdmm2);
  p3 = __builtin_elementwise_fma(p3, d2, negdmm2);
  return make_frag(p0, p1, p2, p3);
}

__device__ __forceinline__ half2v splat(f16 x) { half2v r; r[0] = x; r[1] = x; return r; }

// Q4_K / Q5_K half-block decoder: a per-half setup, then the lane's 8
// weights of k-step g = 0..3 (values 128hb + 32g + 8kq .. +7 of its row).
// Decoding is exact up to one f16 rounding: (1024 + q) * sc - 1024 * sc =
// sc * q exactly (sc * q <= 63 * 31 < 2048), then w = (sc * q) * d - dmin * m.
// The four sub-blocks' scales and mins become exact f16 pairs with packed
// arithmetic: magic f16 (1024 + byte) - 1024; bias = -1024 * sc is exact (a
// power-of-two product; |bias| <= 64512), and -dmin * m is one correctly
// rounded f16 product.  Q4_K: HAS_QH = false (no fifth bit).
template <bool HAS_QH>
struct Q45Half {
  half2v sc01, sc23, b01, b23, m01, m23, d2;
  uint32_t a0, a1, b0, b1;      // qsA.x, qsA.y, qsB.x, qsB.y
  uint32_t qhx, qhy;            // fifth bits of this half's sub-blocks at bits 0..3

  __device__ __forceinline__ void init(uint4 hdr, uint2 qsA, uint2 qsB, uint2 qh, int hb) {
    const uint32_t w0 = hdr.y, w1 = hdr.z, w2 = hdr.w;
    // bytes g = 0..3: scale / min of sub-block 4hb + g (selected without a
    // branch, so that the setup schedules freely among the matrix-core work)
    const uint32_t hi = 0u - (uint32_t)hb;
    const uint32_t scb = (w0 & 0x3F3F3F3Fu & ~hi) |
                         (((w2 & 0x0F0F0F0Fu) | ((w0 >> 2) & 0x30303030u)) & hi);
    const uint32_t mb = (w1 & 0x3F3F3F3Fu & ~hi) |
                        ((((w2 >> 4) & 0x0F0F0F0Fu) | ((w1 >> 2) & 0x30303030u)) & hi);
    const half2v k1024 = splat((f16)1024.f), nk = splat((f16)-1024.f);
    sc01 = magic_pair(scb, 0x04010400u) - k1024;
    sc23 = magic_pair(scb, 0x04030402u) - k1024;
    b01 = sc01 * nk;
    b23 = sc23 * nk;
    const half2v ndmin = splat(-__builtin_bit_cast(f16, (uint16_t)(hdr.x >> 16)));
    m01 = (magic_pair(mb, 0x04010400u) - k1024) * ndmin;
    m23 = (magic_pair(mb, 0x04030402u) - k1024) * ndmin;
    d2 = splat(__builtin_bit_cast(f16, (uint16_t)(hdr.x & 0xFFFF)));
    a0 = qsA.x; a1 = qsA.y; b0 = qsB.x; b1 = qsB.y;
    if constexpr (HAS_QH) {
      qhx = qh.x >> (4 * hb);
      qhy = qh.y >> (4 * hb);
    } else {
      qhx = qhy = 0;
    }
  }
  __device__ __forceinline__ half8v frag(int g) const {
    const int sh = 4 * (g & 1);
    const uint32_t s0 = g < 2 ? a0 : b0, s1 = g < 2 ? a1 : b1;
    uint32_t c0 = (s0 >> sh) & 0x0F0F0F0Fu;
    uint32_t c1 = (s1 >> sh) & 0x0F0F0F0Fu;
    if constexpr (HAS_QH) {
      c0 |= (qhx << (4 - g)) & 0x10101010u;
      c1 |= (qhy << (4 - g)) & 0x10101010u;
    }
    const half2v scp = g < 2 ? sc01 : sc23, bp = g < 2 ? b01 : b23, mp = g < 2 ? m01 : m23;
    return decode8(c0, c1, splat(scp[g & 1]), splat(bp[g & 1]), d2, splat(mp[g & 1]));
  }
};

// Q6_K half-block decoder (same k-step layout).  w = (q - 32) * (sc * d):
// (1024 + q) - 1056 = q - 32 exactly, and sc * d is one f16 product of the
// signed 8-bit scale and d; two roundings in all, with no intermediate
// beyond the weight's own magnitude for any scale in [-128, 127].
struct Q6Half {
  half2v scd01, scd23;          // sc * d of the lane's sub-blocks for k-steps 0, 1 | 2, 3
  uint32_t la0, la1, lb0, lb1;  // qlA.x, qlA.y, qlB.x, qlB.y
  uint32_t qhx, qhy;

  __device__ __forceinline__ void init(uint2 qlA, uint2 qlB, uint2 qh, uint2 sc, uint32_t dbits,
                                       int kq) {
    // sub-block of k-step g within the half: 2g + kq/2 (bytes p, 2 + p of
    // sc.x and p, 2 + p of sc.y, p = kq/2), offset to unsigned for the magic
    const uint32_t p = (uint32_t)(kq >> 1);
    const uint32_t sel = p | ((p + 2) << 8) | ((p + 4) << 16) | ((p + 6) << 24);
    const uint32_t u = __builtin_amdgcn_perm(sc.y, sc.x, sel) ^ 0x80808080u;
    const half2v k1152 = splat((f16)1152.f);
    const half2v d2 = splat(__builtin_bit_cast(f16, (uint16_t)(dbits & 0xFFFF)));
    scd01 = (magic_pair(u, 0x04010400u) - k1152) * d2;
    scd23 = (magic_pair(u, 0x04030402u) - k1152) * d2;
    la0 = qlA.x; la1 = qlA.y; lb0 = qlB.x; lb1 = qlB.y;
    qhx = qh.x;
    qhy = qh.y;
  }
  __device__ __forceinline__ half8v frag(int g) const {
    const int sh = 4 * (g >> 1);
    const uint32_t s0 = (g & 1) ? lb0 : la0, s1 = (g & 1) ? lb1 : la1;
    const uint32_t hx = g < 3 ? (qhx << (4 - 2 * g)) : (qhx >> 2);
    const uint32_t hy = g < 3 ? (qhy << (4 - 2 * g)) : (qhy >> 2);
    const uint32_t c0 = ((s0 >> sh) & 0x0F0F0F0Fu) | (hx & 0x30303030u);
    const uint32_t c1 = ((s1 >> sh) & 0x0F0F0F0Fu) | (hy & 0x30303030u);
    const half2v scd = splat((g < 2 ? scd01 : scd23)[g & 1]);
    const half2v k1056 = splat((f16)1056.f);
    const half2v p0 = (magic_pair(c0, 0x04010400u) - k1056) * scd;
    const half2v p1 = (magic_pair(c0, 0x04030402u) - k1056) * scd;
    const half2v p2 = (magic_pair(c1, 0x04010400u) - k1056) * scd;
    const half2v p3 = (magic_pair(c1, 0x04030402u) - k1056) * scd;
    return make_frag(p0, p1, p2, p3);
  }
};

__device__ __forceinline__ void decode_q5k_half(const RawQ5& r, int hb, half8v out[4]) {
  Q45Half<true> h;
  h.init(r.hdr, r.qsA, r.qsB, r.qh, hb);
#pragma unroll
  for (int g = 0; g < 4; ++g) out[g] = h.frag(g);
}
__device__ __forceinline__ void decode_q4k_half(const RawQ4& r, int hb, half8v out[4]) {
  Q45Half<false> h;
  h.init(r.hdr, r.qsA, r.qsB, uint2{0u, 0u}, hb);
#pragma unroll
  for (int g = 0; g < 4; ++g) out[g] = h.frag(g);
}
__device__ __forceinline__ void decode_q6k_half(const RawQ6& r, int kq, half8v out[4]) {
  Q6Half h;
  h.init(r.qlA, r.qlB, r.qh, r.sc, r.d, kq);
#pragma unroll
  for (int g = 0; g < 4; ++g) out[g] = h.frag(g);
}


// Per-thread view of the tile rows.  Thread tid stages the 16-byte chunks
// c = tid + 256*i (i < MT) of the activation tile: tile row c >> 4 (inside
// half i), column chunk c & 15.  a_ld[i] points at that row of A; rows past
// the end of the tile point at any valid row (their outputs are never
// stored, and an output row depends only on its own activation row).
template <int MT>
struct TileRows {
  const f16* a_ld[MT];
};

// Main loop of one tile over the stages [s_begin, s_end) of K, walked from
// stage s_begin + rot (wrapping), for the first MTA (<= MT) 16-row halves of
// the tile.  W is one weight matrix [N, K] in the tiled device layout of
// layout.h.  n0 is its
// first weight row (rows past N are clamped to N - 1: loaded, never stored).
// acc[i][j] receives C[n][m] of the 16x16 sub-tile (half i < MTA, weight
// sub-tile j).  A stage is SH half super-blocks (128*SH values of K; stages
// are numbered in those units).  PD = 1: the next stage's loads are in flight
// while a stage computes; PD = 2: the next two stages' (three register sets).
// The loop body has no data-dependent branches.
template <int QT, int MT, int NT, int MTA, int PD, int SH = 1>
__device__ __forceinline__ void tile_mainloop(const uint8_t* W, int N,
                                              int K, int n0, int s_begin, int s_end, int rot,
                                              const TileRows<MT>& rows,
                                              f16 (*As)[16 * MT * astr(SH)],
                                              floatx4 (&acc)[MT][NT]) {
  static_assert(MTA >= 1 && MTA <= MT, "active halves");
  static_assert(PD == 1 || PD == 2, "prefetch depth");
  static_assert(SH == 1 || SH == 2, "halves per stage");
  constexpr int AS = astr(SH);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kq = lane >> 4;

  // rows of this lane's weight fragments
  int nrow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = n0 + wave * 16 * NT + 16 * j + (lane & 15);
    nrow[j] = n < N ? n : N - 1;
  }

  const WMap L(N, K);
  // raw bytes of the lane's rows for stage s (half-block hb of block kb):
  // 8-byte slices of the 16-byte pieces.  A piece's byte offset in a plane
  // of P pieces per block, ((n/16 * KBp/4 + kb/4) * P + p) * 1024 +
  // ((kb%4) * 16 + n%16) * 16, splits into a part that depends on the lane
  // only (its row, its k-quarter's piece and half) and a part that depends on
  // the stage only, so each load is a wave-uniform base plus a 32-bit lane
  // offset fixed for the whole loop (one matrix is far below 4 GB).
  const uint32_t G4 = (uint32_t)(L.KBp / TILE_KB);
  const uint32_t sub = 8u * (uint32_t)(kq & 1), pq = (uint32_t)(kq >> 1);
  uint32_t rtile[NT], drow[NT];   // tiles before the row's row tile; the row's offset in D
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    rtile[j] = (uint32_t)nrow[j] / TILE_ROWS * G4;
    drow[j] = rtile[j] * 128u + ((uint32_t)nrow[j] % TILE_ROWS) * 2u;
  }
  auto rowoff = [&](int j, uint32_t P) -> uint32_t {  // the lane's offset in a P-piece plane
    return ((rtile[j] * P) << 10) + ((uint32_t)nrow[j] % TILE_ROWS) * 16u;
  };
  // the stage part: block kb's tile and slot column
  auto kbterm = [&](int kb, uint32_t P) -> uint32_t {
    return (((uint32_t)kb >> 2) * P << 10) + (((uint32_t)kb & 3u) << 8);
  };
  auto load_raw_q5 = [&](int s, RawQ5* raw) {
    const int kb = s >> 1, hb = s & 1;
    const uint8_t* Ws = W + kbterm(kb, 11);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t o = rowoff(j, 11);
      raw[j].hdr = *(const uint4*)(Ws + o);
      raw[j].qsA = *(const uint2*)(Ws + (o + ((3u + 4u * hb + pq) << 10) + sub));
      raw[j].qsB = *(const uint2*)(Ws + (o + ((5u + 4u * hb + pq) << 10) + sub));
      raw[j].qh = *(const uint2*)(Ws + (o + ((1u + pq) << 10) + sub));
    }
  };
  auto load_raw_q4 = [&](int s, RawQ4* raw) {
    const int kb = s >> 1, hb = s & 1;
    const uint8_t* Ws = W + kbterm(kb, 9);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t o = rowoff(j, 9);
      raw[j].hdr = *(const uint4*)(Ws + o);
      raw[j].qsA = *(const uint2*)(Ws + (o + ((1u + 4u * hb + pq) << 10) + sub));
      raw[j].qsB = *(const uint2*)(Ws + (o + ((3u + 4u * hb + pq) << 10) + sub));
    }
  };
  auto load_raw_q6 = [&](int s, RawQ6* raw) {
    const int kb = s >> 1, hb = s & 1;
    const uint8_t* Wl = W + kbterm(kb, 8);
    const uint8_t* Wh = W + L.qh_base() + kbterm(kb, 4);
    const uint8_t* Wc = W + L.sc_base() + kbterm(kb, 1);
    const uint8_t* Wd = W + L.d_base() + ((uint32_t)kb >> 2) * 128u + ((uint32_t)kb & 3u) * 32u;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t ol = rowoff(j, 8), oh = rowoff(j, 4), oc = rowoff(j, 1);
      raw[j].qlA = *(const uint2*)(Wl + (ol + ((4u * hb + pq) << 10) + sub));
      raw[j].qlB = *(const uint2*)(Wl + (ol + ((4u * hb + 2u + pq) << 10) + sub));
      raw[j].qh = *(const uint2*)(Wh + (oh + ((2u * hb + pq) << 10) + sub));
      raw[j].sc = *(const uint2*)(Wc + (oc + 8u * hb));
      raw[j].d = *(const uint16_t*)(Wd + drow[j]);
    }
  };
  using Raw = typename std::conditional<
      QT == QT_Q5K, RawQ5, typename std::conditional<QT == QT_Q4K, RawQ4, RawQ6>::type>::type;
  // the raw bytes of stage s: its SH half-blocks (half index SH*s + x)
  auto load_raw = [&](int s, Raw (*raw)[NT]) {
#pragma unroll
    for (int x = 0; x < SH; ++x) {
      if constexpr (QT == QT_Q5K) load_raw_q5(SH * s + x, raw[x]);
      else if constexpr (QT == QT_Q4K) load_raw_q4(SH * s + x, raw[x]);
      else load_raw_q6(SH * s + x, raw[x]);
    }
  };

  // activation stage: 16*MTA rows x 128*SH halves, MTA*SH chunks of 16 B per thread
  auto load_a = [&](int s, u32x4 (*areg)[SH]) {
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int x = 0; x < SH; ++x)
        areg[i][x] = *(const u32x4*)(rows.a_ld[i] + (size_t)(SH * s + x) * KSTAGE + 8 * (tid & 15));
  };
  auto store_a = [&](int buf, u32x4 (*areg)[SH]) {
#pragma unroll
    for (int i = 0; i < MTA; ++i) {
      const int c = tid + 256 * i;
#pragma unroll
      for (int x = 0; x < SH; ++x)
        *(u32x4*)(&As[buf][(c >> 4) * AS + KSTAGE * x + 8 * (c & 15)]) = areg[i][x];
    }
  };
  // one stage on the matrix cores: decode the lane's weight fragments, then
  // C += W_frag x A_frag over the four 32-value k-steps of each half
  auto compute = [&](int s, int buf, Raw (*raw)[NT]) {
#pragma unroll
    for (int x = 0; x < SH; ++x) {
      half8v wf[NT][4];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if constexpr (QT == QT_Q5K) decode_q5k_half(raw[x][j], (SH * s + x) & 1, wf[j]);
        else if constexpr (QT == QT_Q4K) decode_q4k_half(raw[x][j], (SH * s + x) & 1, wf[j]);
        else decode_q6k_half(raw[x][j], kq, wf[j]);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        half8v af[MTA];
#pragma unroll
        for (int i = 0; i < MTA; ++i)
          af[i] = *(const half8v*)(&As[buf][(16 * i + (lane & 15)) * AS + KSTAGE * x + 32 * g + 8 * kq]);
#pragma unroll
        for (int i = 0; i < MTA; ++i)
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[j][g], af[i], acc[i][j], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int i = 0; i < MTA; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // stage t of the loop is stage s_begin + (t + rot) mod nst of K
  const int nst = s_end - s_begin;
  auto stage = [&](int t) {
    int u = t + rot;
    if (u >= nst) u -= nst;
    return s_begin + u;
  };

  if constexpr (PD == 1) {
    Raw rawc[SH][NT], rawn[SH][NT];
    u32x4 areg[MTA][SH];
    if (nst > 0) {
      load_a(stage(0), areg);
      load_raw(stage(0), rawc);
      store_a(0, areg);
    }
    // drain the prologue: the loop then starts with no load in flight, and
    // the waits of its body cover only the loads of the body itself
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < nst; ++t) {
      const bool more = t + 1 < nst;
      if (more) {
        load_a(stage(t + 1), areg);
        load_raw(stage(t + 1), rawn);
      }
      // keep the next stage's loads here, ahead of this stage's work:
      // without the fence the compiler sinks them to their first use and
      // the prefetch is lost
      asm volatile("" ::: "memory");
      compute(stage(t), t & 1, rawc);
      if (more) {
        store_a((t + 1) & 1, areg);
#pragma unroll
        for (int x = 0; x < SH; ++x)
#pragma unroll
          for (int j = 0; j < NT; ++j) rawc[x][j] = rawn[x][j];
      }
      __syncthreads();
    }
  } else {
    // three register sets, rotated by unrolling the loop three times: stage
    // t computes from set t % 3 while the sets of t + 1 and t + 2 fill
    Raw raw[3][SH][NT];
    u32x4 areg[3][MTA][SH];
    if (nst > 0) {
      load_a(stage(0), areg[0]);
      load_raw(stage(0), raw[0]);
      store_a(0, areg[0]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (nst > 1) {
      load_a(stage(1), areg[1]);
      load_raw(stage(1), raw[1]);
    }
    __syncthreads();
    auto step = [&](int t, auto cc) {
      constexpr int C = decltype(cc)::value;
      constexpr int C1 = (C + 1) % 3, C2 = (C + 2) % 3;
      if (t + 2 < nst) {
        load_a(stage(t + 2), areg[C2]);
        load_raw(stage(t + 2), raw[C2]);
      }
      asm volatile("" ::: "memory");
      compute(stage(t), t & 1, raw[C]);
      if (t + 1 < nst) store_a((t + 1) & 1, areg[C1]);
      __syncthreads();
    };
    for (int t = 0; t < nst; t += 3) {
      step(t, std::integral_constant<int, 0>{});
      if (t + 1 < nst) step(t + 1, std::integral_constant<int, 1>{});
      if (t + 2 < nst) step(t + 2, std::integral_constant<int, 2>{});
    }
  }
}

// The residual of one lane's 4 consecutive outputs n .. n + 3 of a row r
// (packed f16; zeros past N).  An epilogue loads all of a lane's residuals
// before its first store: Y may be R (in-place residual), so the compiler
// cannot move a residual load above an earlier store, and one load / wait /
// store round trip per output group would serialise the epilogue on memory
// latency.  Every output element belongs to one lane, which reads its
// residual before writing it, so the early loads are exact even in place.
__device__ __forceinline__ uint2 load4_r(const f16* r, int n, int N) {
  if (n + 3 < N && ((N & 3) == 0)) return *(const uint2*)(r + n);
  uint16_t h[4] = {0, 0, 0, 0};
  for (int q = 0; q < 4 && n + q < N; ++q) h[q] = __builtin_bit_cast(uint16_t, r[n + q]);
  return make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
}

// f16 store of one lane's 4 consecutive outputs v + (the residual rr, if
// has_r) of row y at n .. n + 3, each rounded once.
__device__ __forceinline__ void store4_y(f16* y, int n, int N, const floatx4& v, uint2 rr, bool has_r) {
  float o4[4] = {v[0], v[1], v[2], v[3]};
  if (has_r) {
    o4[0] += h2f(rr.x); o4[1] += h2f(rr.x >> 16);
    o4[2] += h2f(rr.y); o4[3] += h2f(rr.y >> 16);
  }
  if (n + 3 < N && ((N & 3) == 0)) {
    uint2 o;
    o.x = (uint32_t)f2h_bits(o4[0]) | ((uint32_t)f2h_bits(o4[1]) << 16);
    o.y = (uint32_t)f2h_bits(o4[2]) | ((uint32_t)f2h_bits(o4[3]) << 16);
    *(uint2*)(y + n) = o;
  } else {
    for (int q = 0; q < 4 && n + q < N; ++q) y[n + q] = (f16)o4[q];
  }
}

// f16 store of one lane's 4 consecutive outputs C[n..n+3] of row y (+ r),
// each rounded once; n + 3 < N and 8-byte alignment when N % 4 == 0.
__device__ __forceinline__ void store4_f16(f16* y, const f16* r, int n,
                                           int N, const floatx4& v) {
  if (n + 3 < N && ((N & 3) == 0)) {
    float o4[4] = {v[0], v[1], v[2], v[3]};
    if (r) {
      const uint2 rr = *(const uint2*)(r + n);
      o4[0] += h2f(rr.x); o4[1] += h2f(rr.x >> 16);
      o4[2] += h2f(rr.y); o4[3] += h2f(rr.y >> 16);
    }
    uint2 o;
    o.x = (uint32_t)f2h_bits(o4[0]) | ((uint32_t)f2h_bits(o4[1]) << 16);
    o.y = (uint32_t)f2h_bits(o4[2]) | ((uint32_t)f2h_bits(o4[3]) << 16);
    *(uint2*)(y + n) = o;
  } else {
    for (int q = 0; q < 4 && n + q < N; ++q) {
      float o = v[q];
      if (r) o += (float)r[n + q];
      y[n + q] = (f16)o;
    }
  }
}

}  // namespace fcg
