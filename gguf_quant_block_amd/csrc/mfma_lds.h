// Decode-once prefill tile: producer waves decode each weight block once
// into an f16 tile in LDS, consumer waves run the matrix cores on
// register-blocked 64 x 64 wave tiles read from LDS.
//
// OpenVINO PR #39119, section Implementation: the prefill kernel decodes each
// 256-value weight block into on-chip (local) memory once, double-buffered,
// and reuses it across the activation rows of the tile.  Here the work is
// split over specialised waves of one workgroup, so that the decode (vector
// ALU) and the matrix-core work come from different waves of a SIMD and run
// at the same time:
//   * one loader wave streams the activation tile into a ring of LDS slots
//     with global_load_lds_dwordx4 (LT_AHEAD stages ahead of the consumers);
//   * four producer waves each own 32 of the tile's 128 weight rows: they
//     load their rows' raw super-blocks straight into registers one block
//     ahead, decode a stage exactly to f16 (byte-permute magic numbers, packed
//     f16 FMAs) and write it to a ring of decoded-weight slots, two stages
//     ahead of the consumers;
//   * four consumer waves each own a 64 x 64 block of the 128 x 128 output
//     tile and run v_mfma_f32_32x32x16_f16 on it (16 instructions per stage),
//     reading the operands of the next 16-value k-step while the current
//     k-step's instructions run.
// A stage is 64 values of K (a quarter super-block).  One workgroup barrier
// per stage keeps the three roles in step; every wave passes exactly
// nst + 2 barriers (the last one hands the consumers' partial sums over).
// Workgroups that share activation rows walk K from different super-blocks
// (rot), so that all but one of them find each activation stage in the L2
// another has already fetched, instead of all missing on it together.
//
// LDS slot layout (activation and decoded weight slots alike): one row of a
// stage is 64 halves = 128 bytes = 8 chunks of 16 bytes; chunk c of row r is
// stored at position c ^ f(r) of the row, f(r) = (r & 7) ^ ((r >> 3) & 1), so
// that the 16-byte operand reads of 16 consecutive rows (one chunk each) hit
// 16 distinct 16-byte bank groups of a 256-byte bank window, and those of any
// 8 consecutive rows 8 distinct groups of a 128-byte window.
#pragma once

#include "common.h"
#include "layout.h"
#include "mfma_dma.h"
#include "mfma_tile.h"

namespace fcg {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int LT_BM = 128;                // activation rows per tile
constexpr int LT_BN = 128;                // weight rows per tile
constexpr int LT_KS = 64;                 // values of K per stage
constexpr int LT_AHEAD = 4;               // activation stages in flight ahead of the consumers
constexpr int LT_ASLOTS = LT_AHEAD + 1;
constexpr int LT_WSLOTS = 3;
constexpr int LT_ROWB = LT_KS * 2;        // bytes of one row of a stage
constexpr int LT_A_SLOT = LT_BM * LT_ROWB;
constexpr int LT_W_SLOT = LT_BN * LT_ROWB;
constexpr int LT_W_OFF = LT_ASLOTS * LT_A_SLOT;
constexpr int LT_LDS = LT_W_OFF + LT_WSLOTS * LT_W_SLOT;   // 128 KB
constexpr int LT_NI = LT_A_SLOT / 1024;   // activation load instructions per stage
constexpr int LT_WAVES = 13;              // 1 loader, 4 producers, 8 consumers
constexpr int LT_THREADS = 64 * LT_WAVES;

__device__ __forceinline__ int lt_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// byte offset of chunk c of row r within a slot
__device__ __forceinline__ int lt_off(int r, int c) { return r * LT_ROWB + 16 * (c ^ lt_swz(r)); }

// s_waitcnt vmcnt for a run-time count of outstanding stages of NI loads
template <int NI>
__device__ __forceinline__ void lt_wait_stages(int k) {
  switch (k) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<NI>(); break;
    case 2: wait_vmcnt<2 * NI>(); break;
    default: wait_vmcnt<3 * NI>(); break;
  }
}

// ---------------------------------------------------------------- loader --
// The activation tile of stage s: BM rows x 64 values, 16 instructions of
// 1 KB (8 rows each).  Lane l of instruction i fills position l & 7 of row
// 8i + (l >> 3), i.e. chunk (l & 7) ^ f(row) of that row.  Rows past M are
// clamped to M - 1 (loaded, never stored).
__device__ __forceinline__ void lt_loader(const f16* A, int M, int K, int m0, int k0,
                                          uint8_t* smem, int nst, int rot) {
  static_assert(LT_AHEAD - 2 <= 3, "lt_wait_stages covers up to 3 stages");
  const int lane = threadIdx.x & 63;
  const f16* rp[LT_NI];
#pragma unroll
  for (int i = 0; i < LT_NI; ++i) {
    const int r = 8 * i + (lane >> 3);
    int m = m0 + r;
    m = m < M ? m : M - 1;
    rp[i] = A + (size_t)m * K + k0 + 8 * ((lane & 7) ^ lt_swz(r));
  }
  // loop stage s holds K stage (s + rot) mod nst of the split
  auto issue = [&](int s) {
    uint8_t* base = smem + (s % LT_ASLOTS) * LT_A_SLOT;
    int ks = s + rot;
    ks = ks < nst ? ks : ks - nst;
#pragma unroll
    for (int i = 0; i < LT_NI; ++i) dma16(rp[i] + (size_t)ks * LT_KS, base + 1024 * i);
  };
  const int pro = nst < LT_AHEAD ? nst : LT_AHEAD;
  for (int s = 0; s < pro; ++s) issue(s);
  // stages 0 and 1 landed before the first barrier
  lt_wait_stages<LT_NI>(pro > 2 ? pro - 2 : 0);
  stage_barrier();
  for (int t = 0; t < nst; ++t) {
    if (t + LT_AHEAD < nst) issue(t + LT_AHEAD);
    // stage t + 2 landed before barrier t (the consumers read its first
    // operands during iteration t + 1); later stages may stay in flight
    const int last = (t + LT_AHEAD < nst ? t + LT_AHEAD : nst - 1);
    const int after = last - (t + 2);
    lt_wait_stages<LT_NI>(after > 0 ? after : 0);
    stage_barrier();
  }
}

// -------------------------------------------------------------- producers --
// Raw bytes of one super-block of the lane's row.  Lane l of producer wave p
// owns row 32p + (l & 31) of the tile and half h = l >> 5 of every 32-value
// run: Q4_K / Q5_K positions 16h .. 16h + 15 of each sub-block, Q6_K
// positions 16h .. 16h + 15 of each 32-value group.
template <int QT> struct LtRaw;
template <> struct LtRaw<QT_Q5K> {       // header, qh[16h ..], qs[32c + 16h ..] for c = 0..3
  uint4 hdr, qh, qs[4];
};
template <> struct LtRaw<QT_Q4K> {       // header, qs[32c + 16h ..] for c = 0..3
  uint4 hdr, qs[4];
};
template <> struct LtRaw<QT_Q6K> {       // ql[64j + 16h ..], ql[64j + 32 + 16h ..], qh[32j + 16h ..]
  uint4 qlA[2], qlB[2], qh[2], sc;       // for j = 0, 1; all 16 scales; d bits
  uint32_t d;
};

template <int QT>
__device__ __forceinline__ void lt_load_raw(const uint8_t* W, const WMap& L, int n, int kb, int h,
                                            LtRaw<QT>& r) {
  if constexpr (QT == QT_Q5K) {
    r.hdr = *(const uint4*)(W + L.piece(n, kb, 11, 0));
    r.qh = *(const uint4*)(W + L.piece(n, kb, 11, 1 + h));
#pragma unroll
    for (int c = 0; c < 4; ++c) r.qs[c] = *(const uint4*)(W + L.piece(n, kb, 11, 3 + 2 * c + h));
  } else if constexpr (QT == QT_Q4K) {
    r.hdr = *(const uint4*)(W + L.piece(n, kb, 9, 0));
#pragma unroll
    for (int c = 0; c < 4; ++c) r.qs[c] = *(const uint4*)(W + L.piece(n, kb, 9, 1 + 2 * c + h));
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      r.qlA[j] = *(const uint4*)(W + L.piece(n, kb, 8, 4 * j + h));
      r.qlB[j] = *(const uint4*)(W + L.piece(n, kb, 8, 4 * j + 2 + h));
      r.qh[j] = *(const uint4*)(W + L.qh_base() + L.piece(n, kb, 4, 2 * j + h));
    }
    r.sc = *(const uint4*)(W + L.sc(n, kb));
    r.d = *(const uint16_t*)(W + L.d(n, kb));
  }
}

template <int QT> constexpr int lt_raw_loads() { return QT == QT_Q5K ? 6 : (QT == QT_Q4K ? 5 : 8); }

// bit j of every byte of x moved to bit 4 (j = 0..7)
template <int J>
__device__ __forceinline__ uint32_t bit_to4(uint32_t x) {
  if constexpr (J <= 4) return (x << (4 - J)) & 0x10101010u;
  else return (x >> (J - 4)) & 0x10101010u;
}
// bits 2g, 2g + 1 of every byte of x moved to bits 4, 5 (g = 0..3)
template <int G>
__device__ __forceinline__ uint32_t pair_to45(uint32_t x) {
  if constexpr (2 * G <= 4) return (x << (4 - 2 * G)) & 0x30303030u;
  else return (x >> (2 * G - 4)) & 0x30303030u;
}

__device__ __forceinline__ uint32_t u4w(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Decode quarter C (values 64C .. 64C + 63) of the lane's super-block into
// out[0..3]: the lane's 8-value chunks 2h, 2h + 1 (first 32-value run) and
// 4 + 2h, 5 + 2h (second run) of the stage.  Exact up to the f16 rounding
// of the weight (Q4_K / Q5_K: (1024 + q) * sc - 1024 * sc = sc * q exactly,
// then one fma with d and the rounded -dmin * m; Q6_K: ((1024 + q) - 1056) *
// (sc * d), sc * d rounded once).
template <int QT, int C>
__device__ __forceinline__ void lt_decode(const LtRaw<QT>& r, int h, half8v (&out)[4]) {
  if constexpr (QT == QT_Q5K || QT == QT_Q4K) {
    const uint32_t w0 = r.hdr.y, w1 = r.hdr.z, w2 = r.hdr.w;
    // scale / min bytes of sub-blocks 2C, 2C + 1 (bytes 2(C%2), 2(C%2)+1 of
    // the 4-byte group of sub-blocks 0..3 or 4..7)
    uint32_t scb, mb;
    if constexpr (C < 2) {
      scb = w0 & 0x3F3F3F3Fu;
      mb = w1 & 0x3F3F3F3Fu;
    } else {
      scb = (w2 & 0x0F0F0F0Fu) | ((w0 >> 2) & 0x30303030u);
      mb = ((w2 >> 4) & 0x0F0F0F0Fu) | ((w1 >> 2) & 0x30303030u);
    }
    constexpr uint32_t sel = (C & 1) ? 0x04030402u : 0x04010400u;
    const half2v k1024 = splat((f16)1024.f);
    const half2v sc = magic_pair(scb, sel) - k1024;                 // (sc_2C, sc_2C+1), exact
    const half2v bias = sc * splat((f16)-1024.f);                   // exact
    const half2v ndmin = splat(-__builtin_bit_cast(f16, (uint16_t)(r.hdr.x >> 16)));
    const half2v nm = (magic_pair(mb, sel) - k1024) * ndmin;        // -dmin * m, rounded once
    const half2v d2 = splat(__builtin_bit_cast(f16, (uint16_t)(r.hdr.x & 0xFFFF)));
    const uint4 qs = r.qs[C];
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t q = u4w(qs, w);
      lo[w] = q & 0x0F0F0F0Fu;
      hi[w] = (q >> 4) & 0x0F0F0F0Fu;
      if constexpr (QT == QT_Q5K) {
        const uint32_t b = u4w(r.qh, w);
        lo[w] |= bit_to4<2 * C>(b);
        hi[w] |= bit_to4<2 * C + 1>(b);
      }
    }
    out[0] = decode8(lo[0], lo[1], splat(sc[0]), splat(bias[0]), d2, splat(nm[0]));
    out[1] = decode8(lo[2], lo[3], splat(sc[0]), splat(bias[0]), d2, splat(nm[0]));
    out[2] = decode8(hi[0], hi[1], splat(sc[1]), splat(bias[1]), d2, splat(nm[1]));
    out[3] = decode8(hi[2], hi[3], splat(sc[1]), splat(bias[1]), d2, splat(nm[1]));
  } else {
    constexpr int J = C >> 1, NIB = C & 1;       // 128-value half, nibble
    constexpr int G0 = 2 * NIB, G1 = G0 + 1;     // the stage's two 32-value groups
    // scales of the lane's 16-value runs: sub-blocks 8J + 2G + h
    const uint32_t sw = u4w(r.sc, (8 * J + 2 * G0) >> 2);   // bytes 2G0 .. 2G0+3 of the half
    const uint32_t s0 = (sw >> (8 * (((2 * G0) & 3) + h))) & 0xFFu;
    const uint32_t s1 = (sw >> (8 * (((2 * G1) & 3) + h))) & 0xFFu;
    // signed byte -> f16 via the magic (1024 + (b ^ 0x80)) - 1152
    const uint32_t sb = ((s0 | (s1 << 16)) ^ 0x00800080u) | 0x64006400u;
    const half2v d2 = splat(__builtin_bit_cast(f16, (uint16_t)(r.d & 0xFFFF)));
    const half2v scd = (__builtin_bit_cast(half2v, sb) - splat((f16)1152.f)) * d2;
    const uint4 qa = r.qlA[J], qb = r.qlB[J], qh = r.qh[J];
    uint32_t c0[4], c1[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t hb = u4w(qh, w);
      c0[w] = ((u4w(qa, w) >> (4 * NIB)) & 0x0F0F0F0Fu) | pair_to45<G0>(hb);
      c1[w] = ((u4w(qb, w) >> (4 * NIB)) & 0x0F0F0F0Fu) | pair_to45<G1>(hb);
    }
    const half2v k1056 = splat((f16)1056.f);
    auto dec = [&](uint32_t x0, uint32_t x1, f16 s) {
      const half2v sc2 = splat(s);
      const half2v p0 = (magic_pair(x0, 0x04010400u) - k1056) * sc2;
      const half2v p1 = (magic_pair(x0, 0x04030402u) - k1056) * sc2;
      const half2v p2 = (magic_pair(x1, 0x04010400u) - k1056) * sc2;
      const half2v p3 = (magic_pair(x1, 0x04030402u) - k1056) * sc2;
      return make_frag(p0, p1, p2, p3);
    };
    out[0] = dec(c0[0], c0[1], scd[0]);
    out[1] = dec(c0[2], c0[3], scd[0]);
    out[2] = dec(c1[0], c1[1], scd[1]);
    out[3] = dec(c1[2], c1[3], scd[1]);
  }
}

// Producer wave p: rows 32p .. 32p + 31 of the tile, super-blocks
// kb0 .. kb0 + nst/4 - 1.  Decodes stage u into decoded slot u % 3; passes
// barrier u - 2 after writing stage u (u >= 1), then the last two.
template <int QT>
__device__ __forceinline__ void lt_producer(const uint8_t* W, int N, int K, int n0, int kb0,
                                            uint8_t* smem, int nst, int rot, int p) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, rl = 32 * p + (lane & 31);
  int n = n0 + rl;
  n = n < N ? n : N - 1;
  const WMap L(N, K);
  uint8_t* wbase = smem + LT_W_OFF;
  const int o0 = lt_off(rl, 2 * h), o1 = lt_off(rl, 2 * h + 1);
  const int o2 = lt_off(rl, 4 + 2 * h), o3 = lt_off(rl, 5 + 2 * h);
  const int nsb = nst >> 2, rsb = rot >> 2;
  // loop super-block b holds super-block (b + rot / 4) mod nsb of the split
  auto kb_of = [&](int b) {
    int x = b + rsb;
    return kb0 + (x < nsb ? x : x - nsb);
  };
  // raw super-blocks in registers: the one being decoded and the next one
  // in flight
  LtRaw<QT> cur, nxt;
  lt_load_raw<QT>(W, L, n, kb_of(0), h, cur);
  if (nsb > 1) {
    lt_load_raw<QT>(W, L, n, kb_of(1), h, nxt);
    wait_vmcnt<lt_raw_loads<QT>()>();
  } else {
    wait_vmcnt<0>();
  }
  auto stage = [&](auto cc, int u) {
    constexpr int C = decltype(cc)::value;
    half8v o[4];
    lt_decode<QT, C>(cur, h, o);
    uint8_t* s = wbase + (u % LT_WSLOTS) * LT_W_SLOT;
    *(half8v*)(s + o0) = o[0];
    *(half8v*)(s + o1) = o[1];
    *(half8v*)(s + o2) = o[2];
    *(half8v*)(s + o3) = o[3];
    if (u >= 1) compute_stage_barrier();            // LDS writes done, then barrier u - 2
  };
  for (int sb = 0; sb < nsb; ++sb) {
    if (sb > 0) {
      wait_vmcnt<0>();
      cur = nxt;
      if (sb + 1 < nsb) lt_load_raw<QT>(W, L, n, kb_of(sb + 1), h, nxt);
    }
    stage(std::integral_constant<int, 0>{}, 4 * sb);
    stage(std::integral_constant<int, 1>{}, 4 * sb + 1);
    stage(std::integral_constant<int, 2>{}, 4 * sb + 2);
    stage(std::integral_constant<int, 3>{}, 4 * sb + 3);
  }
  stage_barrier();                                  // barriers nst - 2, nst - 1
  stage_barrier();
}

// -------------------------------------------------------------- consumers --
// Consumer wave c (0..7) works on output block c & 3: activation rows
// 64 (c & 1) .. + 63 and weight rows 64 ((c >> 1) & 1) .. + 63 of the tile,
// on the k-steps s = q, q + 2 of every stage (q = c >> 2): the two consumers
// of a block share a SIMD and its matrix core, and split the operand reads,
// since one wave sustains only about one 16-byte-per-lane LDS read every
// 32 cycles.  acc[a][b] holds the 32 x 32 block of weight rows 32a and
// activation rows 32b: lane l, register v holds
// C[n = 8 (v / 4) + 4 (l / 32) + v % 4][m = l % 32].
__device__ __forceinline__ void lt_consumer(const uint8_t* smem, int nst, int c,
                                            floatx16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63;
  const int q = c >> 2, wm = c & 1, wn = (c >> 1) & 1;
  const int hl = lane >> 5;
  const int fl = lt_swz(lane & 15);
  const int rowoff = (lane & 31) * LT_ROWB;
  // the lane's chunk of k-steps q and q + 2, swizzled
  int koff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    koff[i] = rowoff + 16 * ((2 * (q + 2 * i) + hl) ^ fl);
    asm("" : "+v"(koff[i]));
  }
  const int aoff = 64 * wm * LT_ROWB, woff = LT_W_OFF + 64 * wn * LT_ROWB;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  // operands of the wave's k-step i (0, 1) of stage t
  auto load = [&](int t, int i, half8v (&f)[4]) {
    const uint8_t* As = smem + (t % LT_ASLOTS) * LT_A_SLOT + aoff + koff[i];
    const uint8_t* Ws = smem + (t % LT_WSLOTS) * LT_W_SLOT + woff + koff[i];
    f[0] = *(const half8v*)(Ws);
    f[1] = *(const half8v*)(Ws + 32 * LT_ROWB);
    f[2] = *(const half8v*)(As);
    f[3] = *(const half8v*)(As + 32 * LT_ROWB);
  };
  auto mfma4 = [&](const half8v (&f)[4]) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f[a], f[2 + b], acc[a][b], 0, 0, 0);
  };
  // The reads run two of the wave's k-steps (one stage) ahead of its MFMAs:
  // k-step j = 2t + i of the wave (stage t, its i-th k-step) computes from
  // buffer j % 3, filled while k-steps j - 2 and j - 1 ran.  The next
  // stage's operands are read during this one (its slots were complete at
  // the previous barrier).  The reads are unconditional (past the last stage
  // they read slots whose contents are never used), so that the compiler's
  // wait counts stay exact: a branch around them would make it wait for
  // every outstanding read before each k-step.
  stage_barrier();                                  // barrier -1: stages 0, 1 ready
  half8v f[3][4];
  load(0, 0, f[0]);
  load(0, 1, f[1]);
  auto step = [&](int t, int i, auto jj) {
    constexpr int J = decltype(jj)::value;          // k-step index mod 3
    load(t + 1, i, f[(J + 2) % 3]);
    mfma4(f[J]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // three stages per trip (six k-steps), so that the buffer of every k-step
  // is known at compile time
  for (int t = 0; t < nst; t += 3) {
    step(t, 0, std::integral_constant<int, 0>{});
    step(t, 1, std::integral_constant<int, 1>{});
    stage_barrier();                                // barrier t
    if (t + 1 >= nst) break;
    step(t + 1, 0, std::integral_constant<int, 2>{});
    step(t + 1, 1, std::integral_constant<int, 0>{});
    stage_barrier();                                // barrier t + 1
    if (t + 2 >= nst) break;
    step(t + 2, 0, std::integral_constant<int, 1>{});
    step(t + 2, 1, std::integral_constant<int, 2>{});
    stage_barrier();                                // barrier t + 2
  }
}

// After the last stage: consumers 4..7 hand their partial sums to consumers
// 0..3 through LDS (the activation slots, free by then), which add them in
// that fixed order.  Every wave of the workgroup passes this barrier.
__device__ __forceinline__ void lt_pair_sum(uint8_t* smem, int c, floatx16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63;
  float* part = (float*)smem + (c & 3) * (64 * 64) + lane;
  if (c >= 4) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) part[64 * (16 * (2 * a + b) + v)] = acc[a][b][v];
  }
  compute_stage_barrier();
  if (c < 4) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][b][v] += part[64 * (16 * (2 * a + b) + v)];
  }
}

}  // namespace fcg
