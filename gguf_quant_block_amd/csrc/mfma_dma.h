// Matrix-core tile with decoupled loads: loader waves stream the activation
// tile and the raw weight pieces straight into a ring of LDS stages with
// global_load_lds_dwordx4; compute waves only read LDS, decode the weights
// into MFMA operands and run the matrix cores.
//
// OpenVINO PR #39119, section Implementation: every weight value is decoded
// once per workgroup and reused across all the activation rows of the tile,
// with loads and decode double-buffered.  Here the buffering is a ring of
// three stages, so two stages of loads are in flight while one computes, and
// no register holds data in flight.
//
// Workgroup: 640 threads.  Eight compute waves (compute wave c owns weight
// rows 16c .. 16c+15 of the 128-row tile: two compute waves per SIMD, each
// reading every activation operand of the stage, so the LDS reads double
// while each weight is still decoded once; a lone wave issues VALU only about
// every 7 cycles, two per SIMD about every 4) and two loader waves, one for
// the activation tile and one for the weight pieces.  The loaders are the
// workgroup's first waves (dma_role), the oldest in issue arbitration.  A
// stage is half a super-block (128 values of K).
// LDS stage slot:
//   A: BM rows x 16 chunks of 16 B; chunk c of row r sits at position
//      c ^ (r & 15) of the row, so that the 16 rows of an MFMA operand read
//      hit 16 distinct bank groups;
//   W: WP pieces x 128 rows x 16 B (the 16-byte pieces of the half-block
//      that the decode reads: Q5_K header, the two fifth-bit pieces, four
//      code pieces (WP = 7); Q4_K header and four code pieces (WP = 5); Q6_K
//      four QL pieces, two QH pieces, the scales (WP = 7)), then for Q6_K
//      the 4-byte word holding each row's d.
// One barrier per stage: a compute wave reaches it after reading its slot,
// a loader wave after its loads for the next stage have landed.
#pragma once

#include <type_traits>

#include "common.h"
#include "layout.h"
#include "mfma_tile.h"

namespace fcg {

constexpr int DMA_SLOTS = 3;                      // LDS ring depth (stages)
constexpr int DMA_ALOADERS = 1;                   // waves loading the activation tile
constexpr int DMA_CWAVES = 8;                    // compute waves
constexpr int DMA_NTW = 8 / DMA_CWAVES;           // 16-row weight sub-tiles per compute wave
constexpr int DMA_THREADS = 64 * (DMA_CWAVES + DMA_ALOADERS + 1);

template <int QT, int MT>
struct DmaCfg {
  static constexpr int BM = 16 * MT;
  static constexpr int BN = 128;
  static constexpr int WP = QT == QT_Q4K ? 5 : 7;   // weight pieces per row per stage
  static constexpr int A_BYTES = BM * 256;
  static constexpr int W_OFF = A_BYTES;             // the weight pieces within a slot
  static constexpr int W_BYTES = WP * BN * 16 + (QT == QT_Q6K ? BN * 4 : 0);
  static constexpr int SLOT = A_BYTES + W_BYTES;
  static constexpr int LDS = DMA_SLOTS * SLOT;
};

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A compute wave's end-of-stage barrier: its LDS reads of the slot have
// returned (lgkmcnt(0)) before it arrives, since a loader may refill the slot
// as soon as the barrier opens.  (s_waitcnt immediate, gfx9 encoding: vmcnt
// 63, expcnt 7, lgkmcnt 0.)
__device__ __forceinline__ void compute_stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The role of this thread's wave: compute waves 0 .. DMA_CWAVES - 1, then the
// activation loaders, then the weight loader.  Hardware waves 0 ..
// DMA_ALOADERS are the loaders and hardware wave DMA_ALOADERS + 1 + c is
// compute wave c, so that the loaders win issue arbitration (ties go to the
// older wave) and their loads are never held behind the compute waves.
__device__ __forceinline__ int dma_role() {
  return ((int)(threadIdx.x >> 6) + DMA_CWAVES) % (DMA_CWAVES + DMA_ALOADERS + 1);
}

// stage t of the loop -> stage of K (rotated start, wrapping)
__device__ __forceinline__ int dma_stage(int t, int s_begin, int nst, int rot) {
  int u = t + rot;
  if (u >= nst) u -= nst;
  return s_begin + u;
}

// The activation loader (role DMA_CWAVES): the activation tile.  arow(r) points at the activation row
// of tile row r (any valid row for rows past the tile's end).  Only the
// first MTA halves are loaded.
template <int QT, int MT, int MTA, class ARow>
__device__ __forceinline__ void dma_load_a(ARow arow, uint8_t* smem, int s_begin, int s_end,
                                           int rot, int which) {
  using C = DmaCfg<QT, MT>;
  static_assert((4 * MTA) % DMA_ALOADERS == 0 || 4 * MTA < DMA_ALOADERS, "split");
  constexpr int NI = (4 * MTA + DMA_ALOADERS - 1) / DMA_ALOADERS;   // instructions per stage
  const int lane = threadIdx.x & 63;
  const int nst = s_end - s_begin;
  const int k0 = which * NI;                        // this wave's first instruction
  const f16* rp[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    const int kk = k0 + k < 4 * MTA ? k0 + k : 4 * MTA - 1;
    rp[k] = arow(4 * kk + (lane >> 4));
  }
  auto issue = [&](int t) {
    const int s = dma_stage(t, s_begin, nst, rot);
    uint8_t* base = smem + (t % DMA_SLOTS) * C::SLOT;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int kk = k0 + k < 4 * MTA ? k0 + k : 4 * MTA - 1;   // (a duplicate is harmless)
      const int r = 4 * kk + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      dma16(rp[k] + (size_t)s * KSTAGE + 8 * c, base + 1024 * kk);
    }
  };
  constexpr int AHEAD = DMA_SLOTS - 1;              // stages in flight beyond the current one
  for (int t = 0; t < AHEAD && t < nst; ++t) issue(t);
  // stage 0 landed: at most the later prologue stages still in flight
  if (nst >= AHEAD) wait_vmcnt<NI * (AHEAD - 1)>(); else wait_vmcnt<0>();
  stage_barrier();
  for (int t = 0; t < nst; ++t) {
    if (t + AHEAD < nst) { issue(t + AHEAD); wait_vmcnt<NI * (AHEAD - 1)>(); }
    else if (t + AHEAD - 1 < nst && AHEAD > 1) { wait_vmcnt<NI * (AHEAD - 2)>(); }
    else { wait_vmcnt<0>(); }
    stage_barrier();
  }
}

// The weight loader (role DMA_CWAVES + 1): the weight pieces of the tile's 128 rows (rows past N are
// clamped to N - 1: loaded, never stored).  In the tiled layout each piece
// load of the wave is four contiguous 256-byte runs (16 rows each).
// C: the slot layout (SLOT bytes per slot, the pieces at W_OFF, WP of them).
template <int QT, int MT, class C = DmaCfg<QT, MT>>
__device__ __forceinline__ void dma_load_w(const uint8_t* W, int N, int K, int n0, uint8_t* smem,
                                           int s_begin, int s_end, int rot) {
  constexpr int NI = 2 * C::WP + (QT == QT_Q6K ? 2 : 0);
  const int lane = threadIdx.x & 63;
  const int nst = s_end - s_begin;
  const WMap L(N, K);
  int rn[2];                                        // the lane's two rows
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = n0 + 64 * h + lane;
    rn[h] = n < N ? n : N - 1;
  }
  auto issue = [&](int t) {
    const int s = dma_stage(t, s_begin, nst, rot);
    const int kb = s >> 1, hb = s & 1;
    uint8_t* base = smem + (t % DMA_SLOTS) * C::SLOT + C::W_OFF;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = rn[h];
#pragma unroll
      for (int q = 0; q < C::WP; ++q) {
        size_t off;
        if constexpr (QT == QT_Q5K) {
          off = L.piece(n, kb, 11, q < 3 ? q : q + 4 * hb);
        } else if constexpr (QT == QT_Q4K) {
          off = L.piece(n, kb, 9, q < 1 ? q : q + 4 * hb);
        } else {
          if (q < 4) off = L.piece(n, kb, 8, 4 * hb + q);
          else if (q < 6) off = L.qh_base() + L.piece(n, kb, 4, 2 * hb + (q - 4));
          else off = L.sc(n, kb);
        }
        dma16(W + off, base + (q * 128 + 64 * h) * 16);
      }
      // the aligned word holding this row's d (and a neighbour's)
      if constexpr (QT == QT_Q6K)
        dma4(W + (L.d(n, kb) & ~(size_t)3), base + C::WP * 128 * 16 + 64 * h * 4);
    }
  };
  constexpr int AHEAD = DMA_SLOTS - 1;
  for (int t = 0; t < AHEAD && t < nst; ++t) issue(t);
  if (nst >= AHEAD) wait_vmcnt<NI * (AHEAD - 1)>(); else wait_vmcnt<0>();
  stage_barrier();
  for (int t = 0; t < nst; ++t) {
    if (t + AHEAD < nst) { issue(t + AHEAD); wait_vmcnt<NI * (AHEAD - 1)>(); }
    else if (t + AHEAD - 1 < nst && AHEAD > 1) { wait_vmcnt<NI * (AHEAD - 2)>(); }
    else { wait_vmcnt<0>(); }
    stage_barrier();
  }
}

// The half-block decoder of a weight type.
template <int QT> struct HalfDec { using type = Q6Half; };
template <> struct HalfDec<QT_Q5K> { using type = Q45Half<true>; };
template <> struct HalfDec<QT_Q4K> { using type = Q45Half<false>; };

// Per-half setup of the lane's decoders for stage s.  Pointers into the
// stage's slot: W0 the lane's row (weight sub-tile 0) in piece 0, W1 that row
// plus the lane's sub-block within a piece (k-quarter kq: piece pair kq / 2,
// half kq & 1), W2 the aligned Q6_K d word of that row.  Sub-tile j lies 16
// rows further on.
template <int QT, int MT>
__device__ __forceinline__ void dma_dec_init(typename HalfDec<QT>::type (&h)[DMA_NTW],
                                             const uint8_t* W0, const uint8_t* W1,
                                             const uint8_t* W2, const int (&rn)[DMA_NTW], int s,
                                             int kq) {
  using C = DmaCfg<QT, MT>;
  constexpr int PB = C::BN * 16;                    // bytes of one piece over the tile's rows
  const int hb = s & 1;
#pragma unroll
  for (int j = 0; j < DMA_NTW; ++j) {
    const uint8_t* p0 = W0 + 256 * j;
    const uint8_t* p1 = W1 + 256 * j;
    if constexpr (QT == QT_Q5K) {
      h[j].init(*(const uint4*)p0, *(const uint2*)(p1 + 3 * PB), *(const uint2*)(p1 + 5 * PB),
                *(const uint2*)(p1 + PB), hb);
    } else if constexpr (QT == QT_Q4K) {
      h[j].init(*(const uint4*)p0, *(const uint2*)(p1 + PB), *(const uint2*)(p1 + 3 * PB),
                uint2{0u, 0u}, hb);
    } else {
      const uint32_t dw = *(const uint32_t*)(W2 + 64 * j);
      // the row's half of the word: the blocks of rows n and n ^ 1 share it
      const int half = rn[j] & 1;
      h[j].init(*(const uint2*)p1, *(const uint2*)(p1 + 2 * PB), *(const uint2*)(p1 + 4 * PB),
                *(const uint2*)(p0 + 6 * PB + 8 * hb), dw >> (16 * half), kq);
    }
  }
}

// Compute waves: acc[i][j] += C[n][m] of the 16x16 sub-tiles (half i < MTA,
// weight sub-tile j of the wave's 16 NTW rows) over the stages.  Wave w owns
// weight rows 16 NTW w .. 16 NTW (w + 1) - 1.
//
// Software pipeline, one k-step deep: while the matrix cores run the MFMAs
// of k-step g, the wave reads the activation operands of its next k-step and
// decodes that k-step's weight fragments (the VALU work overlaps the matrix
// cores).  The stage barrier sits before the last k-step of the stage, once
// the wave has read everything it needs from the slot; right after it,
// the next stage's raw pieces and first operands are read and its decoders
// set up, still under those MFMAs.  (After the last stage the same reads hit
// a slot whose contents are never used.)  Each k-step is one scheduling
// region: its LDS reads first, then each MFMA followed by a few VALU
// instructions.
template <int QT, int MT, int MTA>
__device__ __forceinline__ void dma_compute(int N, int K, int n0, const uint8_t* smem, int s_begin,
                                            int s_end, int rot, floatx4 (&acc)[MT][DMA_NTW]) {
  constexpr int NTW = DMA_NTW, KS = 4;        // k-steps per stage
  using C = DmaCfg<QT, MT>;
  using Dec = typename HalfDec<QT>::type;
  const int lane = threadIdx.x & 63, wn = dma_role();
  const int kq = lane >> 4;
  const int nst = s_end - s_begin;
  int nloc[NTW], rn[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    nloc[j] = wn * 16 * NTW + 16 * j + (lane & 15);
    const int n = n0 + nloc[j];
    rn[j] = n < N ? n : N - 1;                      // the row the loader fetched
  }
#pragma unroll
  for (int i = 0; i < MTA; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (nst <= 0) {
    stage_barrier();
    return;
  }
  // The lane's LDS read offsets within a slot, the same for every stage:
  // la[g] the activation operand of k-step g for row half 0 (row half i is
  // 4096 i further on), lw0 / lw1 / lw2 the weight pointers of
  // dma_dec_init.  The empty asm hides how they were made, so that each
  // address in the loop is one add of the slot's offset (the compiler
  // otherwise rebuilds every address from the stage index, at two VALU
  // instructions apiece).
  uint32_t la[KS];
  const int l15 = lane & 15;
#pragma unroll
  for (int g = 0; g < KS; ++g) {
    la[g] = (16 * l15 + ((4 * g + kq) ^ l15)) * 16;
    asm("" : "+v"(la[g]));
  }
  uint32_t lw0 = C::A_BYTES + 16 * nloc[0];
  uint32_t lw1 = lw0 + C::BN * 16 * (kq >> 1) + 8 * (kq & 1);
  uint32_t lw2 = C::A_BYTES + C::WP * C::BN * 16 + 4 * nloc[0];
  asm("" : "+v"(lw0));
  asm("" : "+v"(lw1));
  asm("" : "+v"(lw2));
  // activation operands of k-step g of the stage in slot As
  auto lda = [&](const uint8_t* As, int g, half8v* af) {
#pragma unroll
    for (int i = 0; i < MTA; ++i) af[i] = *(const half8v*)(As + la[g] + 4096 * i);
  };
  auto dec_init = [&](Dec (&hh)[NTW], const uint8_t* Ss, int t) {
    dma_dec_init<QT, MT>(hh, Ss + lw0, Ss + lw1, Ss + lw2, rn,
                             dma_stage(t, s_begin, nst, rot), kq);
  };

  stage_barrier();                                  // stage 0 has landed
  Dec h[NTW];
  half8v wc[NTW], afc[MTA];
  lda(smem, 0, afc);
  dec_init(h, smem, 0);
#pragma unroll
  for (int j = 0; j < NTW; ++j) wc[j] = h[j].frag(0);

  for (int t = 0; t < nst; ++t) {
    // the slot offsets, hidden likewise (the compiler would split t % 3
    // into two running sums and apply each to every address)
    uint32_t so = (t % DMA_SLOTS) * C::SLOT, sn = ((t + 1) % DMA_SLOTS) * C::SLOT;
    asm("" : "+s"(so));
    asm("" : "+s"(sn));
    const uint8_t* As = smem + so;
#pragma unroll
    for (int gg = 0; gg < KS; ++gg) {
      half8v wnext[NTW], afn[MTA];
      if (gg + 1 < KS) {
        lda(As, gg + 1, afn);
#pragma unroll
        for (int j = 0; j < NTW; ++j) wnext[j] = h[j].frag(gg + 1);
      } else {
        compute_stage_barrier();                    // slot t read; stage t + 1 landed
        const uint8_t* An = smem + sn;
        lda(An, 0, afn);
        dec_init(h, An, t + 1);
#pragma unroll
        for (int j = 0; j < NTW; ++j) wnext[j] = h[j].frag(0);
      }
#pragma unroll
      for (int i = 0; i < MTA; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wc[j], afc[i], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NTW; ++j) wc[j] = wnext[j];
#pragma unroll
      for (int i = 0; i < MTA; ++i) afc[i] = afn[i];
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
      for (int k = 0; k < MTA * NTW; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (gg + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        else __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

}  // namespace fcg
