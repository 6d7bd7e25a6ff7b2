// Decode path (M < 8, and f32 activations): per-32 int8 activation
// quantisation fused into an int8 GEMV that streams the raw Q4_K / Q5_K /
// Q6_K blocks once.
//
// OpenVINO PR #39119, section Implementation: the GEMV quantises the
// activations per 32 values and takes int8 dot products directly against the
// blocks; the residual Add is fused into the output store.
//
// Work layout (one launch):
//   * A workgroup owns one row tile of the device layout (layout.h): 16
//     weight rows over all of K.  It has nw = min(KBp/4, 8) waves; wave w
//     takes the 16 x 4-block tiles w, w + nw, ... of the row tile, one block
//     per lane (lane = (kb % 4) * 16 + row % 16), so every 16-byte piece load
//     of the wave is one contiguous kilobyte.
//   * Every thread first issues the activation loads of its quantisation
//     groups, then its block's weight loads, then quantises (waiting only
//     for the activation loads, which complete first) into LDS: int8 codes
//     and a per-(row, block) record of the f32 group scales s and the code
//     sums the scale algebra needs (Q4_K, Q5_K: s*T per 32-group for the min
//     term; Q6_K: 16-value sums for the -32 offset).  The weights arrive
//     meanwhile.
//   * After the barrier each lane decodes its block with compile-time field
//     offsets, takes v_dot4_i32_i8 integer sums per sub-block and applies the
//     scales in f32.  The lanes of a wave read the activations of only four
//     blocks at a time (one per kb % 4), so the LDS reads are broadcasts.
//   * Row sums in a fixed order: over a lane's tiles, then across the four
//     lanes of a row (butterfly), then across the waves in wave order; R is
//     added and the result is rounded once to the output type.
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "layout.h"
#include "quant.h"

namespace fcg {

constexpr int GEMV_MAX_WAVES = 8;
constexpr int GEMV_MAX_THREADS = 64 * GEMV_MAX_WAVES;

// ------------------------------------------------------ LDS layout ----

template <int QT> struct GemvFmt;
template <> struct GemvFmt<QT_Q5K> {
  static constexpr int REC = 20;           // words per (m, kb) record: s[8], s*T[8], pad[4]
};
template <> struct GemvFmt<QT_Q4K> : GemvFmt<QT_Q5K> {};
template <> struct GemvFmt<QT_Q6K> {
  static constexpr int REC = 28;           // s[8], T16[16], pad[4]
};

struct GemvLayout {
  size_t rec, part, total;
};

// Waves per workgroup (one row tile) for K: one wave per 4-block tile of the
// row tile, at most 8.
__host__ __device__ inline int gemv_waves(int K) {
  const int g = tiled_kb(K / QK) / TILE_KB;
  return g < GEMV_MAX_WAVES ? g : GEMV_MAX_WAVES;
}

// LDS: qa int8 [MR][KBp] records of QA_REC bytes (256 codes + 16 bytes of
// padding, so that the four blocks a wave reads at once start on different
// banks) | rec u32 [MR][KBp][REC] | part f32 [waves][MR][16] (a wave's sums
// for the 16 rows of its row tile).
constexpr int QA_REC = QK + 16;
template <int QT>
__host__ __device__ constexpr GemvLayout gemv_layout(int MR, int KBp, int waves) {
  const size_t rec = (size_t)MR * KBp * QA_REC;
  const size_t part = rec + (size_t)MR * KBp * GemvFmt<QT>::REC * 4;
  const size_t total = part + (size_t)waves * MR * TILE_ROWS * 4;
  return GemvLayout{rec, part, total};
}

// byte offset of the 16-byte code chunk t (0..15) of block kb in row m
__device__ __forceinline__ int qa_chunk(int m, int KBp, int kb, int t) {
  return (m * KBp + kb) * QA_REC + 16 * t;
}

// ------------------------------------------------ activation quantisation --
// Per-32 int8 quantisation of the activations: thread tid takes the 32-value
// groups (tasks) tid, tid + nt, ...
// The activation loads of the first qpre<AT>() rounds are issued before the
// weight loads, so the quantisation waits only for them (loads complete in
// order) while the weights are still in flight.
template <class AT>
constexpr int qpre() { return std::is_same<AT, f16>::value ? 2 : 1; }

template <int QT, int MR, class AT>
__device__ __forceinline__ void quantise_task(int t, int tasks, int K, int KBp, uint4* raw,
                                              uint8_t* smem, uint32_t* rec) {
  constexpr int REC = GemvFmt<QT>::REC;
#pragma unroll
  for (int i = 0; i < act_u4<AT>(); ++i) raw[i] = t < tasks ? raw[i] : make_uint4(0, 0, 0, 0);
  uint32_t q[8];
  float s;
  int tsum, thalf[2];
  quant_group<AT>(raw, q, s, tsum, thalf);
  if (t < tasks) {
    const int e = t * 32;                           // first value (flat over MR x K)
    const int m = e / K, pos = e - m * K;
    const int kb = pos / QK, t16 = (pos % QK) / 16, g = (pos % QK) / 32;
    *(uint4*)(smem + qa_chunk(m, KBp, kb, t16)) = make_uint4(q[0], q[1], q[2], q[3]);
    *(uint4*)(smem + qa_chunk(m, KBp, kb, t16 + 1)) = make_uint4(q[4], q[5], q[6], q[7]);
    uint32_t* r = rec + ((size_t)m * KBp + kb) * REC;
    r[g] = __builtin_bit_cast(uint32_t, s);
    if constexpr (QT != QT_Q6K) {
      r[8 + g] = __builtin_bit_cast(uint32_t, s * (float)tsum);
    } else {
      r[8 + 2 * g] = (uint32_t)thalf[0];
      r[8 + 2 * g + 1] = (uint32_t)thalf[1];
    }
  }
}

template <int MR, class AT>
__device__ __forceinline__ void quant_issue(const AT* A, int K, int tid, int nt,
                                            uint4 (&raw)[qpre<AT>()][act_u4<AT>()]) {
  const int tasks = MR * K / 32;
#pragma unroll
  for (int r = 0; r < qpre<AT>(); ++r) {
    const int t = r * nt + tid;
    const int tc = t < tasks ? t : 0;
#pragma unroll
    for (int i = 0; i < act_u4<AT>(); ++i) raw[r][i] = ((const uint4*)(A + (size_t)tc * 32))[i];
  }
}

template <int QT, int MR, class AT>
__device__ __forceinline__ void quant_finish(const AT* A, int K, int KBp, uint8_t* smem,
                                             uint32_t* rec, int tid, int nt,
                                             uint4 (&raw)[qpre<AT>()][act_u4<AT>()]) {
  constexpr int QP = qpre<AT>(), U4 = act_u4<AT>();
  const int tasks = MR * K / 32;
  const int wbase = tid & ~63;                        // wave-uniform skip of idle waves
#pragma unroll
  for (int r = 0; r < QP; ++r)
    if (r * nt + wbase < tasks)
      quantise_task<QT, MR, AT>(r * nt + tid, tasks, K, KBp, raw[r], smem, rec);
  for (int t0 = QP * nt; t0 < tasks; t0 += nt) {
    if (t0 + wbase >= tasks) break;
    const int t = t0 + tid;
    const int tc = t < tasks ? t : 0;
    uint4 v[U4];
#pragma unroll
    for (int i = 0; i < U4; ++i) v[i] = ((const uint4*)(A + (size_t)tc * 32))[i];
    quantise_task<QT, MR, AT>(t, tasks, K, KBp, v, smem, rec);
  }
}

// ----------------------------------------- codes and integer sub-block sums --
// Q5_K: 176 B = d|dmin, scales[12], qh[32], qs[128] (11 x 16 B).  For the
// sub-block pair (2c, 2c+1): qs[32c + l] low nibble -> value 64c + l, high
// nibble -> 64c + 32 + l; bits 2c / 2c+1 of qh[l] are the fifth bits.
// Q4_K: 144 B = d|dmin, scales[12], qs[128] (9 x 16 B); the same nibbles,
// no fifth bit (mobius GGUF proposal, section 7.3).
// lo[w] / hi[w]: packed codes (0..31 / 0..15) of values 64c + 4w.. /
// 64c + 32 + 4w..
template <int QT, int C>
__device__ __forceinline__ void q45k_codes(const uint32_t* qh, const uint32_t* qs, uint32_t* lo,
                                           uint32_t* hi) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t d = qs[8 * C + w];
    lo[w] = d & 0x0F0F0F0Fu;
    hi[w] = (d >> 4) & 0x0F0F0F0Fu;
    if constexpr (QT == QT_Q5K) {
      const uint32_t h = qh[w];
      lo[w] |= (4 - 2 * C >= 0 ? h << (4 - 2 * C) : h >> (2 * C - 4)) & 0x10101010u;
      hi[w] |= (3 - 2 * C >= 0 ? h << (3 - 2 * C) : h >> (2 * C - 3)) & 0x10101010u;
    }
  }
}

// Q6_K: ql[64h + 32a + l] low nibble -> value 128h + 32a + l (pair 2a of
// qh[32h + l]), high nibble -> value 128h + 32(a+2) + l (pair 2a+4).
// lo[w] / hi[w]: packed codes (0..63) of values 128h+32a+4w.. / +64.
template <int H, int A_>
__device__ __forceinline__ void q6k_codes(const uint32_t* ql, const uint32_t* qh, uint32_t* lo,
                                          uint32_t* hi) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t d = ql[16 * H + 8 * A_ + w], h = qh[8 * H + w];
    lo[w] = (d & 0x0F0F0F0Fu) | ((h << (4 - 2 * A_)) & 0x30303030u);
    hi[w] = ((d >> 4) & 0x0F0F0F0Fu) | ((h >> (2 * A_)) & 0x30303030u);
  }
}

__device__ __forceinline__ int dot16u(const uint32_t* c, uint4 a) {
  int s = dot4((int)c[0], (int)a.x, 0);
  s = dot4((int)c[1], (int)a.y, s);
  s = dot4((int)c[2], (int)a.z, s);
  return dot4((int)c[3], (int)a.w, s);
}

// ------------------------------------------------------- block kernels ----

// Q4_K / Q5_K block -> part[m] (lane's contribution to row m): blk = the
// block's 36 / 44 words.
template <int QT, int MR>
__device__ __forceinline__ void q45k_block(const uint32_t* blk, int kb, int KBp, const uint8_t* smem,
                                           const uint32_t* rec, float* part) {
  const float d = h2f(blk[0]), dmin = h2f(blk[0] >> 16);
  const uint32_t w0 = blk[1], w1 = blk[2], w2 = blk[3];
  // 6-bit scales / mins as bytes: j = 0..3 and j = 4..7
  const uint32_t sc_lo = w0 & 0x3F3F3F3Fu, m_lo = w1 & 0x3F3F3F3Fu;
  const uint32_t sc_hi = (w2 & 0x0F0F0F0Fu) | ((w0 >> 2) & 0x30303030u);
  const uint32_t m_hi = ((w2 >> 4) & 0x0F0F0F0Fu) | ((w1 >> 2) & 0x30303030u);
  const uint32_t* qh = blk + 4;
  const uint32_t* qs = blk + (QT == QT_Q5K ? 12 : 4);
  float X[MR], Z[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) X[m] = Z[m] = 0.f;
  auto pair = [&](auto cc) {
    constexpr int C = decltype(cc)::value;
    uint32_t lo[8], hi[8];
    q45k_codes<QT, C>(qh, qs, lo, hi);
    const uint32_t scw = C < 2 ? sc_lo : sc_hi, mw = C < 2 ? m_lo : m_hi;
    const float sc0 = (float)((scw >> (16 * (C & 1))) & 0xFF), sc1 = (float)((scw >> (16 * (C & 1) + 8)) & 0xFF);
    const float mn0 = (float)((mw >> (16 * (C & 1))) & 0xFF), mn1 = (float)((mw >> (16 * (C & 1) + 8)) & 0xFF);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const uint4 a0 = *(const uint4*)(smem + qa_chunk(m, KBp, kb, 4 * C));
      const uint4 a1 = *(const uint4*)(smem + qa_chunk(m, KBp, kb, 4 * C + 1));
      const uint4 a2 = *(const uint4*)(smem + qa_chunk(m, KBp, kb, 4 * C + 2));
      const uint4 a3 = *(const uint4*)(smem + qa_chunk(m, KBp, kb, 4 * C + 3));
      const int S0 = dot16u(lo, a0) + dot16u(lo + 4, a1);
      const int S1 = dot16u(hi, a2) + dot16u(hi + 4, a3);
      const uint32_t* r = rec + ((size_t)m * KBp + kb) * GemvFmt<QT>::REC;
      const float2 s2 = *(const float2*)(r + 2 * C);
      const float2 t2 = *(const float2*)(r + 8 + 2 * C);
      X[m] = fmaf(sc0, s2.x * (float)S0, X[m]);
      X[m] = fmaf(sc1, s2.y * (float)S1, X[m]);
      Z[m] = fmaf(mn0, t2.x, Z[m]);
      Z[m] = fmaf(mn1, t2.y, Z[m]);
    }
  };
  pair(std::integral_constant<int, 0>{});
  pair(std::integral_constant<int, 1>{});
  pair(std::integral_constant<int, 2>{});
  pair(std::integral_constant<int, 3>{});
#pragma unroll
  for (int m = 0; m < MR; ++m) part[m] += d * X[m] - dmin * Z[m];
}

// Q6_K block -> part[m]: ql (32 words), qh (16 words), sc (4 words), d bits.
template <int MR>
__device__ __forceinline__ void q6k_block(const uint32_t* ql, const uint32_t* qh, uint4 scv,
                                          uint32_t dbits, int kb, int KBp, const uint8_t* smem,
                                          const uint32_t* rec, float* part) {
  const float d = h2f(dbits);
  const uint32_t scw[4] = {scv.x, scv.y, scv.z, scv.w};
  float X[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) X[m] = 0.f;
  auto unit = [&](auto hh, auto aa) {
    constexpr int H = decltype(hh)::value, A_ = decltype(aa)::value;
    uint32_t lo[8], hi[8];
    q6k_codes<H, A_>(ql, qh, lo, hi);
    constexpr int s0 = 8 * H + 2 * A_;           // sub-blocks s0, s0+1 (lo) and s0+4, s0+5 (hi)
    const int c0 = sext8(scw[s0 >> 2] >> (8 * (s0 & 3)));
    const int c1 = sext8(scw[s0 >> 2] >> (8 * ((s0 + 1) & 3)));
    const int c4 = sext8(scw[(s0 + 4) >> 2] >> (8 * ((s0 + 4) & 3)));
    const int c5 = sext8(scw[(s0 + 5) >> 2] >> (8 * ((s0 + 5) & 3)));
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const uint4 a0 = *(const uint4*)(smem + qa_chunk(m, KBp, kb, s0));
      const uint4 a1 = *(const uint4*)(smem + qa_chunk(m, KBp, kb, s0 + 1));
      const uint4 a4 = *(const uint4*)(smem + qa_chunk(m, KBp, kb, s0 + 4));
      const uint4 a5 = *(const uint4*)(smem + qa_chunk(m, KBp, kb, s0 + 5));
      const uint32_t* r = rec + ((size_t)m * KBp + kb) * GemvFmt<QT_Q6K>::REC;
      const int2 tl = *(const int2*)(r + 8 + s0);
      const int2 th = *(const int2*)(r + 8 + s0 + 4);
      const int S0 = dot16u(lo, a0) - 32 * tl.x;
      const int S1 = dot16u(lo + 4, a1) - 32 * tl.y;
      const int S4 = dot16u(hi, a4) - 32 * th.x;
      const int S5 = dot16u(hi + 4, a5) - 32 * th.y;
      const int I = __mul24(c0, S0) + __mul24(c1, S1);
      const int J = __mul24(c4, S4) + __mul24(c5, S5);
      const float sI = __builtin_bit_cast(float, r[s0 >> 1]);
      const float sJ = __builtin_bit_cast(float, r[(s0 + 4) >> 1]);
      X[m] = fmaf(sI, (float)I, X[m]);
      X[m] = fmaf(sJ, (float)J, X[m]);
    }
  };
  unit(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
  unit(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
  unit(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
  unit(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
#pragma unroll
  for (int m = 0; m < MR; ++m) part[m] += d * X[m];
}

// ---------------------------------------------------------------- kernel --

// The lane's whole super-block, straight from global memory into registers
// (Q4_K / Q5_K: its 9 / 11 pieces; Q6_K: its QL, QH, SC and D bytes).  The
// lanes of a wave own the 64 blocks of one tile, so every piece load of the
// wave is one contiguous kilobyte.
struct GemvBlock {
  uint32_t w[48];     // Q4_K / Q5_K: the 144 / 176 bytes in w[0..35] / w[0..43];
                      // Q6_K: ql in w[0..31], qh in w[32..47]
  uint4 scv;          // Q6_K scales
  uint32_t dbits;     // Q6_K d
};

// The loads are issued in the order the block is consumed (header and fifth
// bits / scales first, then the code pieces sub-block by sub-block): loads
// complete in order, so the arithmetic on the first sub-blocks starts while
// the later pieces are still in flight.  The empty asm statements keep the
// compiler from reordering the loads.
#define FCG_KEEP_ORDER() asm volatile("" ::: "memory")

template <int QT>
__device__ __forceinline__ void load_block(const uint8_t* W, const WMap& L, int n, int kb,
                                           GemvBlock& b) {
  if constexpr (QT != QT_Q6K) {
    constexpr int P = block_bytes_of(QT) / 16;
#pragma unroll
    for (int c = 0; c < P; ++c) {
      const uint4 v = *(const uint4*)(W + L.piece(n, kb, P, c));
      b.w[4 * c] = v.x; b.w[4 * c + 1] = v.y; b.w[4 * c + 2] = v.z; b.w[4 * c + 3] = v.w;
      FCG_KEEP_ORDER();
    }
  } else {
    b.scv = *(const uint4*)(W + L.sc(n, kb));
    b.dbits = *(const uint16_t*)(W + L.d(n, kb));
    FCG_KEEP_ORDER();
    const uint8_t* qh = W + L.qh_base();
    auto ql_piece = [&](int f) {
      const uint4 v = *(const uint4*)(W + L.piece(n, kb, 8, f));
      b.w[4 * f] = v.x; b.w[4 * f + 1] = v.y; b.w[4 * f + 2] = v.z; b.w[4 * f + 3] = v.w;
      FCG_KEEP_ORDER();
    };
    auto qh_piece = [&](int f) {
      const uint4 v = *(const uint4*)(qh + L.piece(n, kb, 4, f));
      b.w[32 + 4 * f] = v.x; b.w[33 + 4 * f] = v.y; b.w[34 + 4 * f] = v.z; b.w[35 + 4 * f] = v.w;
      FCG_KEEP_ORDER();
    };
    // consumption order: units (h, a) = (0,0) (0,1) (1,0) (1,1)
    ql_piece(0); ql_piece(1); qh_piece(0); qh_piece(1);
    ql_piece(2); ql_piece(3);
    ql_piece(4); ql_piece(5); qh_piece(2); qh_piece(3);
    ql_piece(6); ql_piece(7);
  }
}

// Workgroup barrier after the quantisation: every wave's LDS writes complete
// (lgkmcnt(0)) before it arrives, while its weight loads stay in flight.
// (s_waitcnt immediate, gfx9 encoding: vmcnt 63, expcnt 7, lgkmcnt 0.)
__device__ __forceinline__ void barrier_after_lds_writes() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup = one row tile (16 weight rows), nw waves: wave w works on its
// tiles w, w + nw, ...  Each thread issues its activation loads, then the loads of its lane's first
// block, quantises its activation groups into LDS (waiting only for the
// activation loads) and meets the others at the barrier; the weights arrive
// while this happens.  AT: the type of A, R and Y (f16, or f32 for f32
// activations).
template <int QT, int MR, class AT>
__global__ void __launch_bounds__(GEMV_MAX_THREADS)
gemv_kernel(const uint8_t* __restrict__ W, const AT* A, const AT* R,
            AT* Y, int N, int K) {
  extern __shared__ __align__(16) uint8_t smem[];
  const WMap L(N, K);
  const int KB = L.KB, KBp = L.KBp;
  const int G = KBp / TILE_KB;                        // tiles of a row tile
  const int nt = blockDim.x, nw = nt >> 6;
  const GemvLayout Ly = gemv_layout<QT>(MR, KBp, nw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g0 = wave;
  const int r = lane % TILE_ROWS, kbq = lane / TILE_ROWS;
  const int n = blockIdx.x * TILE_ROWS + r;           // < tiled_rows(N)
  uint32_t* rec = (uint32_t*)(smem + Ly.rec);
  float* part_lds = (float*)(smem + Ly.part);

  uint4 araw[qpre<AT>()][act_u4<AT>()];
  quant_issue<MR, AT>(A, K, tid, nt, araw);
  // the residual of the row this lane stores, fetched now so that its latency
  // hides under the weight stream (unconditional loads from a valid address,
  // so that nothing waits on them before the weight loads are issued;
  // without R they read A and are unused)
  AT rres[MR];
  {
    const int nr = n < N ? n : N - 1;
#pragma unroll
    for (int m = 0; m < MR; ++m) rres[m] = *(R ? R + (size_t)m * N + nr : A);
  }
  asm volatile("" ::: "memory");                    // activation and residual loads first

  // the lane's first block (waves without a tile re-read tile 0; never used)
  GemvBlock blk;
  load_block<QT>(W, L, n, (g0 < G ? g0 : 0) * TILE_KB + kbq, blk);
  asm volatile("" ::: "memory");                    // ... then the weight loads

  quant_finish<QT, MR, AT>(A, K, KBp, smem, rec, tid, nt, araw);
  barrier_after_lds_writes();                         // quantised activations ready

  float part[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) part[m] = 0.f;
  for (int g = g0; g < G; g += nw) {
    const int kb = g * TILE_KB + kbq;
    if (g != g0) load_block<QT>(W, L, n, kb, blk);
    if (kb < KB) {
      if constexpr (QT == QT_Q6K)
        q6k_block<MR>(blk.w, blk.w + 32, blk.scv, blk.dbits, kb, KBp, smem, rec, part);
      else
        q45k_block<QT, MR>(blk.w, kb, KBp, smem, rec, part);
    }
  }
  // row sums: the four lanes of a row (kbq = 0..3), then the waves in order
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    part[m] += __shfl_xor(part[m], 16, 64);
    part[m] += __shfl_xor(part[m], 32, 64);
  }
  if (lane < TILE_ROWS) {
#pragma unroll
    for (int m = 0; m < MR; ++m) part_lds[(wave * MR + m) * TILE_ROWS + lane] = part[m];
  }
  __syncthreads();
  if (wave == 0 && lane < TILE_ROWS && n < N) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float y = 0.f;
      for (int w = 0; w < nw; ++w) y += part_lds[(w * MR + m) * TILE_ROWS + lane];
      if (R) y += (float)rres[m];
      Y[(size_t)m * N + n] = (AT)y;
    }
  }
}

// ------------------------------------------------------------------ launch --

template <int QT, int MR, class AT>
static hipError_t launch_gemv_t(const uint8_t* W, const AT* A, const AT* R, AT* Y, int N, int K,
                                hipStream_t st) {
  const int nw = gemv_waves(K);
  const size_t lds = gemv_layout<QT>(MR, tiled_kb(K / QK), nw).total;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  auto kern = gemv_kernel<QT, MR, AT>;
  // raise the dynamic-LDS limit (to the CU's 160 KB) once per device
  static std::atomic<uint64_t> lds_raised{0};
  if (lds > 65536) {
    hipError_t e = raise_lds_limit((const void*)kern, 160 * 1024, lds_raised);
    if (e != hipSuccess) return e;
  }
  const int grid = tiled_rows(N) / TILE_ROWS;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * nw), lds, st, W, A, R, Y, N, K);
  return hipGetLastError();
}

template <int QT, class AT>
static hipError_t launch_gemv_q(const uint8_t* W, const AT* A, const AT* R, AT* Y, int M, int N,
                                int K, hipStream_t st) {
  switch (M) {
    case 1: return launch_gemv_t<QT, 1, AT>(W, A, R, Y, N, K, st);
    case 2: return launch_gemv_t<QT, 2, AT>(W, A, R, Y, N, K, st);
    case 3: return launch_gemv_t<QT, 3, AT>(W, A, R, Y, N, K, st);
    case 4: return launch_gemv_t<QT, 4, AT>(W, A, R, Y, N, K, st);
    case 5: return launch_gemv_t<QT, 5, AT>(W, A, R, Y, N, K, st);
    case 6: return launch_gemv_t<QT, 6, AT>(W, A, R, Y, N, K, st);
    default: return launch_gemv_t<QT, 7, AT>(W, A, R, Y, N, K, st);
  }
}

size_t gemv_lds_bytes(int qtype, int M, int K) {
  const int KBp = tiled_kb(K / QK), nw = gemv_waves(K);
  switch (qtype) {
    case QT_Q4K: return gemv_layout<QT_Q4K>(M, KBp, nw).total;
    case QT_Q5K: return gemv_layout<QT_Q5K>(M, KBp, nw).total;
    default: return gemv_layout<QT_Q6K>(M, KBp, nw).total;
  }
}

template <class AT>
static hipError_t launch_gemv_at(int qtype, const uint8_t* W, const AT* A, const AT* R, AT* Y, int M,
                                 int N, int K, hipStream_t st) {
  if (qtype == QT_Q4K) return launch_gemv_q<QT_Q4K, AT>(W, A, R, Y, M, N, K, st);
  if (qtype == QT_Q5K) return launch_gemv_q<QT_Q5K, AT>(W, A, R, Y, M, N, K, st);
  return launch_gemv_q<QT_Q6K, AT>(W, A, R, Y, M, N, K, st);
}

hipError_t launch_gemv(int qtype, const uint8_t* W, const f16* A, const f16* R, f16* Y, int M,
                       int N, int K, hipStream_t st) {
  return launch_gemv_at<f16>(qtype, W, A, R, Y, M, N, K, st);
}

hipError_t launch_gemv_f32(int qtype, const uint8_t* W, const float* A, const float* R, float* Y,
                           int M, int N, int K, hipStream_t st) {
  return launch_gemv_at<float>(qtype, W, A, R, Y, M, N, K, st);
}

// --------------------------------------------------------------- debug ----

// The decode path's quantisation routine (the same quant_group<AT> that
// the GEMV runs), one thread per 32-value group, written out unswizzled to
// global memory.
template <class AT>
__global__ void debug_quantize_kernel(const AT* __restrict__ A, int M, int K, int8_t* qa, float* s,
                                      int* T) {
  constexpr int U4 = act_u4<AT>();
  const int tasks = M * K / 32;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  uint4 raw[U4];
#pragma unroll
  for (int i = 0; i < U4; ++i)
    raw[i] = t < tasks ? ((const uint4*)(A + (size_t)t * 32))[i] : make_uint4(0, 0, 0, 0);
  uint32_t q[8];
  float sc;
  int tsum, thalf[2];
  quant_group<AT>(raw, q, sc, tsum, thalf);
  if (t >= tasks) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) ((uint32_t*)qa)[(size_t)t * 8 + i] = q[i];
  s[t] = sc;
  T[t] = tsum;
}

hipError_t launch_debug_quantize(const void* A, bool f32, int M, int K, int8_t* qa, float* s, int* T,
                                 hipStream_t st) {
  const long long tasks = (long long)M * K / 32;
  const unsigned grid = (unsigned)((tasks + 255) / 256);
  if (f32)
    hipLaunchKernelGGL(debug_quantize_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)A, M,
                       K, qa, s, T);
  else
    hipLaunchKernelGGL(debug_quantize_kernel<f16>, dim3(grid), dim3(256), 0, st, (const f16*)A, M, K,
                       qa, s, T);
  return hipGetLastError();
}

// Integer sub-block sums with the GEMV's code routines: one thread per block
// (n, kb), blocks read straight from the device layout.
template <int QT>
__global__ void debug_int_dots_kernel(const uint8_t* __restrict__ W, const int8_t* __restrict__ qa,
                                      int M, int N, int K, int* __restrict__ S) {
  const int KB = K / QK;
  const long long gb = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gb >= (long long)N * KB) return;
  const int n = (int)(gb / KB), kb = (int)(gb % KB);
  const WMap L(N, K);
  const uint4 ones = make_uint4(0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u);
  if constexpr (QT != QT_Q6K) {
    constexpr int P = block_bytes_of(QT) / 16;
    uint32_t blk[44];
#pragma unroll
    for (int c = 0; c < P; ++c) {
      const uint4 v = *(const uint4*)(W + L.piece(n, kb, P, c));
      blk[4 * c] = v.x; blk[4 * c + 1] = v.y; blk[4 * c + 2] = v.z; blk[4 * c + 3] = v.w;
    }
    const int ns = K / 32;
    for (int m = 0; m < M; ++m) {
      const uint4* a = (const uint4*)(qa + (size_t)m * K + kb * QK);
      int* out = S + ((size_t)m * N + n) * ns + kb * 8;
      auto pair = [&](auto cc) {
        constexpr int C = decltype(cc)::value;
        uint32_t lo[8], hi[8];
        q45k_codes<QT, C>(blk + 4, blk + (QT == QT_Q5K ? 12 : 4), lo, hi);
        out[2 * C] = dot16u(lo, a[4 * C]) + dot16u(lo + 4, a[4 * C + 1]);
        out[2 * C + 1] = dot16u(hi, a[4 * C + 2]) + dot16u(hi + 4, a[4 * C + 3]);
      };
      pair(std::integral_constant<int, 0>{});
      pair(std::integral_constant<int, 1>{});
      pair(std::integral_constant<int, 2>{});
      pair(std::integral_constant<int, 3>{});
    }
  } else {
    uint32_t ql[32], qh[16];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const uint4 v = *(const uint4*)(W + L.piece(n, kb, 8, f));
      ql[4 * f] = v.x; ql[4 * f + 1] = v.y; ql[4 * f + 2] = v.z; ql[4 * f + 3] = v.w;
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint4 v = *(const uint4*)(W + L.qh_base() + L.piece(n, kb, 4, f));
      qh[4 * f] = v.x; qh[4 * f + 1] = v.y; qh[4 * f + 2] = v.z; qh[4 * f + 3] = v.w;
    }
    const int ns = K / 16;
    for (int m = 0; m < M; ++m) {
      const uint4* a = (const uint4*)(qa + (size_t)m * K + kb * QK);
      int* out = S + ((size_t)m * N + n) * ns + kb * 16;
      auto unit = [&](auto hh, auto aa) {
        constexpr int H = decltype(hh)::value, A_ = decltype(aa)::value;
        constexpr int s0 = 8 * H + 2 * A_;
        uint32_t lo[8], hi[8];
        q6k_codes<H, A_>(ql, qh, lo, hi);
        // 16-value code sums, the quantity the GEMV prologue records
        const uint32_t* o = (const uint32_t*)&ones;
        out[s0] = dot16u(lo, a[s0]) - 32 * dot16u(o, a[s0]);
        out[s0 + 1] = dot16u(lo + 4, a[s0 + 1]) - 32 * dot16u(o, a[s0 + 1]);
        out[s0 + 4] = dot16u(hi, a[s0 + 4]) - 32 * dot16u(o, a[s0 + 4]);
        out[s0 + 5] = dot16u(hi + 4, a[s0 + 5]) - 32 * dot16u(o, a[s0 + 5]);
      };
      unit(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
      unit(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
      unit(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
      unit(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
    }
  }
}

hipError_t launch_debug_int_dots(int qtype, const uint8_t* W, const int8_t* qa, int M, int N, int K,
                                 int* S, hipStream_t st) {
  const long long total = (long long)N * (K / QK);
  const int grid = (int)((total + 255) / 256);
  if (qtype == QT_Q4K)
    hipLaunchKernelGGL(debug_int_dots_kernel<QT_Q4K>, dim3(grid), dim3(256), 0, st, W, qa, M, N, K, S);
  else if (qtype == QT_Q5K)
    hipLaunchKernelGGL(debug_int_dots_kernel<QT_Q5K>, dim3(grid), dim3(256), 0, st, W, qa, M, N, K, S);
  else
    hipLaunchKernelGGL(debug_int_dots_kernel<QT_Q6K>, dim3(grid), dim3(256), 0, st, W, qa, M, N, K, S);
  return hipGetLastError();
}

}  // namespace fcg
