// Decode path (M < 8, and f32 activations): per-32 int8 activation
// quantisation fused into an int8 GEMV that streams the raw Q4_K / Q5_K /
// Q6_K blocks once.
//
// OpenVINO PR #39119, section Implementation: the GEMV quantises the
// activations per 32 values and takes int8 dot products directly against the
// blocks; the residual Add is fused into the output store.
//
// Work layout (one launch):
//   * A workgroup works on one row tile of the device layout (layout.h) at a
//     time: 16 weight rows over all of K.  There are at most max_wgs
//     workgroups (one or two per CU); workgroup b takes row tiles b,
//     b + gridDim.x, ...  It has nw = min(4 * KBp/4, 16) waves; wave w takes
//     quarter w % 4 (64 of the 256 values) of the blocks of the 16 x 4-block
//     tiles w/4, w/4 + nw/4, ... of the row tile, one block per lane
//     (lane = (kb % 4) * 16 + row % 16), so every 16-byte piece load of the
//     wave is one contiguous kilobyte.
//   * Every thread first issues its activation loads (16-byte chunks, the
//     lanes of a 32-value group together), then its first unit's weight
//     loads, then quantises (waiting only for the activation loads, which
//     complete first) into LDS: int8 codes and a per-(row, block) record of
//     the f32 group scales s and the code sums the scale algebra needs
//     (Q4_K, Q5_K: s*T per 32-group for the min term; Q6_K: 16-value sums for
//     the -32 offset).  The activations are quantised once per workgroup.
//   * The weight side of a unit (codes, scale factors) is decoded as soon as
//     its pieces arrive; after the barrier only the integer sums (on the
//     int8 matrix core, four activation rows per instruction) and the f32
//     scale algebra remain.  The first unit of the next row tile is loaded
//     before this row tile's last dots.
//   * Row sums in a fixed order: over a lane's units, then across the four
//     lanes of a row ((b0 + b1) + (b2 + b3), from the lanes' sums in LDS),
//     then across the waves in wave order; R is added and the result is
//     rounded once to the output type.
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "layout.h"
#include "quant.h"

namespace fcg {

constexpr int GEMV_MAX_WAVES = 16;
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
  size_t rec, part, zero, total;
};

// Waves per workgroup (one row tile) for K: one wave per quarter of each
// 4-block tile of the row tile, at most 16 (a multiple of 4, so that a wave
// keeps one quarter).
__host__ __device__ inline int gemv_waves(int K) {
  const int w = 4 * (tiled_kb(K / QK) / TILE_KB);
  return w < GEMV_MAX_WAVES ? w : GEMV_MAX_WAVES;
}

// LDS: qa int8 [MR][KBp] records of QA_REC bytes (256 codes + 16 bytes of
// padding, so that the four blocks a wave reads at once start on different
// banks) | rec u32 [MR][KBp][REC] | part f32 [2][waves][MR][16][4] (a wave's
// sums for the 16 rows of a row tile, one per lane: row, then the lane's
// block within the 4-block tile; two buffers, alternating over the
// workgroup's row tiles) | 256 zero bytes (the activation operand of the
// lanes whose matrix-core rows are off the block diagonal, see dot_unit).
constexpr int QA_REC = QK + 16;
template <int QT>
__host__ __device__ constexpr GemvLayout gemv_layout(int MR, int KBp, int waves) {
  const size_t rec = (size_t)MR * KBp * QA_REC;
  const size_t part = rec + (size_t)MR * KBp * GemvFmt<QT>::REC * 4;
  const size_t zero = part + (size_t)2 * waves * MR * 64 * 4;
  return GemvLayout{rec, part, zero, zero + QK};
}

// ------------------------------------------------ activation quantisation --
// The MR x K activations are cut into 16-byte chunks (chunk_vals<AT>()
// values each); thread tid quantises chunks tid, tid + nt, ... with the
// lanes of each 32-value group together (quant_chunk), so every wave load is
// one contiguous kilobyte.  The loads of the first QPRE rounds are issued
// before the weight loads, so the quantisation waits only for them (loads
// complete in order) while the weights are still in flight.
constexpr int QPRE = 4;

template <class AT>
__device__ __forceinline__ int act_chunks(int MR, int K) { return MR * K / chunk_vals<AT>(); }

// The load of chunk c (wbase: the wave's first chunk; waves past the end
// skip, lanes past it load nothing and quantise zeros).
template <class AT>
__device__ __forceinline__ uint4 act_load(const AT* A, int nch, int c, int wbase) {
  uint4 v = make_uint4(0, 0, 0, 0);
  if (wbase < nch && c < nch) v = *(const uint4*)(A + (size_t)c * chunk_vals<AT>());
  return v;
}

// Quantise chunk c (held in raw) into LDS: its codes at their place in the
// (m, kb) code record, and, from the group's first lane (and, for Q6_K, the
// first lane of its second half), the record entries of the group.
// kb_magic = ceil(2^32 / KB) (KB = K / 256 > 1; 0 for KB = 1): the
// activation row of a block index b < MR * KB is umulhi(b, kb_magic),
// exactly, since b < 2^32 / KB.
template <int QT, int MR, class AT>
__device__ __forceinline__ void act_quant(uint4 raw, int c, int nch, int K, int KBp,
                                          uint32_t kb_magic, uint8_t* smem, uint32_t* rec) {
  constexpr int CV = chunk_vals<AT>(), GL = group_lanes<AT>(), REC = GemvFmt<QT>::REC;
  uint32_t q[2];
  float s;
  int tsum, thalf;
  quant_chunk<AT>(raw, q, s, tsum, thalf);
  if (c >= nch) return;
  const uint32_t e = (uint32_t)c * CV;                // first value (flat over MR x K)
  uint32_t m = 0, pos = e;
  if constexpr (MR > 1) {
    m = kb_magic ? __umulhi(e / QK, kb_magic) : e / QK;
    pos = e - __umul24(m, (uint32_t)K);
  }
  const uint32_t kb = pos / QK, off = pos % QK, g = off / 32;
  const uint32_t mk = __umul24(m, (uint32_t)KBp) + kb;  // the (m, kb) record
  uint8_t* dst = smem + __umul24(mk, (uint32_t)QA_REC) + off;
  if constexpr (CV == 8) *(uint2*)dst = make_uint2(q[0], q[1]);
  else *(uint32_t*)dst = q[0];
  uint32_t* r = rec + __umul24(mk, (uint32_t)REC);
  const uint32_t lg = (uint32_t)c % GL;               // lane within the group
  if (lg == 0) r[g] = __builtin_bit_cast(uint32_t, s);
  if constexpr (QT != QT_Q6K) {
    if (lg == 0) r[8 + g] = __builtin_bit_cast(uint32_t, s * (float)tsum);
  } else {
    if (lg == 0) r[8 + 2 * g] = (uint32_t)thalf;
    if (lg == GL / 2) r[8 + 2 * g + 1] = (uint32_t)thalf;
  }
}

// ----------------------------------------- codes and integer sub-block sums --
// Q5_K: 176 B = d|dmin, scales[12], qh[32], qs[128] (11 x 16 B).  For the
// sub-block pair (2c, 2c+1): qs[32c + l] low nibble -> value 64c + l, high
// nibble -> 64c + 32 + l; bits 2c / 2c+1 of qh[l] are the fifth bits.
// Q4_K: 144 B = d|dmin, scales[12], qs[128] (9 x 16 B); the same nibbles,
// no fifth bit (mobius GGUF proposal, section 7.3).
// Q6_K: ql[64h + 32a + l] low nibble -> value 128h + 32a + l (bit pair 2a of
// qh[32h + l]), high nibble -> value 128h + 32(a+2) + l (bit pair 2a+4).
// Codes are packed four to a word, value order.

// sum of four code words times 16 activation codes (the debug kernel's
// activation sums)
__device__ __forceinline__ int dot16u(const uint32_t* c, uint4 a) {
  int s = dot4((int)c[0], (int)a.x, 0);
  s = dot4((int)c[1], (int)a.y, s);
  s = dot4((int)c[2], (int)a.z, s);
  return dot4((int)c[3], (int)a.w, s);
}

__device__ __forceinline__ void words(uint4 v, uint32_t* w) {
  w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
}

// ------------------------------------------------------------ quarters ----
// A unit of work is one quarter of the 64 blocks of a tile: quarter q of a
// block is its values 64q .. 64q + 63 (Q4_K / Q5_K: the sub-block pair
// (2q, 2q + 1)) or, for Q6_K, the values 128h + 32a + [0, 32) and
// 128h + 32a + 64 + [0, 32) with q = 2h + a (the values one ql byte
// half and one qh bit pair feed).  The 16-byte pieces a quarter needs:
//   Q5_K: the header (d, dmin, scales), both qh pieces, qs pieces 2q, 2q+1;
//   Q4_K: the header, qs pieces 2q, 2q+1;
//   Q6_K: ql pieces 2q, 2q+1, qh pieces 2h, 2h+1, the scales piece and d.
template <int QT> struct GemvUnit {
  static constexpr int NV = QT == QT_Q4K ? 3 : QT == QT_Q5K ? 5 : 6;
  uint4 v[NV];
};

// Byte offsets of the lane's block in the planes of tile t.
struct UnitAddr {
  const uint8_t* W;
  size_t qh_base, sc_base, d_base;
  int lane;
};

template <int QT>
__device__ __forceinline__ void load_unit(const UnitAddr& ua, size_t t, int q, GemvUnit<QT>& u) {
  const size_t l16 = (size_t)ua.lane << 4;
  if constexpr (QT != QT_Q6K) {
    constexpr int P = block_bytes_of(QT) / 16;
    const uint8_t* b = ua.W + ((t * P) << 10) + l16;
    constexpr int QS = QT == QT_Q5K ? 3 : 1;          // first qs piece
    u.v[0] = *(const uint4*)b;
    if constexpr (QT == QT_Q5K) {
      u.v[1] = *(const uint4*)(b + 1024);
      u.v[2] = *(const uint4*)(b + 2048);
    }
    u.v[QT == QT_Q5K ? 3 : 1] = *(const uint4*)(b + ((QS + 2 * q) << 10));
    u.v[QT == QT_Q5K ? 4 : 2] = *(const uint4*)(b + ((QS + 2 * q + 1) << 10));
  } else {
    const uint8_t* ql = ua.W + ((t * 8 + 2 * q) << 10) + l16;
    const uint8_t* qh = ua.W + ua.qh_base + ((t * 4 + 2 * (q >> 1)) << 10) + l16;
    u.v[0] = *(const uint4*)ql;
    u.v[1] = *(const uint4*)(ql + 1024);
    u.v[2] = *(const uint4*)qh;
    u.v[3] = *(const uint4*)(qh + 1024);
    u.v[4] = *(const uint4*)(ua.W + ua.sc_base + (t << 10) + l16);
    u.v[5].x = *(const uint16_t*)(ua.W + ua.d_base + t * 128 + ((size_t)ua.lane << 1));
  }
}

// The weight side of a quarter, decoded as soon as its pieces arrive (before
// the activations are needed): the codes and the block's scale factors.
template <int QT> struct QDec {
  uint32_t lo[8], hi[8];    // packed codes of the quarter's lo / hi values (4 per word)
  float f[4];               // Q4_K / Q5_K: d*sc, d*sc', dmin*m, dmin*m' of the pair; Q6_K: d
  int c[4];                 // Q6_K: the int8 scales of sub-blocks s0, s0+1, s0+4, s0+5
};

__device__ __forceinline__ uint32_t rotr(uint32_t x, int k) { return __builtin_amdgcn_alignbit(x, x, k); }

// Q4_K / Q5_K quarter q (sub-block pair (2q, 2q+1)); q is wave-uniform.
template <int QT>
__device__ __forceinline__ void q45k_decode(const GemvUnit<QT>& u, int q, QDec<QT>& o) {
  const uint4 h = u.v[0];
  const float d = h2f(h.x), dmin = h2f(h.x >> 16);
  // 6-bit scales / mins as bytes, j = 0..3 (pairs 0, 1) or j = 4..7 (pairs 2, 3)
  const uint32_t scw = q < 2 ? h.y & 0x3F3F3F3Fu : (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
  const uint32_t mw = q < 2 ? h.z & 0x3F3F3F3Fu : ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
  const int sh = 16 * (q & 1);
  o.f[0] = d * (float)__builtin_amdgcn_ubfe(scw, sh, 8);
  o.f[1] = d * (float)__builtin_amdgcn_ubfe(scw, sh + 8, 8);
  o.f[2] = dmin * (float)__builtin_amdgcn_ubfe(mw, sh, 8);
  o.f[3] = dmin * (float)__builtin_amdgcn_ubfe(mw, sh + 8, 8);
  uint32_t qs[8];
  if constexpr (QT == QT_Q5K) {
    words(u.v[3], qs); words(u.v[4], qs + 4);
  } else {
    words(u.v[1], qs); words(u.v[2], qs + 4);
  }
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    o.lo[w] = qs[w] & 0x0F0F0F0Fu;
    o.hi[w] = (qs[w] >> 4) & 0x0F0F0F0Fu;
  }
  if constexpr (QT == QT_Q5K) {
    // fifth bits: bit 2q (lo) / 2q+1 (hi) of each qh byte to bit 4
    const uint32_t qh[8] = {u.v[1].x, u.v[1].y, u.v[1].z, u.v[1].w,
                            u.v[2].x, u.v[2].y, u.v[2].z, u.v[2].w};
    const int rl = (28 + 2 * q) & 31, rh = (29 + 2 * q) & 31;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      o.lo[w] |= rotr(qh[w], rl) & 0x10101010u;
      o.hi[w] |= rotr(qh[w], rh) & 0x10101010u;
    }
  }
}

// Q6_K quarter q = 2H + A: ql half A of 64-value half H, qh bit pair A.
__device__ __forceinline__ void q6k_decode(const GemvUnit<QT_Q6K>& u, int q, QDec<QT_Q6K>& o) {
  const int H = q >> 1, A_ = q & 1;
  o.f[0] = h2f(u.v[5].x);
  // sub-blocks s0 = 8H + 2A, s0+1 in scale word 2H, s0+4, s0+5 in word 2H+1
  const uint32_t w0 = H ? u.v[4].z : u.v[4].x, w1 = H ? u.v[4].w : u.v[4].y;
  o.c[0] = __builtin_amdgcn_sbfe(w0, 16 * A_, 8);
  o.c[1] = __builtin_amdgcn_sbfe(w0, 16 * A_ + 8, 8);
  o.c[2] = __builtin_amdgcn_sbfe(w1, 16 * A_, 8);
  o.c[3] = __builtin_amdgcn_sbfe(w1, 16 * A_ + 8, 8);
  const uint32_t ql[8] = {u.v[0].x, u.v[0].y, u.v[0].z, u.v[0].w, u.v[1].x, u.v[1].y, u.v[1].z, u.v[1].w};
  const uint32_t qh[8] = {u.v[2].x, u.v[2].y, u.v[2].z, u.v[2].w, u.v[3].x, u.v[3].y, u.v[3].z, u.v[3].w};
  const int rl = (28 + 2 * A_) & 31;                  // bits 2A, 2A+1 -> 4, 5
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    o.lo[w] = (ql[w] & 0x0F0F0F0Fu) | (rotr(qh[w], rl) & 0x30303030u);
    o.hi[w] = ((ql[w] >> 4) & 0x0F0F0F0Fu) | ((qh[w] >> (2 * A_)) & 0x30303030u);
  }
}

template <int QT>
__device__ __forceinline__ void decode_unit(const GemvUnit<QT>& u, int q, QDec<QT>& o) {
  if constexpr (QT == QT_Q6K) q6k_decode(u, q, o);
  else q45k_decode<QT>(u, q, o);
}

// ------------------------------------------ integer sums on the matrix core --
// The integer sums come from v_mfma_i32_16x16x64_i8 with a block-diagonal
// activation operand, which gives every lane the sums of its own block for
// four activation rows at once.
// Lane l (block (row l % 16, kb = 4g + l / 16) of the tile) supplies the B
// operand: 16 codes of its block.  Row i = 4 gi + mi of the A operand holds
// activation row 4 s + mi of block 4g + gi in the K slice of lane group gi and
// zeros in the other three slices.  Lane l supplies row l % 16 in slice
// l / 16, so only the lanes with (l / 4) % 4 == l / 16 load activation codes;
// the others read zero bytes.  The instruction sums over each lane group's
// slice separately for a given (row, column), so D row 4 gi + r, column w is
// the dot product of block (w, 4g + gi)'s 16 codes with activation row
// 4 s + r's codes of that block; in D's layout (lane l holds rows
// 4 (l / 16) + r of column l % 16) that is lane l's own block, rows 4 s + r.
// The sums are exact integers.  Against v_dot4_i32_i8 sums (one instruction
// per four codes and activation row) this takes the GEMV at four and seven
// rows 9-20 % faster; at one row the two are even.
typedef int int4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int4v mx_dot(uint4 a, const uint32_t* c, int4v acc) {
  const int4v av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
  const int4v cv = {(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, cv, acc, 0, 0, 0);
}

// The lanes whose A-operand row lies on the block diagonal.
__device__ __forceinline__ bool mx_diag(int lane) { return ((lane >> 2) & 3) == (lane >> 4); }

// Byte offset, within a block's 256 codes, of the quarter's activation
// operand j: Q4_K / Q5_K values 64q + 16j + [0, 16); Q6_K the sub-blocks
// s0, s0 + 1, s0 + 4, s0 + 5 of 16 values.
template <int QT>
__device__ __forceinline__ int mx_off(int q, int j) {
  if constexpr (QT != QT_Q6K) return 64 * q + 16 * j;
  else return 16 * (4 * (q & 2) + 2 * (q & 1)) + 16 * (j & 1) + 64 * (j >> 1);
}

// The quarter's integer sums for four activation rows from its four
// activation operands: Q4_K / Q5_K S[0] group 2q, S[1] group 2q + 1; Q6_K
// S[0..3] the sub-blocks s0, s0 + 1, s0 + 4, s0 + 5 (codes 0..63, without
// the -32 offset).
template <int QT>
__device__ __forceinline__ void mx_sums(const QDec<QT>& o, const uint4* a, int4v* S) {
  const int4v z = {0, 0, 0, 0};
  if constexpr (QT != QT_Q6K) {
    S[0] = mx_dot(a[1], o.lo + 4, mx_dot(a[0], o.lo, z));
    S[1] = mx_dot(a[3], o.hi + 4, mx_dot(a[2], o.hi, z));
  } else {
    S[0] = mx_dot(a[0], o.lo, z);
    S[1] = mx_dot(a[1], o.lo + 4, z);
    S[2] = mx_dot(a[2], o.hi, z);
    S[3] = mx_dot(a[3], o.hi + 4, z);
  }
}

// The activation side of quarter q of block kb -> part[m] (the lane's
// contribution to row m).  Every lane takes part in the matrix-core
// instructions (the lanes of zero padding blocks too, whose sums are then
// dropped).  zero: the LDS offset of 256 zero bytes.
template <int QT, int MR>
__device__ __forceinline__ void dot_unit(const QDec<QT>& o, int q, int kb, int KB, int KBp,
                                            const uint8_t* smem, uint32_t zero, const uint32_t* rec,
                                            float* part) {
  constexpr int REC = GemvFmt<QT>::REC, SETS = (MR + 3) / 4;
  const int lane = threadIdx.x & 63;
  int4v S[SETS][4];
#pragma unroll
  for (int s = 0; s < SETS; ++s) {
    const int m = 4 * s + (lane & 3);
    const uint32_t base = mx_diag(lane) && m < MR && kb < KB
                              ? __umul24((uint32_t)(m * KBp + kb), (uint32_t)QA_REC)
                              : zero;
    uint4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *(const uint4*)(smem + base + mx_off<QT>(q, j));
    mx_sums<QT>(o, a, S[s]);
  }
  if (kb >= KB) return;                               // zero padding block
  const uint32_t r0 = __umul24((uint32_t)kb, (uint32_t)REC);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const uint32_t* r = rec + r0 + (uint32_t)(m * KBp * REC);
    const int4v* Sm = S[m / 4];
    if constexpr (QT != QT_Q6K) {
      const int S0 = Sm[0][m % 4], S1 = Sm[1][m % 4];
      const float2 s2 = *(const float2*)(r + 2 * q);
      const float2 t2 = *(const float2*)(r + 8 + 2 * q);
      float X = o.f[0] * (s2.x * (float)S0);
      X = fmaf(o.f[1], s2.y * (float)S1, X);
      float Z = o.f[2] * t2.x;
      Z = fmaf(o.f[3], t2.y, Z);
      part[m] += X - Z;
    } else {
      const int s0 = 4 * (q & 2) + 2 * (q & 1);
      const int2 tl = *(const int2*)(r + 8 + s0);
      const int2 th = *(const int2*)(r + 8 + s0 + 4);
      const int S0 = Sm[0][m % 4] - 32 * tl.x;
      const int S1 = Sm[1][m % 4] - 32 * tl.y;
      const int S4 = Sm[2][m % 4] - 32 * th.x;
      const int S5 = Sm[3][m % 4] - 32 * th.y;
      const int I = __mul24(o.c[0], S0) + __mul24(o.c[1], S1);
      const int J = __mul24(o.c[2], S4) + __mul24(o.c[3], S5);
      const float sI = __builtin_bit_cast(float, r[s0 >> 1]);
      const float sJ = __builtin_bit_cast(float, r[(s0 + 4) >> 1]);
      float X = sI * (float)I;
      X = fmaf(sJ, (float)J, X);
      part[m] = fmaf(o.f[0], X, part[m]);
    }
  }
}

// ---------------------------------------------------------------- kernel --

// Cross-row lane exchanges on the gfx950 permlane-swap instructions (VALU,
// no LDS round trip).  lane_xor16_even_rows(x) is x of lane l ^ 16 in the
// even 16-lane rows (lanes 0-15, 32-47); lane_xor32_low_half(x) is x of lane
// l + 32 in lanes 0-31.  Other lanes receive values that are not used.
__device__ __forceinline__ float lane_xor16_even_rows(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_permlane16_swap(u, u, false, false)[1]);
}
__device__ __forceinline__ float lane_xor32_low_half(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_permlane32_swap(u, u, false, false)[1]);
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

// Workgroup = one row tile (16 weight rows), nw = 4 * nwq waves: wave w takes
// quarter w % 4 of the tiles w / 4, w / 4 + nwq, ...  Each thread issues its
// activation loads, then the loads of its first unit, quantises its
// activation groups into LDS (waiting only for the activation loads) and
// meets the others at the barrier; the weights arrive while this happens.
// AT: the type of A, R and Y (f16, or f32 for f32 activations).
template <int QT, int MR, class AT, bool MULTI>
__global__ void __launch_bounds__(GEMV_MAX_THREADS)
gemv_kernel(const uint8_t* __restrict__ W, const AT* A, const AT* R,
            AT* Y, int N, int K) {
  extern __shared__ __align__(16) uint8_t smem[];
  const WMap L(N, K);
  const int KB = L.KB, KBp = L.KBp;
  const int G = KBp / TILE_KB;                        // tiles of a row tile
  const int nrt = tiled_rows(N) / TILE_ROWS;          // row tiles
  const int nt = blockDim.x, nw = nt >> 6, nwq = nw >> 2;
  const GemvLayout Ly = gemv_layout<QT>(MR, KBp, nw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = wave & 3, g0 = wave >> 2;             // g0 < G: nwq <= G
  const int kbq = lane / TILE_ROWS;
  uint32_t* rec = (uint32_t*)(smem + Ly.rec);
  float* part_lds = (float*)(smem + Ly.part);

  const int nch = act_chunks<AT>(MR, K);
  const uint32_t kb_magic = KB > 1 ? 0xFFFFFFFFu / (uint32_t)KB + 1u : 0u;
  uint4 araw[QPRE];
#pragma unroll
  for (int r = 0; r < QPRE; ++r) araw[r] = act_load<AT>(A, nch, r * nt + tid, r * nt + wave * 64);
  // the residual this thread adds in the final sums of a row tile (thread
  // t < 16 * MR: row t / 16, column of row tile row t % 16), fetched a row
  // tile ahead so that its latency hides under the weight stream
  const int fm = tid / TILE_ROWS, fr = tid % TILE_ROWS;
  const bool fin = tid < TILE_ROWS * MR;
  // (as raw bits, converted where they are added: a conversion right after
  // the load would make the wave wait for it there)
  auto load_r = [&](int rt) -> uint32_t {
    const int c = rt * TILE_ROWS + fr;
    if (!R || !fin) return 0u;
    const AT* p = R + (size_t)fm * N + (c < N ? c : N - 1);
    if constexpr (sizeof(AT) == 2) return *(const uint16_t*)p;
    else return *(const uint32_t*)p;
  };
  auto r_value = [](uint32_t bits) -> float {
    if constexpr (sizeof(AT) == 2) return h2f(bits);
    else return __builtin_bit_cast(float, bits);
  };
  int rt = blockIdx.x;
  uint32_t rres = load_r(rt);
  asm volatile("" ::: "memory");                    // activation and residual loads first

  const UnitAddr ua{W, L.qh_base(), L.sc_base(), L.d_base(), lane};
  GemvUnit<QT> cur;
  load_unit<QT>(ua, (size_t)rt * G + g0, q, cur);
  asm volatile("" ::: "memory");                    // ... then the weight loads

#pragma unroll
  for (int r = 0; r < QPRE; ++r)
    if (r * nt + wave * 64 < nch)
      act_quant<QT, MR, AT>(araw[r], r * nt + tid, nch, K, KBp, kb_magic, smem, rec);
  for (int c0 = QPRE * nt; c0 + wave * 64 < nch; c0 += nt)
    act_quant<QT, MR, AT>(act_load<AT>(A, nch, c0 + tid, c0 + wave * 64), c0 + tid, nch, K, KBp,
                          kb_magic, smem, rec);
  // the first unit's weight side, while the other waves finish quantising
  if (tid < QK / 16) *(uint4*)(smem + Ly.zero + 16 * tid) = make_uint4(0, 0, 0, 0);
  QDec<QT> dec;
  decode_unit<QT>(cur, q, dec);
  barrier_after_lds_writes();                         // quantised activations ready

  // row tiles blockIdx.x, + gridDim.x, ...: the first unit of the next row
  // tile (and its residual) is loaded before this row tile's last dots
  for (int i = 0;; ++i) {
    float part[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) part[m] = 0.f;
    const size_t t0 = (size_t)rt * G;                 // first tile of the row tile
    int g = g0;
    if constexpr (MULTI) {
      // later units: the next unit's loads are issued before this unit's dots
      for (; g + nwq < G; g += nwq) {
        load_unit<QT>(ua, t0 + g + nwq, q, cur);
        dot_unit<QT, MR>(dec, q, g * TILE_KB + kbq, KB, KBp, smem, (uint32_t)Ly.zero, rec, part);
        decode_unit<QT>(cur, q, dec);
      }
    }
    const int rtn = rt + gridDim.x;
    const bool more = rtn < nrt;
    uint32_t rnext = 0u;
    if (more) {
      load_unit<QT>(ua, (size_t)rtn * G + g0, q, cur);
      rnext = load_r(rtn);
    }
    dot_unit<QT, MR>(dec, q, g * TILE_KB + kbq, KB, KBp, smem, (uint32_t)Ly.zero, rec, part);
    // row sums: the four lanes of a row (kbq = 0..3), then the waves in order
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      part[m] += lane_xor16_even_rows(part[m]);
      part[m] += lane_xor32_low_half(part[m]);
    }
    float* pb = part_lds + (size_t)(i & 1) * nw * MR * 64;
    if (lane < TILE_ROWS) {
#pragma unroll
      for (int m = 0; m < MR; ++m) pb[(wave * MR + m) * TILE_ROWS + lane] = part[m];
    }
    __syncthreads();
    if (fin) {
      float v[GEMV_MAX_WAVES];
#pragma unroll
      for (int w = 0; w < GEMV_MAX_WAVES; ++w)
        v[w] = w < nw ? pb[(w * MR + fm) * TILE_ROWS + fr] : 0.f;
      float y = 0.f;
#pragma unroll
      for (int w = 0; w < GEMV_MAX_WAVES; ++w) y += v[w];
      const int c = rt * TILE_ROWS + fr;
      if (c < N) Y[(size_t)fm * N + c] = (AT)(y + r_value(rres));
    }
    if (!more) break;
    rt = rtn;
    rres = rnext;
    decode_unit<QT>(cur, q, dec);
  }
}

// ------------------------------------------------------------------ launch --

// grid: one workgroup per row tile, at most max_wgs (then each takes row
// tiles blockIdx.x, + gridDim.x, ...).
template <int QT, int MR, class AT>
static hipError_t launch_gemv_t(const uint8_t* W, const AT* A, const AT* R, AT* Y, int N, int K,
                                int max_wgs, hipStream_t st) {
  const int nw = gemv_waves(K);
  const int G = tiled_kb(K / QK) / TILE_KB;
  const size_t lds = gemv_layout<QT>(MR, tiled_kb(K / QK), nw).total;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  auto kern = 4 * G > nw ? gemv_kernel<QT, MR, AT, true> : gemv_kernel<QT, MR, AT, false>;
  // raise the dynamic-LDS limit (to the CU's 160 KB) once per device and kernel
  static std::atomic<uint64_t> lds_raised[2];
  if (lds > 65536) {
    hipError_t e = raise_lds_limit((const void*)kern, 160 * 1024, lds_raised[4 * G > nw]);
    if (e != hipSuccess) return e;
  }
  const int nrt = tiled_rows(N) / TILE_ROWS;
  const int grid = nrt < max_wgs ? nrt : max_wgs;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * nw), lds, st, W, A, R, Y, N, K);
  return hipGetLastError();
}

template <int QT, class AT>
static hipError_t launch_gemv_q(const uint8_t* W, const AT* A, const AT* R, AT* Y, int M, int N,
                                int K, int max_wgs, hipStream_t st) {
  switch (M) {
    case 1: return launch_gemv_t<QT, 1, AT>(W, A, R, Y, N, K, max_wgs, st);
    case 2: return launch_gemv_t<QT, 2, AT>(W, A, R, Y, N, K, max_wgs, st);
    case 3: return launch_gemv_t<QT, 3, AT>(W, A, R, Y, N, K, max_wgs, st);
    case 4: return launch_gemv_t<QT, 4, AT>(W, A, R, Y, N, K, max_wgs, st);
    case 5: return launch_gemv_t<QT, 5, AT>(W, A, R, Y, N, K, max_wgs, st);
    case 6: return launch_gemv_t<QT, 6, AT>(W, A, R, Y, N, K, max_wgs, st);
    default: return launch_gemv_t<QT, 7, AT>(W, A, R, Y, N, K, max_wgs, st);
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
                                 int N, int K, int max_wgs, hipStream_t st) {
  if (qtype == QT_Q4K) return launch_gemv_q<QT_Q4K, AT>(W, A, R, Y, M, N, K, max_wgs, st);
  if (qtype == QT_Q5K) return launch_gemv_q<QT_Q5K, AT>(W, A, R, Y, M, N, K, max_wgs, st);
  return launch_gemv_q<QT_Q6K, AT>(W, A, R, Y, M, N, K, max_wgs, st);
}

hipError_t launch_gemv(int qtype, const uint8_t* W, const f16* A, const f16* R, f16* Y, int M,
                       int N, int K, int max_wgs, hipStream_t st) {
  return launch_gemv_at<f16>(qtype, W, A, R, Y, M, N, K, max_wgs, st);
}

hipError_t launch_gemv_f32(int qtype, const uint8_t* W, const float* A, const float* R, float* Y,
                           int M, int N, int K, int max_wgs, hipStream_t st) {
  return launch_gemv_at<float>(qtype, W, A, R, Y, M, N, K, max_wgs, st);
}

// --------------------------------------------------------------- debug ----

// The decode path's quantisation routine (the quant_chunk<AT> that the GEMV
// runs), one thread per 16-byte chunk, written out unswizzled to global
// memory: codes, per group its scale and code sum, and (H not null) the
// code sum of each 16-value half of a group.
template <class AT>
__global__ void debug_quantize_kernel(const AT* __restrict__ A, int M, int K, int8_t* qa, float* s,
                                      int* T, int* H) {
  constexpr int CV = chunk_vals<AT>(), GL = group_lanes<AT>();
  const int nch = M * K / CV;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const uint4 raw = c < nch ? *(const uint4*)(A + (size_t)c * CV) : make_uint4(0, 0, 0, 0);
  uint32_t q[2];
  float sc;
  int tsum, thalf;
  quant_chunk<AT>(raw, q, sc, tsum, thalf);           // every lane takes part
  if (c >= nch) return;
  if constexpr (CV == 8) *(uint2*)(qa + (size_t)c * CV) = make_uint2(q[0], q[1]);
  else *(uint32_t*)(qa + (size_t)c * CV) = q[0];
  if (c % GL == 0) {
    s[c / GL] = sc;
    T[c / GL] = tsum;
  }
  if (H && c % (GL / 2) == 0) H[c / (GL / 2)] = thalf;
}

hipError_t launch_debug_quantize(const void* A, bool f32, int M, int K, int8_t* qa, float* s, int* T,
                                 int* H, hipStream_t st) {
  const long long chunks = (long long)M * K / (f32 ? chunk_vals<float>() : chunk_vals<f16>());
  const unsigned grid = (unsigned)((chunks + 255) / 256);
  if (f32)
    hipLaunchKernelGGL(debug_quantize_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)A, M,
                       K, qa, s, T, H);
  else
    hipLaunchKernelGGL(debug_quantize_kernel<f16>, dim3(grid), dim3(256), 0, st, (const f16*)A, M, K,
                       qa, s, T, H);
  return hipGetLastError();
}

// Integer sub-block sums with the GEMV's own unit loads, decoder and
// matrix-core sums, in the GEMV's lane mapping: workgroup = one 16 x 4-block
// tile t of the device layout, wave = quarter; Q6_K sums include the -32
// offset.
template <int QT>
__global__ void __launch_bounds__(256)
debug_int_dots_kernel(const uint8_t* __restrict__ W, const int8_t* __restrict__ qa, int M, int N,
                         int K, int* __restrict__ S) {
  const WMap L(N, K);
  const int KB = L.KB, G = L.KBp / TILE_KB;
  const int t = blockIdx.x, lane = threadIdx.x & 63;
  const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = (t / G) * TILE_ROWS + lane % TILE_ROWS, kb = (t % G) * TILE_KB + lane / TILE_ROWS;
  const UnitAddr ua{W, L.qh_base(), L.sc_base(), L.d_base(), lane};
  GemvUnit<QT> u;
  load_unit<QT>(ua, (size_t)t, q, u);
  QDec<QT> o;
  decode_unit<QT>(u, q, o);
  constexpr int NS = QT == QT_Q6K ? 16 : 8;
  const uint4 ones = make_uint4(0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u);
  for (int s = 0; 4 * s < M; ++s) {                   // wave-uniform
    const int md = 4 * s + (lane & 3);
    const bool live = mx_diag(lane) && md < M && kb < KB;
    uint4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[j] = live ? *(const uint4*)(qa + (size_t)md * K + kb * QK + mx_off<QT>(q, j))
                  : make_uint4(0, 0, 0, 0);
    int4v R[4];
    mx_sums<QT>(o, a, R);
    if (n >= N || kb >= KB) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * s + r;
      if (m >= M) break;
      int* out = S + ((size_t)m * N + n) * (KB * NS) + kb * NS;
      if constexpr (QT != QT_Q6K) {
        out[2 * q] = R[0][r];
        out[2 * q + 1] = R[1][r];
      } else {
        const int s0 = 4 * (q & 2) + 2 * (q & 1);
        const uint32_t* e = (const uint32_t*)&ones;
        const uint4* ar = (const uint4*)(qa + (size_t)m * K + kb * QK);
        out[s0] = R[0][r] - 32 * dot16u(e, ar[s0]);
        out[s0 + 1] = R[1][r] - 32 * dot16u(e, ar[s0 + 1]);
        out[s0 + 4] = R[2][r] - 32 * dot16u(e, ar[s0 + 4]);
        out[s0 + 5] = R[3][r] - 32 * dot16u(e, ar[s0 + 5]);
      }
    }
  }
}

hipError_t launch_debug_int_dots(int qtype, const uint8_t* W, const int8_t* qa, int M, int N, int K,
                                 int* S, hipStream_t st) {
  const int tiles = (tiled_rows(N) / TILE_ROWS) * (tiled_kb(K / QK) / TILE_KB);
  if (qtype == QT_Q4K)
    hipLaunchKernelGGL(debug_int_dots_kernel<QT_Q4K>, dim3(tiles), dim3(256), 0, st, W, qa, M, N, K, S);
  else if (qtype == QT_Q5K)
    hipLaunchKernelGGL(debug_int_dots_kernel<QT_Q5K>, dim3(tiles), dim3(256), 0, st, W, qa, M, N, K, S);
  else
    hipLaunchKernelGGL(debug_int_dots_kernel<QT_Q6K>, dim3(tiles), dim3(256), 0, st, W, qa, M, N, K, S);
  return hipGetLastError();
}

}  // namespace fcg
