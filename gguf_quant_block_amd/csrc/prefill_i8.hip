// Int8 matrix-core prefill: a variant of the prefill FC that multiplies
// per-32 int8 activations by the blocks' integer codes on the int8 matrix
// cores (v_mfma_i32_16x16x32_i8) and applies the scales in f32 per 32-value
// group.  It computes exactly what the decode path computes (the int8
// emulation of the FC: the same quantisation routine, exact integer
// sub-block sums, f32 scale algebra), at any row count; the f16 prefill
// path's tolerance (fp64 FC) does not apply to it.
//
// OpenVINO PR #39119, sections Transformation and Implementation: per-32
// dynamic int8 quantisation of the activations and integer dot products on
// the raw blocks (there for the GEMV).  The ROCm llama.cpp pull request 37,
// section Motivation, compares such an int8 matrix-core kernel (MMQ) with an
// f16 GEMM over dequantised weights; this variant is that comparison on the
// same tile machinery as the f16 prefill.
//
// Two launches:
//   * quant_i8_kernel: A [M, K] f16 -> codes qa [M, K] int8, and per group
//     the scale s and u = s * T (T the sum of the group's 32 codes) stored
//     group-major, sT[K/32][Mp], uT[K/32][Mp] (Mp = M rounded up to 128; the
//     padding rows hold zeros).
//   * prefill_i8_kernel: the loader-wave structure of the f16 prefill
//     (mfma_dma.h) with four compute waves: wave 4 streams the activation
//     codes and their scales, wave 5 the weight pieces (the f16 path's
//     loader), into a ring of three LDS stages; waves 0-3 compute, wave w on
//     weight rows 32w .. 32w + 31.  Per k-step (32 values = one activation
//     group) a compute wave turns its weight pieces into int8 codes, runs one
//     int8 MFMA per 16x16 sub-tile (two for Q6_K, whose 16-value sub-blocks
//     carry their own scales) and adds the group's contribution in f32:
//       Q4_K / Q5_K  acc += s * (d sc_j) * S, and per stage the min term
//                    - sum_g u[m][g] (dmin m_g)[n] as one f32 MFMA (k = 4)
//       Q6_K         acc += s * d * (sc_lo * S_lo + sc_hi * S_hi)
//     The activations are the MFMA's first operand, so that the output lane
//     holds D[m = 4 (lane / 16) + r][n = lane % 16]: its weight row is the row
//     it decoded, and its weight scales stay in its own registers.
//
// LDS stage slot: codes BM rows x 128 bytes (16-byte unit u of row r at
// u ^ (r & 7)) | s [4 groups][BM] f32 | u [4][BM] f32 (Q4_K / Q5_K) | the
// weight pieces of the f16 prefill.
#include "common.h"
#include "internal.h"
#include "layout.h"
#include "mfma_dma.h"
#include "quant.h"

namespace fcg {

typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int I8_MROUND = 128;   // rows of the group-major scale arrays are padded to this
constexpr int I8_CWAVES = 4;     // compute waves (weight rows 32w .. 32w + 31), then the two loaders
constexpr int I8_THREADS = 64 * (I8_CWAVES + 2);
constexpr int I8_NTW = 2;        // 16-row weight sub-tiles per compute wave

// ----------------------------------------------------------- quantisation --

// One thread per 16-byte chunk of the rows m < Mp (the decode path's per-32
// routine, four lanes per group; rows past M quantise as zeros and store only
// their zero scales).
__global__ void __launch_bounds__(256)
quant_i8_kernel(const f16* __restrict__ A, int M, int K, int Mp, int8_t* __restrict__ qa,
                float* __restrict__ sT, float* __restrict__ uT) {
  constexpr int CV = chunk_vals<f16>(), GL = group_lanes<f16>();
  const int KC = K / CV;                                  // chunks per row
  const long long nch = (long long)Mp * KC;
  const long long c = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = c < nch;
  const int m = valid ? (int)(c / KC) : 0, kc = valid ? (int)(c % KC) : 0;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (valid && m < M) raw = *(const uint4*)(A + (size_t)m * K + (size_t)kc * CV);
  uint32_t q[2];
  float s;
  int tsum, thalf;
  quant_chunk<f16>(raw, q, s, tsum, thalf);               // every lane takes part
  if (!valid) return;
  if (m < M) *(uint2*)(qa + (size_t)m * K + (size_t)kc * CV) = make_uint2(q[0], q[1]);
  if (kc % GL == 0) {
    const int g = kc / GL;
    sT[(size_t)g * Mp + m] = s;
    uT[(size_t)g * Mp + m] = s * (float)tsum;
  }
}

// ----------------------------------------------------------- slot layout --

template <int QT, int MT>
struct I8Cfg {
  static constexpr int BM = 16 * MT;
  static constexpr int BN = 128;
  static constexpr bool HAS_U = QT != QT_Q6K;
  static constexpr int WP = QT == QT_Q4K ? 5 : 7;
  static constexpr int A_BYTES = BM * 128;          // codes
  static constexpr int S_OFF = A_BYTES;             // s [4][BM]
  static constexpr int U_OFF = S_OFF + 16 * BM;     // u [4][BM]
  static constexpr int W_OFF = U_OFF + (HAS_U ? 16 * BM : 0);
  static constexpr int W_BYTES = WP * BN * 16 + (QT == QT_Q6K ? BN * 4 : 0);
  static constexpr int SLOT = W_OFF + W_BYTES;
  static constexpr int LDS = DMA_SLOTS * SLOT;
  // loader instructions per stage: codes, then s (and u), 64 lanes each
  static constexpr int NI_CODES = BM * 8 / 64;
  static constexpr int NI_SC = (BM * 16 + 1023) / 1024;
  static constexpr int NI = NI_CODES + NI_SC * (HAS_U ? 2 : 1);
};

// Loader wave 4: the activation codes of the tile's BM rows (rows past M
// repeat row M - 1: loaded, never stored) and the stage's four group scales
// (and u) of every row, from the group-major arrays.
template <int QT, int MT>
__device__ __forceinline__ void i8_load_a(const int8_t* qa, const float* sT, const float* uT,
                                          int M, int K, int Mp, int m0, uint8_t* smem, int s_begin,
                                          int s_end, int rot) {
  using C = I8Cfg<QT, MT>;
  constexpr int NI = C::NI;
  const int lane = threadIdx.x & 63;
  const int nst = s_end - s_begin;
  auto issue = [&](int t) {
    const int s = dma_stage(t, s_begin, nst, rot);
    uint8_t* base = smem + (t % DMA_SLOTS) * C::SLOT;
#pragma unroll
    for (int k = 0; k < C::NI_CODES; ++k) {
      const int U = 64 * k + lane;                  // 16-byte unit of the slot's code area
      const int row = U >> 3, gu = (U & 7) ^ (row & 7);
      const int m = m0 + row < M ? m0 + row : M - 1;
      dma16(qa + (size_t)m * K + 128 * s + 16 * gu, base + 1024 * k);
    }
#pragma unroll
    for (int k = 0; k < C::NI_SC; ++k) {
      const int c = 64 * k + lane;                  // 4-float chunk: group c / (BM/4)
      if (c < C::BM) {
        const size_t off = (size_t)(4 * s + c / (C::BM / 4)) * Mp + m0 + 4 * (c % (C::BM / 4));
        dma16(sT + off, base + C::S_OFF + 1024 * k);
        if constexpr (C::HAS_U) dma16(uT + off, base + C::U_OFF + 1024 * k);
      }
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

// ------------------------------------------------------ int8 weight codes --

// The lane's 8 codes of k-step g (values 32g + 8kq .. +7 of its row within
// the half-block, the f16 decoders' lane mapping) as int8 bytes, and the f32
// scale factors of the k-step's sub-blocks.
struct Q45I8 {
  uint32_t a0, a1, b0, b1, qhx, qhy;
  float dsc[4];                     // d * sc_j of sub-blocks 4hb + g
  float ndmm;                       // -dmin * m_j of sub-block 4hb + kq (the lane's k quarter)

  template <bool HAS_QH>
  __device__ __forceinline__ void init(uint4 hdr, uint2 qsA, uint2 qsB, uint2 qh, int hb, int kq) {
    const uint32_t w0 = hdr.y, w1 = hdr.z, w2 = hdr.w;
    const uint32_t hi = 0u - (uint32_t)hb;
    const uint32_t scb = (w0 & 0x3F3F3F3Fu & ~hi) |
                         (((w2 & 0x0F0F0F0Fu) | ((w0 >> 2) & 0x30303030u)) & hi);
    const uint32_t mb = (w1 & 0x3F3F3F3Fu & ~hi) |
                        ((((w2 >> 4) & 0x0F0F0F0Fu) | ((w1 >> 2) & 0x30303030u)) & hi);
    const float d = h2f(hdr.x), dmin = h2f(hdr.x >> 16);
#pragma unroll
    for (int g = 0; g < 4; ++g) dsc[g] = d * (float)((scb >> (8 * g)) & 0xFF);
    ndmm = -dmin * (float)((mb >> (8 * kq)) & 0xFF);
    a0 = qsA.x; a1 = qsA.y; b0 = qsB.x; b1 = qsB.y;
    if constexpr (HAS_QH) {
      qhx = qh.x >> (4 * hb);
      qhy = qh.y >> (4 * hb);
    } else {
      qhx = qhy = 0;
    }
  }
  template <bool HAS_QH>
  __device__ __forceinline__ long codes(int g) const {
    const int sh = 4 * (g & 1);
    const uint32_t s0 = g < 2 ? a0 : b0, s1 = g < 2 ? a1 : b1;
    uint32_t c0 = (s0 >> sh) & 0x0F0F0F0Fu;
    uint32_t c1 = (s1 >> sh) & 0x0F0F0F0Fu;
    if constexpr (HAS_QH) {
      c0 |= (qhx << (4 - g)) & 0x10101010u;
      c1 |= (qhy << (4 - g)) & 0x10101010u;
    }
    return (long)(((uint64_t)c1 << 32) | c0);
  }
};

struct Q6I8 {
  uint32_t la0, la1, lb0, lb1, qhx, qhy;
  uint2 sc;                         // sc[8hb .. 8hb + 7] (int8)
  float d;

  __device__ __forceinline__ void init(uint2 qlA, uint2 qlB, uint2 qh, uint2 scv, uint32_t dbits) {
    la0 = qlA.x; la1 = qlA.y; lb0 = qlB.x; lb1 = qlB.y;
    qhx = qh.x;
    qhy = qh.y;
    sc = scv;
    d = h2f(dbits);
  }
  // codes q - 32 in [-32, 31] as int8
  __device__ __forceinline__ long codes(int g) const {
    const int sh = 4 * (g >> 1);
    const uint32_t s0 = (g & 1) ? lb0 : la0, s1 = (g & 1) ? lb1 : la1;
    const uint32_t hx = g < 3 ? (qhx << (4 - 2 * g)) : (qhx >> 2);
    const uint32_t hy = g < 3 ? (qhy << (4 - 2 * g)) : (qhy >> 2);
    uint32_t c0 = ((s0 >> sh) & 0x0F0F0F0Fu) | (hx & 0x30303030u);
    uint32_t c1 = ((s1 >> sh) & 0x0F0F0F0Fu) | (hy & 0x30303030u);
    // 6-bit q -> q - 32 as int8: flip bit 5, then copy it into bits 6 and 7
    c0 ^= 0x20202020u;
    c1 ^= 0x20202020u;
    c0 |= ((c0 & 0x20202020u) << 1) | ((c0 & 0x20202020u) << 2);
    c1 |= ((c1 & 0x20202020u) << 1) | ((c1 & 0x20202020u) << 2);
    return (long)(((uint64_t)c1 << 32) | c0);
  }
  // the scales of k-step g's two 16-value sub-blocks (2g: lanes kq < 2, 2g + 1)
  __device__ __forceinline__ int sc_lo(int g) const {
    return sext8((g < 2 ? sc.x : sc.y) >> (16 * (g & 1)));
  }
  __device__ __forceinline__ int sc_hi(int g) const {
    return sext8((g < 2 ? sc.x : sc.y) >> (16 * (g & 1) + 8));
  }
};

template <int QT> struct I8Dec { using type = Q6I8; };
template <> struct I8Dec<QT_Q5K> { using type = Q45I8; };
template <> struct I8Dec<QT_Q4K> { using type = Q45I8; };

// ------------------------------------------------------------ compute ------

// Compute waves 0-3: acc[i][j][r] = C[m = 16i + 4 (lane / 16) + r][n = 32w +
// 16j + lane % 16] of the tile, over the stages.
template <int QT, int MT>
__device__ __forceinline__ void i8_compute(int N, int K, int n0, const uint8_t* smem, int s_begin,
                                           int s_end, int rot, floatx4 (&acc)[MT][I8_NTW]) {
  (void)K;                                          // stages are counted by the caller
  constexpr int NTW = I8_NTW, BM = 16 * MT;
  using C = I8Cfg<QT, MT>;
  using Dec = typename I8Dec<QT>::type;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kq = lane >> 4, sub = 8 * (kq & 1), pq = kq >> 1;
  const int nst = s_end - s_begin;
  int nloc[NTW], rn[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    nloc[j] = wave * 16 * NTW + 16 * j + (lane & 15);
    const int n = n0 + nloc[j];
    rn[j] = n < N ? n : N - 1;                      // the row the loader fetched
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int4v zero = {0, 0, 0, 0};

  stage_barrier();                                  // stage 0 has landed
  for (int t = 0; t < nst; ++t) {
    const int s = dma_stage(t, s_begin, nst, rot);
    const int hb = s & 1;
    const uint8_t* As = smem + (t % DMA_SLOTS) * C::SLOT;
    const float* Ss = (const float*)(As + C::S_OFF);
    const float* Us = (const float*)(As + C::U_OFF);
    const uint8_t* Ws = As + C::W_OFF;
    Dec h[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      auto pc = [&](int q) { return Ws + (q * 128 + nloc[j]) * 16; };
      if constexpr (QT == QT_Q5K) {
        h[j].template init<true>(*(const uint4*)pc(0), *(const uint2*)(pc(3 + pq) + sub),
                                 *(const uint2*)(pc(5 + pq) + sub),
                                 *(const uint2*)(pc(1 + pq) + sub), hb, kq);
      } else if constexpr (QT == QT_Q4K) {
        h[j].template init<false>(*(const uint4*)pc(0), *(const uint2*)(pc(1 + pq) + sub),
                                  *(const uint2*)(pc(3 + pq) + sub), uint2{0u, 0u}, hb, kq);
      } else {
        // the row's half of its d word (tiled layout: rows n and n ^ 1 share it)
        const uint32_t dw = *(const uint32_t*)(Ws + C::WP * 128 * 16 + 4 * nloc[j]);
        h[j].init(*(const uint2*)(pc(pq) + sub), *(const uint2*)(pc(2 + pq) + sub),
                  *(const uint2*)(pc(4 + pq) + sub), *(const uint2*)(pc(6) + 8 * hb),
                  dw >> (16 * (rn[j] & 1)));
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      long w[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        if constexpr (QT == QT_Q6K) w[j] = h[j].codes(g);
        else w[j] = h[j].template codes<QT == QT_Q5K>(g);
      }
      // the k-step's activation codes and group scales, all read first
      long av[MT];
      floatx4 sv[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int r = 16 * i + (lane & 15);
        av[i] = *(const long*)(As + r * 128 + (((2 * g + pq) ^ (r & 7)) << 4) + sub);
        sv[i] = *(const floatx4*)(Ss + g * BM + 16 * i + 4 * kq);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const long a = av[i];
        const floatx4 s4 = sv[i];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          if constexpr (QT == QT_Q6K) {
            // the two 16-value sub-blocks: lanes kq < 2 hold the first
            const long wlo = kq < 2 ? w[j] : 0, whi = kq < 2 ? 0 : w[j];
            const int4v Slo = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, wlo, zero, 0, 0, 0);
            const int4v Shi = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, whi, zero, 0, 0, 0);
            const int clo = h[j].sc_lo(g), chi = h[j].sc_hi(g);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int I = __mul24(clo, Slo[q]) + __mul24(chi, Shi[q]);
              acc[i][j][q] = fmaf((float)I, s4[q] * h[j].d, acc[i][j][q]);
            }
          } else {
            const int4v S = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, w[j], zero, 0, 0, 0);
            const float dsc = h[j].dsc[g];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf((float)S[q], s4[q] * dsc, acc[i][j][q]);
          }
        }
      }
      // one scheduling region per k-step: the LDS reads, then each MFMA
      // followed by a share of the scale arithmetic
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * MT, 0);
#pragma unroll
      for (int k = 0; k < MT * NTW * (QT == QT_Q6K ? 2 : 1); ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, QT == QT_Q6K ? 7 : 12, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (QT != QT_Q6K) {
      // the min term of the stage's four groups is itself a small matrix
      // product, sum_g u[m][g] * (-dmin m_g)[n], one f32 MFMA (k = 4 groups)
      // per sub-tile: lane (row l % 16, group l / 16) gives u of activation
      // row 16i + l % 16 and -dmin * m of its own weight row
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const float u = Us[kq * BM + 16 * i + (lane & 15)];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(u, h[j].ndmm, acc[i][j], 0, 0, 0);
      }
    }
    compute_stage_barrier();                        // done reading this slot; next one landed
  }
}

// Store of a compute wave's sub-tiles: + R and one f16 rounding, or f32
// split-K partials P[split][M][N].
template <int MT>
__device__ __forceinline__ void i8_epilogue(const floatx4 (&acc)[MT][I8_NTW],
                                            const f16* R, f16* Y,
                                            float* __restrict__ P, int M, int N, int m0, int n0,
                                            int sp, int splits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = n0 + wave * 16 * I8_NTW + (lane & 15);
  // every residual first, then the stores: Y may be R, so the compiler would
  // otherwise wait for each residual load right before its store (each
  // element is read and written by its own lane only, so the early loads are
  // exact in place)
  f16 rr[MT][4][I8_NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < I8_NTW; ++j) {
        const int m = m0 + 16 * i + 4 * (lane >> 4) + q, nn = n + 16 * j;
        rr[i][q][j] = (R && splits == 1 && m < M && nn < N) ? R[(size_t)m * N + nn] : (f16)0.f;
      }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = m0 + 16 * i + 4 * (lane >> 4) + q;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < I8_NTW; ++j) {
        const int nn = n + 16 * j;
        if (nn >= N) continue;
        const float v = acc[i][j][q];
        if (splits > 1) P[((size_t)sp * M + m) * N + nn] = v;
        else Y[(size_t)m * N + nn] = (f16)(R ? v + (float)rr[i][q][j] : v);
      }
    }
}

template <int QT, int MT>
__global__ void __launch_bounds__(I8_THREADS)
prefill_i8_kernel(const uint8_t* W, const int8_t* qa, const float* sT, const float* uT,
                  const f16* R, f16* Y, float* __restrict__ P, int M,
                  int N, int K, int Mp, int tiles_m, int tiles_n, int splits,
                  int stages_per_split) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int BM = 16 * MT, BN = 128;
  int mt, sp, nt;
  // XCD-aware order, as the f16 prefill: m fastest, then split, then n
  {
    const int Gt = tiles_m * tiles_n * splits;
    int bid = blockIdx.x;
    const int per = Gt / 8, rem = Gt % 8, x = bid % 8, jj = bid / 8;
    bid = x * per + (x < rem ? x : rem) + jj;
    mt = bid % tiles_m;
    const int rest = bid / tiles_m;
    sp = rest % splits;
    nt = rest / splits;
  }
  const int m0 = mt * BM, n0 = nt * BN;
  const int S_total = K / KSTAGE;
  const int s_begin = sp * stages_per_split;
  int s_end = s_begin + stages_per_split;
  if (s_end > S_total) s_end = S_total;
  if (s_end < s_begin) s_end = s_begin;
  const int nst = s_end - s_begin;
  const int rot = nst > 0 ? (nt + mt) % nst : 0;
  const int wave = threadIdx.x >> 6;
  if (wave == I8_CWAVES) {
    i8_load_a<QT, MT>(qa, sT, uT, M, K, Mp, m0, smem, s_begin, s_end, rot);
    return;
  }
  if (wave == I8_CWAVES + 1) {
    dma_load_w<QT, MT, I8Cfg<QT, MT>>(W, N, K, n0, smem, s_begin, s_end, rot);
    return;
  }
  floatx4 acc[MT][I8_NTW];
  i8_compute<QT, MT>(N, K, n0, smem, s_begin, s_end, rot, acc);
  i8_epilogue<MT>(acc, R, Y, P, M, N, m0, n0, sp, splits);
}

// ------------------------------------------------------------------ launch --

size_t prefill_i8_workspace_bytes(int M, int N, int K, int splits) {
  const size_t Mp = (size_t)(M + I8_MROUND - 1) / I8_MROUND * I8_MROUND;
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  return al(Mp * K) + 2 * al(Mp * (K / 32) * sizeof(float)) +
         (splits > 1 ? al((size_t)splits * M * N * sizeof(float)) : 0);
}

template <int QT, int MT>
static hipError_t launch_i8_t(const uint8_t* W, const int8_t* qa, const float* sT, const float* uT,
                              const f16* R, f16* Y, float* P, int M, int N, int K, int Mp,
                              int splits, hipStream_t st) {
  constexpr int BM = 16 * MT, BN = 128;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int S_total = K / KSTAGE;
  const int per = (S_total + splits - 1) / splits;
  const int grid = tiles_m * tiles_n * splits;
  constexpr int lds = I8Cfg<QT, MT>::LDS;
  static_assert(lds <= 160 * 1024, "LDS ring");
  static std::atomic<uint64_t> lds_raised{0};
  hipError_t ea = raise_lds_limit((const void*)prefill_i8_kernel<QT, MT>, lds, lds_raised);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL((prefill_i8_kernel<QT, MT>), dim3(grid), dim3(I8_THREADS), lds, st, W, qa, sT,
                     uT, R, Y, P, M, N, K, Mp, tiles_m, tiles_n, splits, per);
  return hipGetLastError();
}

hipError_t launch_prefill_i8(int qtype, const uint8_t* W, const f16* A, const f16* R, f16* Y,
                             void* ws, int M, int N, int K, int mt, int splits, hipStream_t st) {
  const int Mp = (M + I8_MROUND - 1) / I8_MROUND * I8_MROUND;
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  uint8_t* p = (uint8_t*)ws;
  int8_t* qa = (int8_t*)p;
  p += al((size_t)Mp * K);
  float* sT = (float*)p;
  p += al((size_t)Mp * (K / 32) * sizeof(float));
  float* uT = (float*)p;
  p += al((size_t)Mp * (K / 32) * sizeof(float));
  float* P = splits > 1 ? (float*)p : nullptr;
  {
    const long long chunks = (long long)Mp * (K / chunk_vals<f16>());
    hipLaunchKernelGGL(quant_i8_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, A,
                       M, K, Mp, qa, sT, uT);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipErrorInvalidValue;
#define FCG_I8(QT_, MT_) \
  if (qtype == QT_ && mt == MT_) e = launch_i8_t<QT_, MT_>(W, qa, sT, uT, R, Y, P, M, N, K, Mp, splits, st);
  FCG_I8(QT_Q4K, 1) FCG_I8(QT_Q4K, 2) FCG_I8(QT_Q4K, 4) FCG_I8(QT_Q4K, 8)
  FCG_I8(QT_Q5K, 1) FCG_I8(QT_Q5K, 2) FCG_I8(QT_Q5K, 4) FCG_I8(QT_Q5K, 8)
  FCG_I8(QT_Q6K, 1) FCG_I8(QT_Q6K, 2) FCG_I8(QT_Q6K, 4) FCG_I8(QT_Q6K, 8)
#undef FCG_I8
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(P, R, Y, (long long)M * N, splits, st);
}

}  // namespace fcg
