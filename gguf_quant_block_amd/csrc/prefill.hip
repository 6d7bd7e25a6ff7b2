// Prefill path (M >= 8): f16 matrix-core FC on raw Q5_K / Q6_K blocks.
//
// OpenVINO PR #39119, section Implementation: each 256-value weight block is
// decoded once into on-chip memory and reused across many activation rows,
// loads and decode are double-buffered, and the tile grows with the number of
// rows; the residual Add is fused into the output store.
//
// gfx950 design (one workgroup = 4 waves, tile BM x BN, BM = 16*MT activation
// rows, BN = 64*NT weight rows, K walked in half super-blocks of 128 values):
//   * The activation tile [BM x 128] f16 is staged global -> registers -> LDS,
//     double-buffered: the next stage's loads are in flight while the current
//     stage runs on the matrix cores.
//   * Each wave owns 16*NT weight rows.  Its lanes load those rows' raw block
//     bytes for the next stage (prefetched one stage ahead) and decode them
//     straight into the v_mfma_f32_16x16x32_f16 operand registers: each weight
//     value is decoded exactly once per workgroup and then reused across all
//     BM activation rows.  Decoding is exact up to one f16 rounding:
//       magic f16 (1024 + q) from a byte permute, t = fma(1024+q, sc, -1024*sc
//       [Q6_K: -1056*sc]) = sc*q [sc*(q-32)] exactly, then w = t*d - dmin*m
//       [Q6_K: t*d] with a single rounding.
//   * f32 accumulation; epilogue adds R once and rounds to f16, or writes f32
//     partials for a split-K reduction when the tile grid is too small to fill
//     the 256 compute units.
//   * Tile ids are remapped so that the workgroups sharing weight columns land
//     on the same XCD (one L2 per XCD).
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace fcg {

constexpr int KSTAGE = 128;          // values of K per stage (half super-block)
constexpr int ASTR = KSTAGE + 8;     // LDS row stride in halves (pad 16 B)

struct RawQ5 {  // one lane, one row, one half-block
  uint4 hdr;    // d | dmin, scales[0..3], scales[4..7], scales[8..11]
  uint2 qsA;    // qs[64hb + 8kq .. +8]      : sub-blocks 4hb+0 (lo), 4hb+1 (hi)
  uint2 qsB;    // qs[64hb + 32 + 8kq .. +8] : sub-blocks 4hb+2 (lo), 4hb+3 (hi)
  uint2 qh;     // qh[8kq .. +8]
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

// Decode the lane's 4 x 8 weights of one half-block (k-step g = 0..3 covers
// values 128hb + 32g + 8kq .. +7 of its row).
__device__ __forceinline__ void decode_q5k_half(const RawQ5& r, int hb, half8v out[4]) {
  const uint32_t w0 = r.hdr.y, w1 = r.hdr.z, w2 = r.hdr.w;
  uint32_t scb, mb;   // bytes g = 0..3: scale / min of sub-block 4hb + g
  if (hb == 0) {
    scb = w0 & 0x3F3F3F3Fu;
    mb = w1 & 0x3F3F3F3Fu;
  } else {
    scb = (w2 & 0x0F0F0F0Fu) | ((w0 >> 2) & 0x30303030u);
    mb = ((w2 >> 4) & 0x0F0F0F0Fu) | ((w1 >> 2) & 0x30303030u);
  }
  const f16 d = __builtin_bit_cast(f16, (uint16_t)(r.hdr.x & 0xFFFF));
  const float dmin = h2f(r.hdr.x >> 16);
  const half2v d2 = splat(d);
  const uint32_t src[4] = {r.qsA.x, r.qsA.x, r.qsB.x, r.qsB.x};
  const uint32_t src1[4] = {r.qsA.y, r.qsA.y, r.qsB.y, r.qsB.y};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int sh = 4 * (g & 1);
    const int j = 4 * hb + g;
    const uint32_t c0 = ((src[g] >> sh) & 0x0F0F0F0Fu) | (((r.qh.x >> j) & 0x01010101u) << 4);
    const uint32_t c1 = ((src1[g] >> sh) & 0x0F0F0F0Fu) | (((r.qh.y >> j) & 0x01010101u) << 4);
    const int sc = (scb >> (8 * g)) & 0xFF;
    const int mn = (mb >> (8 * g)) & 0xFF;
    const f16 scf = (f16)(float)sc;
    const half2v sc2 = splat(scf);
    const half2v bias2 = splat((f16)(float)(-1024 * sc));
    const half2v negdmm2 = splat((f16)(-(dmin * (float)mn)));
    out[g] = decode8(c0, c1, sc2, bias2, d2, negdmm2);
  }
}

__device__ __forceinline__ void decode_q6k_half(const RawQ6& r, int kq, half8v out[4]) {
  const f16 d = __builtin_bit_cast(f16, (uint16_t)(r.d & 0xFFFF));
  const half2v d2 = splat(d);
  const half2v zero2 = splat((f16)0.f);
  const uint32_t srcx[4] = {r.qlA.x, r.qlB.x, r.qlA.x, r.qlB.x};
  const uint32_t srcy[4] = {r.qlA.y, r.qlB.y, r.qlA.y, r.qlB.y};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int sh = 4 * (g >> 1);
    const uint32_t c0 = ((srcx[g] >> sh) & 0x0F0F0F0Fu) | (((r.qh.x >> (2 * g)) & 0x03030303u) << 4);
    const uint32_t c1 = ((srcy[g] >> sh) & 0x0F0F0F0Fu) | (((r.qh.y >> (2 * g)) & 0x03030303u) << 4);
    // sub-block of values 32g + 8kq .. +7 within the half: 2g + kq/2
    const int si = 2 * g + (kq >> 1);
    const uint32_t scw = si < 4 ? r.sc.x : r.sc.y;
    const int sc = sext8(scw >> (8 * (si & 3)));
    const half2v sc2 = splat((f16)(float)sc);
    const half2v bias2 = splat((f16)(float)(-1056 * sc));
    out[g] = decode8(c0, c1, sc2, bias2, d2, zero2);
  }
}

template <int QT, int MT, int NT>
__global__ void __launch_bounds__(256)
prefill_kernel(const uint8_t* __restrict__ W, const f16* __restrict__ A, const f16* __restrict__ R,
               f16* __restrict__ Y, float* __restrict__ P, int M, int N, int K, int tiles_m,
               int tiles_n, int splits, int stages_per_split) {
  constexpr int BM = 16 * MT;
  constexpr int BN = 64 * NT;
  __shared__ __align__(16) f16 As[2][BM * ASTR];

  // XCD-aware remap: the hardware deals workgroups round-robin over 8 XCDs;
  // give each XCD a contiguous run of logical tiles (m fastest, then split,
  // then n) so tiles sharing weight columns share an L2.
  const int Gt = tiles_m * tiles_n * splits;
  int bid = blockIdx.x;
  {
    const int per = Gt / 8, rem = Gt % 8, x = bid % 8, j = bid / 8;
    bid = x * per + (x < rem ? x : rem) + j;
  }
  const int mt = bid % tiles_m;
  const int rest = bid / tiles_m;
  const int sp = rest % splits;
  const int nt = rest / splits;
  const int m0 = mt * BM, n0 = nt * BN;
  const int S_total = K / KSTAGE;
  const int s_begin = sp * stages_per_split;
  int s_end = s_begin + stages_per_split;
  if (s_end > S_total) s_end = S_total;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kq = lane >> 4;
  const int KB = K >> 8;
  const size_t nblk = (size_t)N * KB;

  // rows of this lane's weight fragments
  int nrow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) nrow[j] = n0 + wave * 16 * NT + 16 * j + (lane & 15);

  auto load_raw_q5 = [&](int s, RawQ5* raw) {
    const int kb = s >> 1, hb = s & 1;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (nrow[j] < N) {
        const uint8_t* blk = W + ((size_t)nrow[j] * KB + kb) * Q5K_BYTES;
        raw[j].hdr = *(const uint4*)blk;
        raw[j].qsA = *(const uint2*)(blk + 48 + 64 * hb + 8 * kq);
        raw[j].qsB = *(const uint2*)(blk + 80 + 64 * hb + 8 * kq);
        raw[j].qh = *(const uint2*)(blk + 16 + 8 * kq);
      } else {
        raw[j].hdr = make_uint4(0, 0, 0, 0);
        raw[j].qsA = raw[j].qsB = raw[j].qh = make_uint2(0, 0);
      }
    }
  };
  auto load_raw_q6 = [&](int s, RawQ6* raw) {
    const int kb = s >> 1, hb = s & 1;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (nrow[j] < N) {
        const size_t b = (size_t)nrow[j] * KB + kb;
        raw[j].qlA = *(const uint2*)(W + 128 * b + 64 * hb + 8 * kq);
        raw[j].qlB = *(const uint2*)(W + 128 * b + 64 * hb + 32 + 8 * kq);
        raw[j].qh = *(const uint2*)(W + 128 * nblk + 64 * b + 32 * hb + 8 * kq);
        raw[j].sc = *(const uint2*)(W + 192 * nblk + 16 * b + 8 * hb);
        raw[j].d = *(const uint16_t*)(W + 208 * nblk + 2 * b);
      } else {
        raw[j].qlA = raw[j].qlB = raw[j].qh = raw[j].sc = make_uint2(0, 0);
        raw[j].d = 0;
      }
    }
  };

  // activation stage: BM rows x 128 halves = BM*16 chunks of 16 B, MT per thread
  uint4 areg[MT];
  auto load_a = [&](int s) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 4, col = c & 15;
      const int m = m0 + row;
      if (m < M)
        areg[i] = *(const uint4*)(A + (size_t)m * K + (size_t)s * KSTAGE + 8 * col);
      else
        areg[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 4, col = c & 15;
      *(uint4*)(&As[buf][row * ASTR + 8 * col]) = areg[i];
    }
  };

  floatx4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  using Raw = typename std::conditional<QT == QT_Q5K, RawQ5, RawQ6>::type;
  Raw rawc[NT], rawn[NT];

  if (s_begin < s_end) {
    load_a(s_begin);
    if constexpr (QT == QT_Q5K) load_raw_q5(s_begin, rawc); else load_raw_q6(s_begin, rawc);
    store_a(0);
  }
  __syncthreads();

  for (int s = s_begin; s < s_end; ++s) {
    const int buf = (s - s_begin) & 1;
    const bool more = s + 1 < s_end;
    if (more) {
      load_a(s + 1);
      if constexpr (QT == QT_Q5K) load_raw_q5(s + 1, rawn); else load_raw_q6(s + 1, rawn);
    }
    // decode this stage's weight fragments: wf[j][g]
    half8v wf[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if constexpr (QT == QT_Q5K) decode_q5k_half(rawc[j], s & 1, wf[j]);
      else decode_q6k_half(rawc[j], kq, wf[j]);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      half8v af[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[i] = *(const half8v*)(&As[buf][(16 * i + (lane & 15)) * ASTR + 32 * g + 8 * kq]);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[j][g], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_a(buf ^ 1);
#pragma unroll
      for (int j = 0; j < NT; ++j) rawc[j] = rawn[j];
    }
    __syncthreads();
  }

  // epilogue: lane holds C[n = 4*(lane>>4) + r][m = lane & 15] of each 16x16 tile
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = m0 + 16 * i + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = n0 + wave * 16 * NT + 16 * j + 4 * kq;
      if (n >= N) continue;
      const floatx4 v = acc[i][j];
      if (splits > 1) {
        float* dst = P + ((size_t)sp * M + m) * N + n;
        if (n + 3 < N && ((N & 3) == 0)) {
          *(floatx4*)dst = v;
        } else {
          for (int r = 0; r < 4 && n + r < N; ++r) dst[r] = v[r];
        }
      } else {
        f16* dst = Y + (size_t)m * N + n;
        if (n + 3 < N && ((N & 3) == 0)) {
          float y[4] = {v[0], v[1], v[2], v[3]};
          if (R) {
            const uint2 rr = *(const uint2*)(R + (size_t)m * N + n);
            y[0] += h2f(rr.x); y[1] += h2f(rr.x >> 16);
            y[2] += h2f(rr.y); y[3] += h2f(rr.y >> 16);
          }
          uint2 o;
          o.x = (uint32_t)f2h_bits(y[0]) | ((uint32_t)f2h_bits(y[1]) << 16);
          o.y = (uint32_t)f2h_bits(y[2]) | ((uint32_t)f2h_bits(y[3]) << 16);
          *(uint2*)dst = o;
        } else {
          for (int r = 0; r < 4 && n + r < N; ++r) {
            float y = v[r];
            if (R) y += (float)R[(size_t)m * N + n + r];
            dst[r] = (f16)y;
          }
        }
      }
    }
  }
}

// Y = sum over splits of P + R, rounded once to f16.
__global__ void splitk_reduce_kernel(const float* __restrict__ P, const f16* __restrict__ R,
                                     f16* __restrict__ Y, long long MN, int splits) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= MN) return;
  float y = 0.f;
  for (int s = 0; s < splits; ++s) y += P[(size_t)s * MN + i];
  if (R) y += (float)R[i];
  Y[i] = (f16)y;
}

template <int QT, int MT, int NT>
static hipError_t launch_prefill_t(const uint8_t* W, const f16* A, const f16* R, f16* Y, float* P,
                                   int M, int N, int K, int splits, hipStream_t st) {
  constexpr int BM = 16 * MT, BN = 64 * NT;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int S_total = K / KSTAGE;
  const int per = (S_total + splits - 1) / splits;
  const int grid = tiles_m * tiles_n * splits;
  hipLaunchKernelGGL((prefill_kernel<QT, MT, NT>), dim3(grid), dim3(256), 0, st, W, A, R, Y, P, M,
                     N, K, tiles_m, tiles_n, splits, per);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const long long MN = (long long)M * N;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, st, P,
                     R, Y, MN, splits);
  return hipGetLastError();
}

void prefill_choose(int qtype, int M, int N, int K, int num_cu, int* mt, int* nt, int* splits) {
  (void)qtype;
  // tile rows grow with M: 16, 32, 64, 128
  int t = 1;
  while (t < 8 && 16 * t < M) t *= 2;
  *mt = t;
  *nt = 2;
  const int BM = 16 * t, BN = 128;
  const long long tiles = (long long)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int S_total = K / KSTAGE;
  int s = 1;
  // split K only while the grid is under one workgroup per CU and every
  // split keeps at least 4 stages
  while (tiles * s < num_cu && S_total / (s * 2) >= 4) s *= 2;
  *splits = s;
}

size_t prefill_workspace_bytes(int M, int N, int splits) {
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

hipError_t launch_prefill(int qtype, const uint8_t* W, const f16* A, const f16* R, f16* Y, float* P,
                          int M, int N, int K, int mt, int nt, int splits, hipStream_t st) {
#define FCG_PF(QT_, MT_, NT_)                                                   \
  if (mt == MT_ && nt == NT_) return launch_prefill_t<QT_, MT_, NT_>(W, A, R, Y, P, M, N, K, splits, st);
  if (qtype == QT_Q5K) {
    FCG_PF(QT_Q5K, 1, 2) FCG_PF(QT_Q5K, 2, 2) FCG_PF(QT_Q5K, 4, 2) FCG_PF(QT_Q5K, 8, 2)
  } else {
    FCG_PF(QT_Q6K, 1, 2) FCG_PF(QT_Q6K, 2, 2) FCG_PF(QT_Q6K, 4, 2) FCG_PF(QT_Q6K, 8, 2)
  }
#undef FCG_PF
  return hipErrorInvalidValue;
}

}  // namespace fcg
