// Prefill path (M >= 8): f16 matrix-core FC on raw Q4_K / Q5_K / Q6_K blocks.
//
// OpenVINO PR #39119, section Implementation: each 256-value weight block is
// decoded once into on-chip memory and reused across many activation rows,
// loads and decode are double-buffered, and the tile grows with the number of
// rows; the residual Add is fused into the output store.
//
// gfx950 design: the loader-wave tile (mfma_dma.h) over a dense range of BM
// activation rows; the epilogue adds R once and rounds to f16, or writes f32
// partials for a split-K reduction when the tile grid is too small to fill
// the 256 compute units.  Tile ids are remapped so that the workgroups
// sharing weight columns land on the same XCD (one L2 per XCD).  This file
// also holds the decode-once LDS tile (mfma_lds.h, forced only) and the
// plan that picks between them and the few-row kernel of skinny.hip, which
// takes M <= 32 rows whenever they fit its LDS.
#include "common.h"
#include "internal.h"

#include <type_traits>
#include "mfma_tile.h"
#include "mfma_dma.h"
#include "mfma_lds.h"


namespace fcg {

static_assert(PREFILL_KSTAGE == KSTAGE, "the host and the tile agree on the stage size");

// Epilogue of a wave's sub-tiles: lane holds C[n = 4*(lane>>4) + r][m = lane & 15]
// of each 16x16 sub-tile (i, j), whose first row is m0 + 16 i and first
// column n0 + 16 j; + R and one f16 rounding, or f32 split-K partials.
template <int MT, int NT>
__device__ __forceinline__ void prefill_epilogue(const floatx4 (&acc)[MT][NT],
                                                 const f16* R, f16* Y,
                                                 float* __restrict__ P, int M, int N, int m0,
                                                 int n0, int sp, int splits) {
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4;
  if (splits > 1) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + 16 * i + (lane & 15);
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int n = n0 + 16 * j + 4 * kq;
        if (n >= N) continue;
        const floatx4 v = acc[i][j];
        float* dst = P + ((size_t)sp * M + m) * N + n;
        if (n + 3 < N && ((N & 3) == 0)) *(floatx4*)dst = v;
        else for (int r = 0; r < 4 && n + r < N; ++r) dst[r] = v[r];
      }
    }
    return;
  }
  // every residual first, then the stores (load4_r)
  uint2 rr[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int m = m0 + 16 * i + (lane & 15), n = n0 + 16 * j + 4 * kq;
      rr[i][j] = (R && m < M && n < N) ? load4_r(R + (size_t)m * N, n, N) : make_uint2(0u, 0u);
    }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = m0 + 16 * i + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = n0 + 16 * j + 4 * kq;
      if (n < N) store4_y(Y + (size_t)m * N, n, N, acc[i][j], rr[i][j], R != nullptr);
    }
  }
}

// Tile index of this workgroup.  XCD-aware remap: the hardware deals
// workgroups round-robin over 8 XCDs; give each XCD a contiguous run of
// logical tiles (m fastest, then n, then split), so that the tiles sharing
// weight rows share an L2 and, in a split-K grid, an XCD reads the
// activations of one part of K only.  (Split before n made every XCD read
// all of A: [2048, 8192] at M = 512 then filled its L2s with 5x the
// algorithmic bytes.)
__device__ __forceinline__ void prefill_tile_id(int tiles_m, int tiles_n, int splits, int& mt,
                                                int& sp, int& nt) {
  const int Gt = tiles_m * tiles_n * splits;
  int bid = blockIdx.x;
  const int per = Gt / 8, rem = Gt % 8, x = bid % 8, j = bid / 8;
  bid = x * per + (x < rem ? x : rem) + j;
  mt = bid % tiles_m;
  const int rest = bid / tiles_m;
  nt = rest % tiles_n;
  sp = rest / tiles_n;
}

// The matrix-core tile with loader waves and an LDS ring (mfma_dma.h).
template <int QT, int MT>
__global__ void __launch_bounds__(DMA_THREADS)
prefill_dma_kernel(const uint8_t* W, const f16* A, const f16* R, f16* Y,
                   float* __restrict__ P, int M, int N, int K, int tiles_m,
                   int tiles_n, int splits, int stages_per_split) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int BM = 16 * MT, BN = 128;
  int mt, sp, nt;
  prefill_tile_id(tiles_m, tiles_n, splits, mt, sp, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int S_total = K / KSTAGE;
  const int s_begin = sp * stages_per_split;
  int s_end = s_begin + stages_per_split;
  if (s_end > S_total) s_end = S_total;
  if (s_end < s_begin) s_end = s_begin;
  const int nst = s_end - s_begin;
  // workgroups sharing activation or weight rows start at different stages
  const int rot = nst > 0 ? (nt + mt) % nst : 0;
  const int wave = dma_role();
  if (wave >= DMA_CWAVES && wave < DMA_CWAVES + DMA_ALOADERS) {
    auto arow = [&](int r) {
      int m = m0 + r;
      m = m < M ? m : M - 1;
      return A + (size_t)m * K;
    };
    dma_load_a<QT, MT, MT>(arow, smem, s_begin, s_end, rot, wave - DMA_CWAVES);
    return;
  }
  if (wave == DMA_CWAVES + DMA_ALOADERS) {
    dma_load_w<QT, MT>(W, N, K, n0, smem, s_begin, s_end, rot);
    return;
  }
  floatx4 acc[MT][DMA_NTW];
  dma_compute<QT, MT, MT>(N, K, n0, smem, s_begin, s_end, rot, acc);
  prefill_epilogue<MT, DMA_NTW>(acc, R, Y, P, M, N, m0, n0 + wave * 16 * DMA_NTW, sp, splits);
}

// The decode-once tile of mfma_lds.h: 128 activation rows x 128 weight rows,
// K in stages of 64 values, super-block aligned splits of K.  Tile ids: split
// slowest, then the weight-row tile, then the activation-row tile, each XCD
// taking a contiguous run (the hardware deals workgroups round-robin over 8
// XCDs), so that the workgroups sharing a weight-row tile share an L2 and
// each XCD reads only its splits' share of the activations.
template <int QT>
__global__ void __launch_bounds__(LT_THREADS)
prefill_lds_kernel(const uint8_t* W, const f16* A, const f16* R, f16* Y, float* __restrict__ P,
                   int M, int N, int K, int tiles_m, int tiles_n, int splits, int sb_per_split) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int Gt = tiles_m * tiles_n * splits;
  int bid = blockIdx.x;
  {
    const int per = Gt / 8, rem = Gt % 8, x = bid % 8, j = bid / 8;
    bid = x * per + (x < rem ? x : rem) + j;
  }
  const int mt = bid % tiles_m;
  const int rest = bid / tiles_m;
  const int nt = rest % tiles_n, sp = rest / tiles_n;
  const int m0 = mt * LT_BM, n0 = nt * LT_BN;
  const int KB = K >> 8;
  const int kb0 = sp * sb_per_split;
  const int kb1 = kb0 + sb_per_split < KB ? kb0 + sb_per_split : KB;
  const int nst = 4 * (kb1 - kb0);                  // >= 4: the host leaves no split empty
  // start stage (super-block aligned): differs between the weight-row tiles
  // of an XCD, which share the activation rows
  const int rot = 4 * (nt % (nst >> 2));
  // Hardware wave 0 is the loader, waves 1..8 the consumers and 9..12 the
  // producers: the consumers are older than the producers, so that when both
  // have an instruction ready the matrix-core work issues first (ties in
  // issue arbitration go to the older wave) and the decode fills the gaps.
  const int w = threadIdx.x >> 6;
  if (w == 0) {
    lt_loader(A, M, K, m0, kb0 * QK, smem, nst, rot);
    stage_barrier();                                // the consumers' partial-sum hand-off
    return;
  }
  if (w >= 9) {
    lt_producer<QT>(W, N, K, n0, kb0, smem, nst, rot, w - 9);
    stage_barrier();
    return;
  }
  const int c = w - 1;
  floatx16 acc[2][2];
  lt_consumer(smem, nst, c, acc);
  lt_pair_sum(smem, c, acc);
  if (c >= 4) return;
  // lane l, register v of block (a, b): n = 8 (v / 4) + 4 (l / 32) + v % 4,
  // m = l % 32 within the block
  const int lane = threadIdx.x & 63;
  auto row = [&](int b) { return m0 + 64 * (c & 1) + 32 * b + (lane & 31); };
  auto col = [&](int a, int q) { return n0 + 64 * (c >> 1) + 32 * a + 8 * q + 4 * (lane >> 5); };
  if (splits > 1) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int m = row(b);
      if (m >= M) continue;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = col(a, q);
          if (n >= N) continue;
          const floatx4 v = {acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                             acc[a][b][4 * q + 3]};
          float* dst = P + ((size_t)sp * M + m) * N + n;
          if (n + 3 < N && ((N & 3) == 0)) *(floatx4*)dst = v;
          else for (int r = 0; r < 4 && n + r < N; ++r) dst[r] = v[r];
        }
    }
    return;
  }
  // every residual first, then the stores (load4_r)
  uint2 rr[2][2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = row(b), n = col(a, q);
        rr[b][a][q] = (R && m < M && n < N) ? load4_r(R + (size_t)m * N, n, N) : make_uint2(0u, 0u);
      }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int m = row(b);
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = col(a, q);
        if (n >= N) continue;
        const floatx4 v = {acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                           acc[a][b][4 * q + 3]};
        store4_y(Y + (size_t)m * N, n, N, v, rr[b][a][q], R != nullptr);
      }
  }
}

// Y = sum over splits of P + R, rounded once to f16.  V consecutive outputs
// per thread (4 when M*N is a multiple of 4: 16-byte partial loads, 8-byte
// R and Y accesses).  The partial sums are added in split order, so the
// result does not depend on V; each thread issues the loads of up to eight
// splits before adding them, so that their latencies overlap.
template <int V>
__global__ void splitk_reduce_kernel(const float* __restrict__ P, const f16* R, f16* Y, long long MN, int splits) {
  constexpr int U = 8;                              // splits in flight per thread
  const long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (i >= MN) return;
  using PT = typename std::conditional<V == 4, float4, float>::type;
  float y[V];
#pragma unroll
  for (int v = 0; v < V; ++v) y[v] = 0.f;
  for (int s0 = 0; s0 < splits; s0 += U) {
    PT p[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + u < splits) p[u] = *(const PT*)(P + (size_t)(s0 + u) * MN + i);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < splits) {
        const float* pu = (const float*)&p[u];
#pragma unroll
        for (int v = 0; v < V; ++v) y[v] += pu[v];
      }
    }
  }
  if constexpr (V == 4) {
    if (R) {
      const uint2 r = *(const uint2*)(R + i);
      const f16* rh = (const f16*)&r;
#pragma unroll
      for (int v = 0; v < 4; ++v) y[v] += (float)rh[v];
    }
    f16 o[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) o[v] = (f16)y[v];
    *(uint2*)(Y + i) = *(const uint2*)o;
  } else {
    if (R) y[0] += (float)R[i];
    Y[i] = (f16)y[0];
  }
}

hipError_t launch_splitk_reduce(const float* P, const f16* R, f16* Y, long long MN, int splits,
                                hipStream_t st) {
  if (MN % 4 == 0) {
    const long long n = MN / 4;
    hipLaunchKernelGGL(splitk_reduce_kernel<4>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       P, R, Y, MN, splits);
  } else {
    hipLaunchKernelGGL(splitk_reduce_kernel<1>, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, st,
                       P, R, Y, MN, splits);
  }
  return hipGetLastError();
}

template <int QT, int MT>
static hipError_t launch_dma_t(const uint8_t* W, const f16* A, const f16* R, f16* Y, float* P,
                               int M, int N, int K, int splits, hipStream_t st) {
  constexpr int BM = 16 * MT, BN = 128;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const int S_total = K / KSTAGE;
  const int per = (S_total + splits - 1) / splits;
  const int grid = tiles_m * tiles_n * splits;
  constexpr int lds = DmaCfg<QT, MT>::LDS;
  static std::atomic<uint64_t> lds_raised{0};
  hipError_t ea = raise_lds_limit((const void*)prefill_dma_kernel<QT, MT>, lds, lds_raised);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL((prefill_dma_kernel<QT, MT>), dim3(grid), dim3(DMA_THREADS), lds, st, W, A, R,
                     Y, P, M, N, K, tiles_m, tiles_n, splits, per);
  return hipGetLastError();
}

template <int QT>
static hipError_t launch_lds_t(const uint8_t* W, const f16* A, const f16* R, f16* Y, float* P,
                               int M, int N, int K, int splits, int sb_per, hipStream_t st) {
  const int tiles_m = (M + LT_BM - 1) / LT_BM;
  const int tiles_n = (N + LT_BN - 1) / LT_BN;
  const int grid = tiles_m * tiles_n * splits;
  static std::atomic<uint64_t> lds_raised{0};
  hipError_t ea = raise_lds_limit((const void*)prefill_lds_kernel<QT>, LT_LDS, lds_raised);
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL((prefill_lds_kernel<QT>), dim3(grid), dim3(LT_THREADS), LT_LDS, st, W, A, R, Y,
                     P, M, N, K, tiles_m, tiles_n, splits, sb_per);
  return hipGetLastError();
}

// The loader-wave tile's row count and K splits for M rows (also the int8
// variant's tile).  Candidates: 16, 32, 64 or 128 activation rows (up to the
// first tile that covers M) and K in 1, 2, 4, ... parts of at least 4 stages
// each.  The choice minimises an estimate of the launch time fitted to
// measurements of this kernel on MI355X: one workgroup per CU at a time, so
// ceil(tiles * splits / CUs) rounds of S / splits stages, a stage costing
// about 0.8 us + 0.0075 us per activation row of the tile; a split adds the
// f32 partials' round trip (8 bytes per partial element at about 4 TB/s) and
// about 2 us for the reduction launch.  Splitting only fills CUs that the
// tile grid leaves idle; a smaller tile fills them too, at the price of
// decoding each weight block once per tile row.
void prefill_choose(int qtype, int M, int N, int K, int num_cu, int* mt, int* nt, int* splits) {
  (void)qtype;
  int tmax = 1;
  while (tmax < 8 && 16 * tmax < M) tmax *= 2;
  const int S_total = K / KSTAGE;
  const long long tiles_n = (N + 127) / 128;
  const int cus = num_cu > 0 ? num_cu : 1;
  double best = 0.0;
  int bt = tmax, bs = 1;
  for (int t = 1; t <= tmax; t *= 2) {
    const long long tiles = (long long)((M + 16 * t - 1) / (16 * t)) * tiles_n;
    for (int s = 1; s == 1 || S_total / s >= 4; s *= 2) {
      const long long rounds = (tiles * s + cus - 1) / cus;
      double cost = (double)rounds * ((double)S_total / s) * (0.8 + 0.0075 * 16 * t);
      if (s > 1) cost += 2.0 + (double)s * M * N * 8.0 / 4.0e6;
      if ((t == 1 && s == 1) || cost < best) {
        best = cost;
        bt = t;
        bs = s;
      }
    }
  }
  *mt = bt;
  *nt = 2;
  *splits = bs;
}

PrefillPlan prefill_plan(int qtype, int M, int N, int K, int num_cu, int kernel) {
  PrefillPlan p{};
  // the few-row kernel wherever its rows fit (faster than the loader-wave
  // tile at every such row count on the benchmark shapes), unless a tile is
  // forced
  if ((kernel == PREFILL_KERNEL_SKINNY || kernel == PREFILL_KERNEL_AUTO) && skinny_fits(M, K)) {
    p.kind = PREFILL_KERNEL_SKINNY;
    p.mt = M > 16 ? 2 : 1;
    p.splits = 1;
    p.wgs = skinny_max_wgs(M, K, num_cu);
    return p;
  }
  const bool lds = kernel == PREFILL_KERNEL_LDS;
  if (!lds) {
    int nt;
    prefill_choose(qtype, M, N, K, num_cu, &p.mt, &nt, &p.splits);
    p.kind = PREFILL_KERNEL_DMA;
    p.sb_per = 0;
    return p;
  }
  p.kind = PREFILL_KERNEL_LDS;
  p.mt = LT_BM / 16;
  const long long tiles = (long long)((M + LT_BM - 1) / LT_BM) * ((N + LT_BN - 1) / LT_BN);
  const int KB = K / QK;
  int s = 1;
  while (tiles * s < num_cu && KB / (s * 2) >= 1) s *= 2;
  p.sb_per = (KB + s - 1) / s;
  p.splits = (KB + p.sb_per - 1) / p.sb_per;        // no split is left empty
  return p;
}

size_t prefill_workspace_bytes(int M, int N, int splits) {
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

hipError_t launch_prefill(const PrefillPlan& p, int qtype, const uint8_t* W, const f16* A,
                          const f16* R, f16* Y, float* P, int M, int N, int K, hipStream_t st) {
  hipError_t e = hipErrorInvalidValue;
  if (p.kind == PREFILL_KERNEL_SKINNY) return launch_skinny(qtype, W, A, R, Y, M, N, K, p.wgs, st);
  if (p.kind == PREFILL_KERNEL_LDS) {
    if (qtype == QT_Q4K) e = launch_lds_t<QT_Q4K>(W, A, R, Y, P, M, N, K, p.splits, p.sb_per, st);
    else if (qtype == QT_Q5K) e = launch_lds_t<QT_Q5K>(W, A, R, Y, P, M, N, K, p.splits, p.sb_per, st);
    else e = launch_lds_t<QT_Q6K>(W, A, R, Y, P, M, N, K, p.splits, p.sb_per, st);
  } else {
#define FCG_PF(QT_, MT_) \
  if (p.mt == MT_) e = launch_dma_t<QT_, MT_>(W, A, R, Y, P, M, N, K, p.splits, st);
    if (qtype == QT_Q4K) {
      FCG_PF(QT_Q4K, 1) else FCG_PF(QT_Q4K, 2) else FCG_PF(QT_Q4K, 4) else FCG_PF(QT_Q4K, 8)
    } else if (qtype == QT_Q5K) {
      FCG_PF(QT_Q5K, 1) else FCG_PF(QT_Q5K, 2) else FCG_PF(QT_Q5K, 4) else FCG_PF(QT_Q5K, 8)
    } else {
      FCG_PF(QT_Q6K, 1) else FCG_PF(QT_Q6K, 2) else FCG_PF(QT_Q6K, 4) else FCG_PF(QT_Q6K, 8)
    }
#undef FCG_PF
  }
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_splitk_reduce(P, R, Y, (long long)M * N, p.splits, st);
}

}  // namespace fcg
