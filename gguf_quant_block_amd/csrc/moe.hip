// Grouped (MoE expert) FC on Q4_K / Q5_K / Q6_K blocks: every expert's routed rows
// times that expert's weights, all experts in one launch.
//
// llama.cpp PR #28301 (Metal mul_mm_id), section Overview: the routed rows are
// grouped by expert, each expert's rows form row tiles against that expert's
// weight tiles, and a tile whose rows end early skips its empty 16-row half.
// Numerics are those of the prefill path (OpenVINO PR #39119, section
// Implementation): weights decoded exactly to f16 once per workgroup, f16
// matrix cores, f32 accumulation, one f16 rounding at the store.
//
// Two launches on the caller's stream:
//   1. moe_bucket_kernel (one workgroup): counting sort of the (token, slot)
//      pairs by expert id -> offsets[E+2] and the pair list, then the tile
//      list: one entry (bucket, first row) per BM routed rows of a bucket.
//      Buckets 0..E-1 are the experts; bucket E holds the pairs whose id is
//      outside [0, E).  The bucketing depends on the routing only, so a
//      second grouped FC with the same routing (the down projection after
//      gate/up) can run on it without sorting again.
//   2. moe_grouped_kernel: one workgroup per (tile, weight-row tile); the
//      grid is sized for the largest possible tile count (known on the host
//      without reading the routing) and workgroups past the real count exit
//      at once.  Rows are gathered through the pair list: token t = p / top_k
//      reads A[t] (shared rows) or A[p] (one row per pair), and writes Y[p];
//      the tiles of bucket E write zero rows.
// The order of the pairs inside one expert's range is unspecified (atomic
// cursors), so the tile and the position within it that a row lands in vary
// from call to call.  Results do not: every output row depends only on its
// own activation row and its expert's weights, and the order in which its
// sum is accumulated (the K stages from a starting stage fixed by the expert
// and the weight-row tile, the same matrix-core instruction sequence) does
// not depend on the row's tile or position.  (An ordered scatter, each
// wave ranking its pairs per expert with ballots, made the one-workgroup
// bucketing about 3 us slower.)
#include "common.h"
#include "internal.h"
#include "mfma_tile.h"

namespace fcg {

constexpr int MOE_BUCKET_THREADS = 1024;
constexpr int MOE_NT = 2;                  // BN = 128 weight rows per workgroup
constexpr int MOE_PD = 1;                  // stages of prefetch in the tile main loop
constexpr int MOE_SH = 1;                  // half super-blocks per stage

// Row tile: 16-row halves, 8 per tile when the routing is dense (64 or more
// pairs per expert on average), else 2.  Empty halves of a tile are skipped,
// so a tall tile costs a short expert nothing, while a tall expert decodes its
// weights fewer times.  The 32-row tile fits four workgroups per CU (128
// registers, 17 KB of LDS), so a launch of a few hundred to a thousand items
// runs in one round instead of one and a fraction: on the benchmark routing
// (828 items of 64 rows at two per CU before, 1.6 rounds) gate/up
// 51.7 -> 48.7 us and down 52.2 -> 50.7 us per grouped launch.
static int moe_mt(int E, long long P) { return P >= 64LL * E ? 8 : 2; }

// tiles of E + 1 buckets holding P pairs in all, at most
static long long moe_max_tiles(int E, long long P, int BM) {
  return (P + BM - 1) / BM + (E + 1 < P ? E + 1 : P);
}

struct MoeWs {
  int2* tiles;      // [max_tiles] (expert, first row within the expert)
  int* offsets;     // [E + 2]: bucket b's pairs are pairs[offsets[b] .. offsets[b+1])
  int* pairs;       // [P] pair index p = t * top_k + j, grouped by expert
  int* ntiles;      // [1]
};

static MoeWs moe_ws(void* ws, int E, long long P, long long max_tiles) {
  MoeWs w;
  w.tiles = (int2*)ws;
  w.offsets = (int*)(w.tiles + max_tiles);
  w.pairs = w.offsets + (E + 2);
  w.ntiles = w.pairs + P;
  return w;
}

size_t moe_workspace_bytes(int E, int T, int top_k) {
  const long long P = (long long)T * top_k;
  const long long mt = moe_max_tiles(E, P, 16 * moe_mt(E, P));
  return (size_t)mt * sizeof(int2) + (size_t)(E + 2 + P + 1) * sizeof(int);
}

// bucket of routing id e: the expert, or E for an id outside [0, E)
__device__ __forceinline__ int moe_bucket(int e, int E) { return (unsigned)e < (unsigned)E ? e : E; }

constexpr int MOE_IDS_PT = 4;   // routing ids a thread keeps in registers between the two passes

__global__ void __launch_bounds__(MOE_BUCKET_THREADS)
moe_bucket_kernel(const int32_t* __restrict__ ids, int P, int E, int BM,
                  int2* __restrict__ tiles, int* __restrict__ offsets,
                  int* __restrict__ pairs, int* __restrict__ ntiles) {
  __shared__ int cnt[MOE_MAX_E + 1];      // rows per bucket, then the scatter cursors
  const int tid = threadIdx.x;
  const int NB = E + 1;                   // buckets
  // the thread's first MOE_IDS_PT pairs' buckets, loaded once
  int bk[MOE_IDS_PT];
#pragma unroll
  for (int i = 0; i < MOE_IDS_PT; ++i) {
    const int p = tid + i * MOE_BUCKET_THREADS;
    bk[i] = p < P ? moe_bucket(ids[p], E) : 0;
  }
  for (int b = tid; b < NB; b += MOE_BUCKET_THREADS) cnt[b] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MOE_IDS_PT; ++i)
    if (tid + i * MOE_BUCKET_THREADS < P) atomicAdd(&cnt[bk[i]], 1);
  for (int p = tid + MOE_IDS_PT * MOE_BUCKET_THREADS; p < P; p += MOE_BUCKET_THREADS)
    atomicAdd(&cnt[moe_bucket(ids[p], E)], 1);
  __syncthreads();

  // one wave scans (rows, tiles) over the buckets: lane l owns the
  // contiguous run of buckets [l per, (l + 1) per) (a block-wide scan over
  // all 16 waves took four times as long)
  unsigned long long tot = 0;
  if (tid < 64) {
    const int per = (NB + 63) / 64;
    const int e0 = tid * per;
    unsigned rows = 0, tl = 0;
    for (int q = 0; q < per; ++q) {
      const int e = e0 + q;
      if (e < NB) {
        rows += cnt[e];
        tl += (cnt[e] + BM - 1) / BM;
      }
    }
    const unsigned long long v = ((unsigned long long)tl << 32) | rows;
    unsigned long long x = v;                     // inclusive wave scan
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const unsigned long long y = __shfl_up(x, d, 64);
      if (tid >= d) x += y;
    }
    tot = __shfl(x, 63, 64);
    const unsigned long long base = x - v;
    int rbase = (int)(base & 0xFFFFFFFFu), tbase = (int)(base >> 32);
    for (int q = 0; q < per; ++q) {
      const int e = e0 + q;
      if (e >= NB) break;
      const int c = cnt[e];
      offsets[e] = rbase;
      for (int r0 = 0; r0 < c; r0 += BM) tiles[tbase++] = make_int2(e, r0);
      cnt[e] = rbase;                       // becomes the scatter cursor
      rbase += c;
    }
  }
  if (tid == 0) {
    offsets[NB] = (int)(tot & 0xFFFFFFFFu);
    *ntiles = (int)(tot >> 32);
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < MOE_IDS_PT; ++i) {
    const int p = tid + i * MOE_BUCKET_THREADS;
    if (p < P) pairs[atomicAdd(&cnt[bk[i]], 1)] = p;
  }
  for (int p = tid + MOE_IDS_PT * MOE_BUCKET_THREADS; p < P; p += MOE_BUCKET_THREADS)
    pairs[atomicAdd(&cnt[moe_bucket(ids[p], E)], 1)] = p;
}

template <int QT, int MT, int NT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT == 2 ? 4 : 1)))
moe_grouped_kernel(const uint8_t* W, size_t expert_bytes, const f16* A,
                   f16* __restrict__ Y, const int2* __restrict__ tiles,
                   const int* __restrict__ offsets, const int* __restrict__ pairs,
                   const int* __restrict__ ntiles, int E, int N, int K, int top_k, int a_per_slot,
                   int tiles_n) {
  constexpr int BM = 16 * MT;
  constexpr int BN = 64 * NT;
  __shared__ __align__(16) f16 As[2][BM * astr(MOE_SH)];

  // XCD-aware remap (round-robin dispatch over 8 XCDs) over the real items
  // (the tile count the bucketing found, times the weight-row tiles): each
  // XCD takes an equal, contiguous run of them, row tiles fastest, so the
  // row tiles of one expert against one weight-row tile share an L2, and the
  // workgroups past its run exit at once.  (Over the grid's upper bound
  // instead, the exiting items fell unevenly: on the benchmark routing two
  // XCDs of gate/up held 121 real items and six held 94-95.)
  const int nreal = *ntiles;
  const int Gr = nreal * tiles_n;
  const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
  const int per = Gr / 8, rem = Gr % 8;
  if (j >= per + (xcd < rem ? 1 : 0)) return;       // whole workgroup
  const int item = xcd * per + (xcd < rem ? xcd : rem) + j;
  const int ti = item % nreal;
  const int nt = item / nreal;

  const int2 t = tiles[ti];
  const int e = t.x;
  const int base = offsets[e] + t.y;
  int cnt = offsets[e + 1] - base;
  if (cnt > BM) cnt = BM;
  const int mt_act = (cnt + 15) / 16;
  const int n0 = nt * BN;

  const int tid = threadIdx.x;
  if (e == E) {
    // pairs routed to no expert: zero output rows (this workgroup's columns)
    for (int i = tid; i < cnt * (BN / 4); i += 256) {
      const int r = i / (BN / 4), n = n0 + 4 * (i % (BN / 4));
      f16* y = Y + (size_t)pairs[base + r] * N;
      if (n + 4 <= N && (N & 3) == 0) {
        *(uint2*)(y + n) = make_uint2(0u, 0u);
      } else {
        for (int c = n; c < n + 4 && c < N; ++c) y[c] = (f16)0.f;
      }
    }
    return;
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int kq = lane >> 4;

  TileRows<MT> rows;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int r = (tid + 256 * i) >> 4;
    const int p = pairs[base + (r < cnt ? r : 0)];
    rows.a_ld[i] = A + (size_t)(a_per_slot ? p : p / top_k) * K;
  }

  // only the halves that hold routed rows run (mt_act is uniform per workgroup)
  floatx4 acc[MT][NT];
  const uint8_t* We = W + (size_t)e * expert_bytes;
  const int S = K / (KSTAGE * MOE_SH);
  // spread concurrent loads over K: the start stage depends on the expert and
  // the weight-row tile only, so a row's summation order never depends on
  // which of its expert's tiles it was scattered to
  const int rot = (e + nt) % S;
  // (active halves rounded up to 1, 2, 4 or MT)
  if (mt_act == 1) tile_mainloop<QT, MT, NT, 1, MOE_PD, MOE_SH>(We, N, K, n0, 0, S, rot, rows, As, acc);
  else if (mt_act == 2 || MT == 2) tile_mainloop<QT, MT, NT, (MT < 2 ? MT : 2), MOE_PD, MOE_SH>(We, N, K, n0, 0, S, rot, rows, As, acc);
  else if (mt_act <= 4) tile_mainloop<QT, MT, NT, (MT < 4 ? MT : 4), MOE_PD, MOE_SH>(We, N, K, n0, 0, S, rot, rows, As, acc);
  else tile_mainloop<QT, MT, NT, MT, MOE_PD, MOE_SH>(We, N, K, n0, 0, S, rot, rows, As, acc);

#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int r = 16 * i + (lane & 15);
    if (r >= cnt) continue;
    f16* y = Y + (size_t)pairs[base + r] * N;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = n0 + wave * 16 * NT + 16 * j + 4 * kq;
      if (n < N) store4_f16(y, nullptr, n, N, acc[i][j]);
    }
  }
}

template <int QT, int MT>
static hipError_t launch_grouped_t(const uint8_t* W, size_t expert_bytes, const f16* A, f16* Y,
                                   const MoeWs& w, int E, int N, int K, int top_k, int a_per_slot,
                                   int max_tiles, hipStream_t st) {
  constexpr int BN = 64 * MOE_NT;
  const int tiles_n = (N + BN - 1) / BN;
  const long long grid = (long long)max_tiles * tiles_n;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((moe_grouped_kernel<QT, MT, MOE_NT>), dim3((unsigned)grid), dim3(256), 0, st,
                     W, expert_bytes, A, Y, w.tiles, w.offsets, w.pairs, w.ntiles, E, N, K, top_k,
                     a_per_slot, tiles_n);
  return hipGetLastError();
}

hipError_t launch_moe(int qtype, const uint8_t* W, size_t expert_bytes, int E, int N, int K,
                      const f16* A, int T, int a_per_slot, const int32_t* ids, int top_k, f16* Y,
                      void* ws, bool bucket, hipStream_t st) {
  if (E > MOE_MAX_E) return hipErrorInvalidValue;
  const long long P = (long long)T * top_k;
  const int mt = moe_mt(E, P);
  const int BM = 16 * mt;
  const long long max_tiles = moe_max_tiles(E, P, BM);
  const MoeWs w = moe_ws(ws, E, P, max_tiles);
  if (bucket) {
    hipLaunchKernelGGL(moe_bucket_kernel, dim3(1), dim3(MOE_BUCKET_THREADS), 0, st, ids, (int)P, E,
                       BM, w.tiles, w.offsets, w.pairs, w.ntiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#define FCG_MOE(QT_, MT_) \
  if (mt == MT_) return launch_grouped_t<QT_, MT_>(W, expert_bytes, A, Y, w, E, N, K, top_k, a_per_slot, (int)max_tiles, st);
  if (qtype == QT_Q4K) {
    FCG_MOE(QT_Q4K, 2) FCG_MOE(QT_Q4K, 8)
  } else if (qtype == QT_Q5K) {
    FCG_MOE(QT_Q5K, 2) FCG_MOE(QT_Q5K, 8)
  } else {
    FCG_MOE(QT_Q6K, 2) FCG_MOE(QT_Q6K, 8)
  }
#undef FCG_MOE
  return hipErrorInvalidValue;
}

hipError_t launch_debug_bucketing(const int32_t* ids, int P, int E, int BM, int* offsets, int* pairs,
                                  int* tiles, int* ntiles, hipStream_t st) {
  if (E > MOE_MAX_E) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_bucket_kernel, dim3(1), dim3(MOE_BUCKET_THREADS), 0, st, ids, P, E, BM,
                     (int2*)tiles, offsets, pairs, ntiles);
  return hipGetLastError();
}

}  // namespace fcg
