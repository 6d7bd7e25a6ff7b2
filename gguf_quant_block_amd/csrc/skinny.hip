// Prefill path for few activation rows (up to 32; 8 .. 32 by default, fewer
// when the prefill path is forced): the f16 matrix-core FC with the decode
// path's work layout, in one launch and without a K split.
//
// OpenVINO PR #39119, section Implementation: at M >= 8 the weights are
// decoded exactly to f16 and multiplied on the matrix cores with f32
// accumulation, with the residual Add fused into the store.  With so few
// rows the tile kernels (mfma_dma.h) cannot fill the chip without splitting
// K (f32 partials and a reduction launch); this kernel instead streams the
// weights the way the decode GEMV does and keeps each row tile's whole K
// inside one workgroup.
//
// Work layout (one launch):
//   * The M activation rows (f16) are copied once per workgroup into LDS with
//     global_load_lds (16 bytes of padding per row, so the 16 rows of an
//     operand read start in different bank groups).
//   * A workgroup works on one row tile (16 weight rows, all of K) at a time,
//     persistent over row tiles b, b + gridDim.x, ...  Its nw = 4 *
//     min(KBp / 4, 4) waves split K as in the GEMV: wave w takes quarter
//     w % 4 (64 values) of the blocks of the 16 x 4-block tiles w / 4,
//     w / 4 + nw / 4, ...; lane l owns block (kb % 4 = l / 16, row l % 16), so
//     every piece load of the wave is one contiguous kilobyte.
//   * Each quarter is eight MFMA fragments of eight values.  Lane l supplies
//     the eight weights of its own block, and the activation operand of lane
//     l reads the same eight K positions of row l % 16 (+16 t): the
//     v_mfma_f32_16x16x32_f16 sum runs over the K positions the four lane
//     groups supply, which need not be contiguous, so the 4-block tile layout
//     feeds the matrix core without any shuffle.
//   * The waves' 16 x 16 partial tiles are added in wave order through LDS,
//     R is added and the result rounded once to f16.
#include "common.h"
#include "internal.h"
#include "layout.h"
#include "mfma_tile.h"

namespace fcg {

constexpr int SK_MAX_WAVES = 16;
constexpr int SK_THREADS = 64 * SK_MAX_WAVES;
constexpr int SK_ZERO = 256;   // bytes of zeros after the activation rows

__host__ __device__ inline int sk_waves(int K) {
  const int w = 4 * (tiled_kb(K / QK) / TILE_KB);
  return w < SK_MAX_WAVES ? w : SK_MAX_WAVES;
}

// LDS: activation rows f16 [M][K + 8] | SK_ZERO zero bytes (the operand of
// lanes with no row or a padding block) | partial tiles f32 [nw][MT][64][4]
__host__ __device__ inline size_t sk_zero_off(int M, int K) { return (size_t)M * (K + 8) * 2; }
__host__ __device__ inline size_t sk_part_off(int M, int K) { return sk_zero_off(M, K) + SK_ZERO; }
__host__ __device__ inline size_t sk_lds(int M, int K, int MT) {
  return sk_part_off(M, K) + (size_t)sk_waves(K) * MT * 256 * 4;
}

// The pieces of one quarter of the lane's block (the GEMV's unit): Q5_K the
// header, both qh pieces, qs pieces 2q, 2q+1; Q4_K the header, qs pieces
// 2q, 2q+1; Q6_K ql pieces 2q, 2q+1, qh pieces 2h, 2h+1, the scales piece
// and d (q = 2h + a).
template <int QT> struct SkUnit {
  static constexpr int NV = QT == QT_Q4K ? 3 : QT == QT_Q5K ? 5 : 6;
  uint4 v[NV];
};

template <int QT>
__device__ __forceinline__ void sk_load(const uint8_t* W, const WMap& L, size_t t, int q, int lane,
                                        SkUnit<QT>& u) {
  const size_t l16 = (size_t)lane << 4;
  if constexpr (QT != QT_Q6K) {
    constexpr int P = block_bytes_of(QT) / 16, QS = QT == QT_Q5K ? 3 : 1;
    const uint8_t* b = W + ((t * P) << 10) + l16;
    u.v[0] = *(const uint4*)b;
    if constexpr (QT == QT_Q5K) {
      u.v[1] = *(const uint4*)(b + 1024);
      u.v[2] = *(const uint4*)(b + 2048);
    }
    u.v[SkUnit<QT>::NV - 2] = *(const uint4*)(b + ((QS + 2 * q) << 10));
    u.v[SkUnit<QT>::NV - 1] = *(const uint4*)(b + ((QS + 2 * q + 1) << 10));
  } else {
    const uint8_t* ql = W + ((t * 8 + 2 * q) << 10) + l16;
    const uint8_t* qh = W + L.qh_base() + ((t * 4 + 2 * (q >> 1)) << 10) + l16;
    u.v[0] = *(const uint4*)ql;
    u.v[1] = *(const uint4*)(ql + 1024);
    u.v[2] = *(const uint4*)qh;
    u.v[3] = *(const uint4*)(qh + 1024);
    u.v[4] = *(const uint4*)(W + L.sc_base() + (t << 10) + l16);
    u.v[5] = make_uint4(*(const uint16_t*)(W + L.d_base() + t * 128 + ((size_t)lane << 1)), 0u, 0u, 0u);
  }
}

__device__ __forceinline__ uint32_t sk_rotr(uint32_t x, int k) { return __builtin_amdgcn_alignbit(x, x, k); }

// Q4_K / Q5_K quarter q: sub-block 2q (fragments 0-3, the low nibbles of qs
// bytes 32q + 8f .. +7) and 2q + 1 (fragments 4-7, the high nibbles); the
// eight values of fragment f are values 64q + 8f .. +7 of the block.  The
// weights are decoded exactly as the tile kernels decode them:
// fma(1024 + q, sc, -1024 sc) = sc q exactly, then (sc q) d - dmin m with one
// rounding.
template <bool HAS_QH>
struct SkDecQ45 {
  half2v sc0, sc1, b0, b1, n0, n1, d2;   // sc, -1024 sc, -dmin m of sub-blocks 2q, 2q + 1 (splat)
  uint32_t qs[8], qh[8];
  int rl;                       // rotation taking bit 2q of each qh byte to bit 4

  __device__ __forceinline__ void init(const uint4 (&v)[HAS_QH ? 5 : 3], int q) {
    const uint4 h = v[0];
    const uint32_t scw = q < 2 ? h.y & 0x3F3F3F3Fu : (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const uint32_t mw = q < 2 ? h.z & 0x3F3F3F3Fu : ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
    const int sh = 16 * (q & 1);
    const half2v k1024 = splat((f16)1024.f), nk = splat((f16)-1024.f);
    const half2v sc = magic_pair(scw >> sh, 0x04010400u) - k1024;
    const half2v bias = sc * nk;
    const half2v ndm = (magic_pair(mw >> sh, 0x04010400u) - k1024) *
                       splat(-__builtin_bit_cast(f16, (uint16_t)(h.x >> 16)));
    // one splat per sub-block (pairs indexed per fragment end up in scratch
    // memory)
    sc0 = splat(sc[0]); sc1 = splat(sc[1]);
    b0 = splat(bias[0]); b1 = splat(bias[1]);
    n0 = splat(ndm[0]); n1 = splat(ndm[1]);
    d2 = splat(__builtin_bit_cast(f16, (uint16_t)(h.x & 0xFFFFu)));
    constexpr int QS = HAS_QH ? 3 : 1;
    const uint4 a = v[QS], b = v[QS + 1];
    qs[0] = a.x; qs[1] = a.y; qs[2] = a.z; qs[3] = a.w;
    qs[4] = b.x; qs[5] = b.y; qs[6] = b.z; qs[7] = b.w;
    if constexpr (HAS_QH) {
      qh[0] = v[1].x; qh[1] = v[1].y; qh[2] = v[1].z; qh[3] = v[1].w;
      qh[4] = v[2].x; qh[5] = v[2].y; qh[6] = v[2].z; qh[7] = v[2].w;
    }
    rl = (28 + 2 * q) & 31;
  }
  __device__ __forceinline__ half8v frag(int f) const {
    const int w = 2 * (f & 3), p = f >> 2;
    uint32_t c0 = (qs[w] >> (4 * p)) & 0x0F0F0F0Fu, c1 = (qs[w + 1] >> (4 * p)) & 0x0F0F0F0Fu;
    if constexpr (HAS_QH) {
      c0 |= sk_rotr(qh[w], rl + p) & 0x10101010u;
      c1 |= sk_rotr(qh[w + 1], rl + p) & 0x10101010u;
    }
    return decode8(c0, c1, p ? sc1 : sc0, p ? b1 : b0, d2, p ? n1 : n0);
  }
  // K offset (values) of fragment f within the block
  __device__ __forceinline__ static int koff(int q, int f) { return 64 * q + 8 * f; }
};

// Q6_K quarter q = 2h + a: fragments 0-3 are the low nibbles of ql bytes
// 64h + 32a + 8f .. +7 (values 128h + 32a + 8f .. +7, qh bit pair 2a),
// fragments 4-7 their high nibbles (values 128h + 32a + 64 + 8(f - 4) .. +7,
// qh bit pair 2a + 4); fragment f lies in sub-block 8h + 2a + 4(f >> 2) +
// ((f >> 1) & 1).  w = (q - 32)(sc d) as the tile kernels decode it.
struct SkDecQ6 {
  half2v s0_, s1_, s4_, s5_;    // sc d of sub-blocks s0, s0 + 1, s0 + 4, s0 + 5 (s0 = 8h + 2a; splat)
  uint32_t ql[8], qh[8];
  int a2, rl;

  __device__ __forceinline__ void init(const uint4 (&v)[6], int q) {
    const int H = q >> 1, A = q & 1;
    const uint32_t w0 = H ? v[4].z : v[4].x, w1 = H ? v[4].w : v[4].y;
    const uint32_t p = (uint32_t)(2 * A);
    // bytes 2a, 2a + 1 of w0 (sub-blocks s0, s0 + 1) and of w1 (s0 + 4, s0 + 5),
    // offset to unsigned for the magic f16
    const uint32_t u = __builtin_amdgcn_perm(w1, w0, p | ((p + 1) << 8) | ((p + 4) << 16) | ((p + 5) << 24)) ^
                       0x80808080u;
    const half2v k1152 = splat((f16)1152.f);
    const half2v d2 = splat(__builtin_bit_cast(f16, (uint16_t)(v[5].x & 0xFFFFu)));
    const half2v s01 = (magic_pair(u, 0x04010400u) - k1152) * d2;
    const half2v s45 = (magic_pair(u, 0x04030402u) - k1152) * d2;
    s0_ = splat(s01[0]); s1_ = splat(s01[1]);
    s4_ = splat(s45[0]); s5_ = splat(s45[1]);
    ql[0] = v[0].x; ql[1] = v[0].y; ql[2] = v[0].z; ql[3] = v[0].w;
    ql[4] = v[1].x; ql[5] = v[1].y; ql[6] = v[1].z; ql[7] = v[1].w;
    qh[0] = v[2].x; qh[1] = v[2].y; qh[2] = v[2].z; qh[3] = v[2].w;
    qh[4] = v[3].x; qh[5] = v[3].y; qh[6] = v[3].z; qh[7] = v[3].w;
    a2 = 2 * A;
    rl = (28 + 2 * A) & 31;
  }
  __device__ __forceinline__ half8v frag(int f) const {
    const int w = 2 * (f & 3);
    uint32_t c0, c1;
    if (f < 4) {
      c0 = (ql[w] & 0x0F0F0F0Fu) | (sk_rotr(qh[w], rl) & 0x30303030u);
      c1 = (ql[w + 1] & 0x0F0F0F0Fu) | (sk_rotr(qh[w + 1], rl) & 0x30303030u);
    } else {
      c0 = ((ql[w] >> 4) & 0x0F0F0F0Fu) | ((qh[w] >> a2) & 0x30303030u);
      c1 = ((ql[w + 1] >> 4) & 0x0F0F0F0Fu) | ((qh[w + 1] >> a2) & 0x30303030u);
    }
    const half2v scd = f < 4 ? ((f >> 1) & 1 ? s1_ : s0_) : ((f >> 1) & 1 ? s5_ : s4_);
    const half2v k1056 = splat((f16)1056.f);
    const half2v p0 = (magic_pair(c0, 0x04010400u) - k1056) * scd;
    const half2v p1 = (magic_pair(c0, 0x04030402u) - k1056) * scd;
    const half2v p2 = (magic_pair(c1, 0x04010400u) - k1056) * scd;
    const half2v p3 = (magic_pair(c1, 0x04030402u) - k1056) * scd;
    return make_frag(p0, p1, p2, p3);
  }
  __device__ __forceinline__ static int koff(int q, int f) {
    return 128 * (q >> 1) + 32 * (q & 1) + 8 * f + 32 * (f >> 2);
  }
};

template <int QT> struct SkDec { using type = SkDecQ6; };
template <> struct SkDec<QT_Q5K> { using type = SkDecQ45<true>; };
template <> struct SkDec<QT_Q4K> { using type = SkDecQ45<false>; };

// s_waitcnt vmcnt(N), the other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void sk_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One quarter unit (tile g of the row tile) on the matrix cores: acc[t] +=
// W-fragments x activation rows 16 t .. 16 t + 15.  a_off[t]: the lane's LDS
// byte offset of fragment 0's operand (the zero bytes for a row past M or a
// padding block).
template <int QT, int MT>
__device__ __forceinline__ void sk_unit(const typename SkDec<QT>::type& dec, int q,
                                        const uint8_t* smem, const uint32_t (&a_off)[MT],
                                        floatx4 (&acc)[MT]) {
  using Dec = typename SkDec<QT>::type;
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const half8v wf = dec.frag(f);
    const uint32_t fo = 2 * (uint32_t)(Dec::koff(q, f) - Dec::koff(q, 0));
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const half8v af = *(const half8v*)(smem + a_off[t] + fo);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf, af, acc[t], 0, 0, 0);
    }
  }
}

template <int QT, int MT, bool MULTI>
__global__ void __launch_bounds__(SK_THREADS)
skinny_kernel(const uint8_t* __restrict__ W, const f16* A, const f16* R, f16* Y, int M, int N,
              int K) {
  extern __shared__ __align__(16) uint8_t smem[];
  using Dec = typename SkDec<QT>::type;
  constexpr int NV = SkUnit<QT>::NV;
  const WMap L(N, K);
  const int KB = L.KB, G = L.KBp / TILE_KB;
  const int nrt = tiled_rows(N) / TILE_ROWS;
  const int nt = blockDim.x, nw = nt >> 6, nwq = nw >> 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = wave & 3, g0 = wave >> 2;
  const uint32_t rowb = (uint32_t)(K + 8) * 2;        // LDS bytes per activation row
  const uint32_t zoff = (uint32_t)sk_zero_off(M, K);
  float* part = (float*)(smem + sk_part_off(M, K));

  // the activation rows into LDS: row m is ceil(K / 512) wave copies of up to
  // 1 KB (the last one half a kilobyte when K / 256 is odd); copy i goes to
  // wave i % nw
  {
    const int per_row = (K + 511) >> 9;
    for (int i = wave; i < M * per_row; i += nw) {
      const int m = i / per_row, j = i - m * per_row;
      const int k = 512 * j + 8 * lane;
      if (k < K)
        __builtin_amdgcn_global_load_lds(A + (size_t)m * K + k,
                                         (__attribute__((address_space(3))) void*)(smem + m * rowb + 1024 * j),
                                         16, 0, 0);
    }
  }
  if (tid < SK_ZERO / 16) *(uint4*)(smem + zoff + 16 * tid) = make_uint4(0u, 0u, 0u, 0u);

  // the residual this thread adds (thread t < 16 M: row t / 16, column t % 16
  // of the row tile), loaded a row tile ahead, kept as raw bits until it is
  // added
  const int fm = tid >> 4, fr = tid & 15;
  const bool fin = tid < 16 * M;
  auto load_r = [&](int rt) -> uint32_t {
    const int c = rt * TILE_ROWS + fr;
    if (!R || !fin) return 0u;
    return *(const uint16_t*)(R + (size_t)fm * N + (c < N ? c : N - 1));
  };
  int rt = blockIdx.x;
  uint32_t rres = load_r(rt);
  asm volatile("" ::: "memory");
  SkUnit<QT> cur;
  sk_load<QT>(W, L, (size_t)rt * G + g0, q, lane, cur);
  // the activation copies and the residual have landed (the weight loads,
  // issued after them, may still be in flight)
  sk_wait_vmcnt<NV>();
  Dec dec;
  dec.init(cur.v, q);
  __syncthreads();

  const int kq = lane >> 4, l15 = lane & 15;
  for (;;) {
    floatx4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    auto unit = [&](int g) {
      const int kb = 4 * g + kq;
      uint32_t a_off[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = l15 + 16 * t;
        a_off[t] = (kb < KB && m < M) ? (uint32_t)m * rowb + 2u * (uint32_t)(kb * QK + Dec::koff(q, 0))
                                      : zoff;
      }
      sk_unit<QT, MT>(dec, q, smem, a_off, acc);
    };
    const size_t t0 = (size_t)rt * G;
    int g = g0;
    if constexpr (MULTI) {
      // the next unit's loads are issued before this unit's matrix-core work
      for (; g + nwq < G; g += nwq) {
        sk_load<QT>(W, L, t0 + g + nwq, q, lane, cur);
        unit(g);
        dec.init(cur.v, q);
      }
    }
    const int rtn = rt + (int)gridDim.x;
    const bool more = rtn < nrt;
    uint32_t rnext = 0u;
    if (more) {
      sk_load<QT>(W, L, (size_t)rtn * G + g0, q, lane, cur);
      rnext = load_r(rtn);
    }
    unit(g);
    // the waves' partial tiles, added in wave order
#pragma unroll
    for (int t = 0; t < MT; ++t) *(floatx4*)(part + ((wave * MT + t) * 64 + lane) * 4) = acc[t];
    __syncthreads();
    if (fin) {
      // output (row fm, column fr of the row tile) sits in lane 16 (fr / 4) +
      // fm % 16, element fr % 4, of partial tile fm / 16
      const int src = ((fm >> 4) * 64 + 16 * (fr >> 2) + (fm & 15)) * 4 + (fr & 3);
      float v[SK_MAX_WAVES];
#pragma unroll
      for (int w = 0; w < SK_MAX_WAVES; ++w) v[w] = w < nw ? part[w * MT * 256 + src] : 0.f;
      float y = 0.f;
#pragma unroll
      for (int w = 0; w < SK_MAX_WAVES; ++w) y += v[w];
      const int c = rt * TILE_ROWS + fr;
      if (c < N) Y[(size_t)fm * N + c] = (f16)(y + h2f(rres));
    }
    if (!more) break;
    __syncthreads();                                // the partial tiles are rewritten
    rt = rtn;
    rres = rnext;
    dec.init(cur.v, q);
  }
}

template <int QT, int MT>
static hipError_t launch_sk_t(const uint8_t* W, const f16* A, const f16* R, f16* Y, int M, int N,
                              int K, int max_wgs, hipStream_t st) {
  const int nw = sk_waves(K);
  const int G = tiled_kb(K / QK) / TILE_KB;
  const size_t lds = sk_lds(M, K, MT);
  if (lds > 160 * 1024 || M > 16 * MT || 16 * M > 64 * nw) return hipErrorInvalidValue;
  auto kern = 4 * G > nw ? skinny_kernel<QT, MT, true> : skinny_kernel<QT, MT, false>;
  static std::atomic<uint64_t> lds_raised[2];
  if (lds > 65536) {
    hipError_t e = raise_lds_limit((const void*)kern, 160 * 1024, lds_raised[4 * G > nw]);
    if (e != hipSuccess) return e;
  }
  const int nrt = tiled_rows(N) / TILE_ROWS;
  const int grid = nrt < max_wgs ? nrt : max_wgs;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * nw), lds, st, W, A, R, Y, M, N, K);
  return hipGetLastError();
}

bool skinny_fits(int M, int K) {
  if (M < 1 || M > 32) return false;
  const int MT = M > 16 ? 2 : 1;
  return sk_lds(M, K, MT) <= 160 * 1024 && 16 * M <= 64 * sk_waves(K);
}

// Two workgroups per CU where two fit the LDS, else one (one per CU
// everywhere measured within a few per cent either way on the benchmark
// shapes).
int skinny_max_wgs(int M, int K, int num_cu) {
  const size_t lds = sk_lds(M, K, M > 16 ? 2 : 1);
  const int per_cu = lds <= 80 * 1024 ? 2 : 1;
  return per_cu * num_cu;
}

hipError_t launch_skinny(int qtype, const uint8_t* W, const f16* A, const f16* R, f16* Y, int M,
                         int N, int K, int max_wgs, hipStream_t st) {
  if (!skinny_fits(M, K)) return hipErrorInvalidValue;
  const bool two = M > 16;
  if (qtype == QT_Q4K)
    return two ? launch_sk_t<QT_Q4K, 2>(W, A, R, Y, M, N, K, max_wgs, st)
               : launch_sk_t<QT_Q4K, 1>(W, A, R, Y, M, N, K, max_wgs, st);
  if (qtype == QT_Q5K)
    return two ? launch_sk_t<QT_Q5K, 2>(W, A, R, Y, M, N, K, max_wgs, st)
               : launch_sk_t<QT_Q5K, 1>(W, A, R, Y, M, N, K, max_wgs, st);
  return two ? launch_sk_t<QT_Q6K, 2>(W, A, R, Y, M, N, K, max_wgs, st)
             : launch_sk_t<QT_Q6K, 1>(W, A, R, Y, M, N, K, max_wgs, st);
}

}  // namespace fcg
