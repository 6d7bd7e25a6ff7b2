// Device layout of the weight blocks (shared by every kernel that reads them).
//
// Block (n, kb) is the kb-th super-block of weight row n (the GGUF tensor
// holds row n's K/256 blocks in order).  Every block is cut into 16-byte
// pieces.
//
// Tiled layout (every handle; the decode, prefill and grouped paths read it):
// the block grid is cut into tiles of 16 rows x 4 blocks (64 blocks; the row
// count is padded to a multiple of 16 and the blocks per row to a multiple
// of 4 with zero bytes).  Tiles are numbered row-tile major,
//     t = (n / 16) * (KBp / 4) + kb / 4,
// and each tile is stored piece-major, the 64 blocks of a piece in the order
// l = (kb % 4) * 16 + n % 16, so that piece p of block (n, kb) sits at
//     (t * P + p) * 1024 + l * 16
// inside its plane (P = pieces per block in that plane).  One 16-byte load
// per lane then reads a contiguous kilobyte for a GEMV wave whose lane l
// owns block l of a tile, and contiguous 256-byte runs (16 consecutive rows
// at one kb) for a matrix-core tile whose lanes own consecutive rows.
//   Q4_K / Q5_K: one plane, P = 9 / 11 (the 144 / 176 bytes of the block).
//   Q6_K: the QL | QH | SC | D planes of OpenVINO PR #39119 (section
//         Transformation), each over the padded block count: QL P = 8,
//         QH P = 4, SC P = 1; D holds 2 bytes per block at t * 128 + l * 2.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fcg {

constexpr int TILE_ROWS = 16;      // rows per tile
constexpr int TILE_KB = 4;         // blocks per row per tile

__host__ __device__ inline int tiled_rows(int N) { return (N + TILE_ROWS - 1) / TILE_ROWS * TILE_ROWS; }
__host__ __device__ inline int tiled_kb(int KB) { return (KB + TILE_KB - 1) / TILE_KB * TILE_KB; }

// Addressing of one [N, K] matrix in the tiled layout.
struct WMap {
  int KB;        // blocks per row
  int KBp;       // blocks per row as stored (padded to TILE_KB)
  size_t nbt;    // blocks per plane, padding included

  __host__ __device__ WMap(int N, int K) {
    KB = K >> 8;
    KBp = tiled_kb(KB);
    nbt = (size_t)tiled_rows(N) * KBp;
  }
  // tile index and position inside the tile of block (n, kb)
  __host__ __device__ size_t tile(int n, int kb) const {
    return (size_t)(n / TILE_ROWS) * (KBp / TILE_KB) + kb / TILE_KB;
  }
  __host__ __device__ static int slot(int n, int kb) {
    return (kb % TILE_KB) * TILE_ROWS + n % TILE_ROWS;
  }
  // byte offset of 16-byte piece p of block (n, kb) in a plane of P pieces per block
  __host__ __device__ size_t piece(int n, int kb, int P, int p) const {
    return ((tile(n, kb) * P + p) << 10) + ((size_t)slot(n, kb) << 4);
  }
  // Q6_K planes
  __host__ __device__ size_t qh_base() const { return 128 * nbt; }
  __host__ __device__ size_t sc_base() const { return 192 * nbt; }
  __host__ __device__ size_t d_base() const { return 208 * nbt; }
  __host__ __device__ size_t sc(int n, int kb) const { return sc_base() + piece(n, kb, 1, 0); }
  __host__ __device__ size_t d(int n, int kb) const {
    return d_base() + tile(n, kb) * 128 + (size_t)slot(n, kb) * 2;
  }
};

}  // namespace fcg
