// Device layout of the weight blocks (shared by every kernel that reads them).
//
// The blocks of one [N, K] matrix are numbered b = n * (K/256) + kb (row-major,
// the order of the GGUF tensor) and split into 16-byte pieces.  Groups of 64
// consecutive blocks are stored piece-major: piece p of block b sits at
//     ((b / 64) * P + p) * 1024 + (b % 64) * 16
// inside its plane (P = pieces per block in that plane).  A wave whose lane l
// owns block 64g + l therefore reads every piece with one fully coalesced
// 1 KB access (wave64 x 16 B), instead of 64 accesses 176 or 210 bytes apart.
// The block count is padded to a multiple of 64 with zero bytes.
//   Q4_K: one plane, P = 9 (the 144 bytes of the block, in order).
//   Q5_K: one plane, P = 11 (the 176 bytes of the block, in order).
//   Q6_K: the QL | QH | SC | D planes of OpenVINO PR #39119 (section
//         Transformation), each over the padded block count: QL P = 8,
//         QH P = 4; SC (16 B per block) and D (2 B per block) are already
//         lane-contiguous, so their pieces are simply in block order.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fcg {

constexpr int LAYOUT_GROUP = 64;

__host__ __device__ inline size_t padded_blocks(size_t nblk) {
  return (nblk + LAYOUT_GROUP - 1) / LAYOUT_GROUP * LAYOUT_GROUP;
}

// byte offset of 16-byte piece p of block b in a plane of P pieces per block
__host__ __device__ inline size_t piece_off(size_t b, int P, int p) {
  return (((b >> 6) * (size_t)P + (size_t)p) << 10) + ((b & 63) << 4);
}

// Q6_K plane bases for nbp (padded) blocks
__host__ __device__ inline size_t q6k_qh_base(size_t nbp) { return 128 * nbp; }
__host__ __device__ inline size_t q6k_sc_base(size_t nbp) { return 192 * nbp; }
__host__ __device__ inline size_t q6k_d_base(size_t nbp) { return 208 * nbp; }

}  // namespace fcg
