// Blocked operand layout of the MFMA contractions.
//
// A GEMM operand with R rows and a reduction length KR is stored as
// ceil(R/256) x ceil(KR/32) blocks of 256 rows x 32 reduction elements (bf16,
// 16 KiB each), blocks of one 256-row panel consecutive along the reduction
// ("panel-major"). Inside a block, row r holds its 32 elements as four 16-byte
// chunks, chunk c stored at position c ^ ((r >> 2) & 3). That is exactly the
// LDS image the MFMA fragment reads want: a direct-to-LDS load copies a block
// 1 KiB per wave instruction with no address arithmetic, and 16 lanes reading
// one logical chunk of 16 consecutive rows touch 16 distinct 16-byte slots of a
// 256-byte LDS cycle (no bank conflicts). Padding rows / reduction elements are
// zero, so the main loop needs no bounds checks.
#pragma once

#include <stdint.h>

namespace arblk {

constexpr int ROWS = 256;                 // rows per block (and per tile)
constexpr int KB = 32;                    // reduction elements per block
constexpr int BLOCK_ELEMS = ROWS * KB;    // 8192 bf16 = 16 KiB
constexpr int BLOCK_BYTES = BLOCK_ELEMS * 2;

__host__ __device__ inline int64_t row_tiles(int64_t R) { return (R + ROWS - 1) / ROWS; }
__host__ __device__ inline int64_t k_blocks(int64_t KR) { return (KR + KB - 1) / KB; }
__host__ __device__ inline int64_t elems(int64_t R, int64_t KR) {
  return row_tiles(R) * k_blocks(KR) * BLOCK_ELEMS;
}

// element offset of (r, k) in a panel-major blocked array with nkb k-blocks
__host__ __device__ inline int64_t offset(int64_t r, int64_t k, int64_t nkb) {
  const int64_t rt = r >> 8, kb = k >> 5;
  const int rr = (int)(r & 255), kk = (int)(k & 31);
  const int c = (kk >> 3) ^ ((rr >> 2) & 3);
  return ((rt * nkb + kb) << 13) + (rr << 5) + (c << 3) + (kk & 7);
}

// offset of the 8-element chunk starting at (r, k), k % 8 == 0
__host__ __device__ inline int64_t chunk_offset(int64_t r, int64_t k, int64_t nkb) {
  return offset(r, k, nkb);
}

}  // namespace arblk
