// Packed expert-weight layout: the order in which the low-precision GEMM waves consume
// their weights, so that every wave reads one contiguous stream, 1 KB per load.
//
// A workgroup of 4 waves owns a block of weight rows; each wave owns 4 tiles of 16 rows
// (mt = 0..3) and walks K in slabs of 128 elements (kb).  One slab of one tile is
// split into 1 KB pieces (h = 0..WL-1, WL = 2 for FP8, 1 for FP4); inside a piece lane
// l's 16 bytes sit at 16*l and hold exactly that lane's MFMA operand bytes:
//   FP8: row (tile row l%16), bytes kb*128 + 64*h + 16*(l/16) .. +16
//   FP4: row (tile row l%16), bytes kb*64 + 16*(l/16) .. +16   (elements 32*(l/16)..)
// Stream order: [block][wave][kb][mt][h][lane][16 B].
//   GEMM1 (W13, inter I'): block nb = I'/128 column blocks; tile rows
//       mt = 0, 1: gate rows nb*128 + 32*wave + 16*mt
//       mt = 2, 3: up rows   I' + nb*128 + 32*wave + 16*(mt-2)
//   GEMM2 (W2): block nb = ceil(H/256) row blocks; tile rows nb*256 + 64*wave + 16*mt
//       (rows >= H of a ragged last block are never written nor read)
// FP4 e8m0 scales: [block][wave][kb][lane][mt] bytes, lane l's byte for tile mt is the
// scale of its row at K block 4*kb + l/16 (the 32 elements its operand holds).
// FP8 block scales keep their plain [rows/128][K/128] layout.
#pragma once
#include <stdint.h>

#include "ctg_moe.h"

__host__ __device__ inline int pack_wl(int wfmt) { return wfmt == MOE_FP4_E2M1 ? 1 : 2; }

// byte offset of (block, wave, kb) in a packed weight stream with contraction length K
__host__ __device__ inline int64_t pack_w_offset(int wfmt, int K, int blk, int wave, int kb) {
  const int KB = K >> 7;
  return ((int64_t)(blk * 4 + wave) * KB + kb) * (4 * pack_wl(wfmt) * 1024);
}
__host__ __device__ inline int64_t pack_e_offset(int K, int blk, int wave, int kb) {
  const int KB = K >> 7;
  return ((int64_t)(blk * 4 + wave) * KB + kb) * 256;
}
__host__ __device__ inline int64_t pack_w13_offset(int wfmt, int K, int nb, int wave, int kb) {
  return pack_w_offset(wfmt, K, nb, wave, kb);
}
__host__ __device__ inline int64_t pack_e13_offset(int K, int nb, int wave, int kb) {
  return pack_e_offset(K, nb, wave, kb);
}
__host__ __device__ inline int64_t pack_w2_offset(int wfmt, int K, int nb, int wave, int kb) {
  return pack_w_offset(wfmt, K, nb, wave, kb);
}
__host__ __device__ inline int64_t pack_e2_offset(int K, int nb, int wave, int kb) {
  return pack_e_offset(K, nb, wave, kb);
}

// Row of weight matrix that tile mt of (block, wave) covers at tile row r.
__host__ __device__ inline int pack_row13(int inter, int nb, int wave, int mt, int r) {
  return (mt >= 2 ? inter : 0) + nb * 128 + 32 * wave + 16 * (mt & 1) + r;
}
__host__ __device__ inline int pack_row2(int nb, int wave, int mt, int r) {
  return nb * 256 + 64 * wave + 16 * mt + r;
}

// Bytes of one expert's packed W13 / W2 and of their packed e8m0 scales.
__host__ __device__ inline int64_t packed_w13_bytes(int wfmt, int H, int inter) {
  return (int64_t)2 * inter * H / (wfmt == MOE_FP4_E2M1 ? 2 : 1);
}
__host__ __device__ inline int64_t packed_w2_bytes(int wfmt, int H, int inter) {
  const int64_t rows = (int64_t)((H + 255) / 256) * 256;
  return rows * inter / (wfmt == MOE_FP4_E2M1 ? 2 : 1);
}
__host__ __device__ inline int64_t packed_e13_bytes(int H, int inter) { return (int64_t)2 * inter * (H / 32); }
__host__ __device__ inline int64_t packed_e2_bytes(int H, int inter) {
  return (int64_t)((H + 255) / 256) * 256 * (inter / 32);
}
