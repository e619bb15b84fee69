// Paged KV cache layout (see the "Paged KV cache layout" comment of
// include/bi.h).  A (page, kv head) block is page_size / 16 tiles of 16 tokens;
// inside a tile, K and V are laid out in the order the attention kernels feed
// them to v_mfma_f32_16x16x32_bf16, so that every 16-byte operand load of a
// wavefront covers whole 128-byte lines:
//   K: (token j, dim d) at (d / 8) * 128 + k_slot(j) * 8 + d % 8
//   V: (token j, dim d) at (d / 16) * 256 + (j / 8) * 128 + (d % 16) * 8 + j % 8
#pragma once

#include "bi_common.hpp"

namespace bi {

constexpr int kTile = 16;   // tokens per tile

// Position of token j (0..15) among the 16 token rows of a K tile: tokens
// 0-3 and 8-11 form the first 128-byte half of every 8-dim group, tokens 4-7
// and 12-15 the second, matching the MFMA row order of the score product.
__device__ __forceinline__ int k_slot(int j) { return 8 * ((j >> 2) & 1) + 4 * (j >> 3) + (j & 3); }

// Element offsets inside one tile.
__device__ __forceinline__ int k_tile_off(int j, int d) { return (d >> 3) * 128 + k_slot(j) * 8 + (d & 7); }
__device__ __forceinline__ int v_tile_off(int j, int d) { return (d >> 4) * 256 + (j >> 3) * 128 + (d & 15) * 8 + (j & 7); }

// Element offset of the tile holding in-page offset `off` (0 .. page_size-1)
// of kv head `head` in physical page `page`.
__device__ __forceinline__ int64_t tile_base(int64_t page, int head, int off, int num_kv_heads, int log2_ps,
                                             int D) {
  return ((page * num_kv_heads + head) << log2_ps) * D + (int64_t)(off >> 4) * (kTile * D);
}

}  // namespace bi
