// Cache row addressing shared by the decode kernels.
#pragma once

#include "kvattn_internal.h"

namespace kvattn {

// Element offset of token t's row (KV head j of sequence b) in a cache whose
// rows are `width` elements wide, or -1 when a paged table entry points
// outside the pool.
//   contiguous: rows of (b, j) are consecutive: ((b*g + j)*cache_len + t)*width
//   paged:      token t sits in block table[b][t / block_size], slot
//               t % block_size; a (block, j) pair holds block_size rows.
__device__ __forceinline__ int64_t cache_row_offset(const DecodeArgs& a, int b, int j, int t, int width) {
  if (a.block_size == 0) {
    return ((int64_t)(b * a.num_kv_heads + j) * a.cache_len + t) * width;
  }
  const int bs = a.block_size;
  const int blk = a.block_table[(int64_t)b * a.max_blocks + t / bs];
  if (blk < 0 || (int64_t)blk >= a.cache_len) return -1;
  return (((int64_t)blk * a.num_kv_heads + j) * bs + (t % bs)) * width;
}

}  // namespace kvattn
