// Host-side choice of the pool addressing form (plain C++, no HIP: also compiled by the host tests).
#pragma once

#include <cstdint>

namespace pkv_host {

// Whether the kernels may address a pool with 32-bit byte offsets built by a 24-bit multiply
// (`__umul24(block, blk_bytes) + in-block offset`, the NARROW instances).  __umul24 multiplies the
// low 24 bits of each operand and keeps the low 32 bits of the product, so the form is exact only
// when both operands fit in 24 bits and every byte offset of the pool fits in 32 bits:
//   * the block id:  num_blocks < 2^24;
//   * the block size in bytes:  blk_bytes = 16 * num_kv_heads * head_dim * elem_bytes < 2^24;
//   * the pool:  num_blocks * blk_bytes < 2^32 (then block * blk_bytes + offset < 2^32 too).
// Other shapes take the 64-bit form of the same kernels.
inline bool narrow_addressing(int64_t num_blocks, int64_t num_kv_heads, int64_t head_dim, int64_t elem_bytes) {
  if (num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0 || elem_bytes <= 0) return false;
  const uint64_t blk_bytes = 16ull * static_cast<uint64_t>(num_kv_heads) * static_cast<uint64_t>(head_dim) *
                             static_cast<uint64_t>(elem_bytes);
  if (num_blocks >= (int64_t{1} << 24) || blk_bytes >= (uint64_t{1} << 24)) return false;
  return static_cast<uint64_t>(num_blocks) * blk_bytes < (uint64_t{1} << 32);
}

}  // namespace pkv_host
