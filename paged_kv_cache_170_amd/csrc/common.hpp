// Shared device/host helpers for the paged-KV kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstddef>

#include "addressing.hpp"
#include "pagedkv.h"

namespace pkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short shortx4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

constexpr int kBlockSize = 16;  // tokens per physical KV block
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------------------------
// Pool addressing.  A pool is [num_blocks, num_kv_heads, 16, head_dim]: inside a block the 16
// token rows of one KV head are contiguous (head_dim * 16 elements), so a KV head's share of a
// block is one contiguous run.  The row of (block, offset, kv_head) starts at
// ((block * num_kv_heads + kv_head) * 16 + offset) * head_dim elements.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int64_t pool_row_offset(int block, int offset, int num_kv_heads, int kv_head,
                                                   int head_dim) {
  return ((static_cast<int64_t>(block) * num_kv_heads + kv_head) * kBlockSize + offset) *
         static_cast<int64_t>(head_dim);
}

// Byte offset, inside a pool, of byte w of a token's full K (or V) row (all KV heads, head_bytes
// per head, head-major inside the row) once written to `slot`.
__device__ __forceinline__ int64_t pool_slot_byte(int64_t slot, int w, int head_bytes, int num_kv_heads) {
  const int h = w / head_bytes;
  return ((slot / kBlockSize * num_kv_heads + h) * kBlockSize + slot % kBlockSize) * head_bytes +
         (w - h * head_bytes);
}

// Byte offset of (block, in-block offset c_bytes) in a pool whose blocks are blk_bytes long.  With
// NARROW (pkv_host::narrow_addressing: block ids and block bytes below 2^24, the whole pool below
// 4 GiB) the offset is a 32-bit value built with a 24-bit multiply, which lets the load use a
// scalar base plus a 32-bit vector offset.
template <bool NARROW>
__device__ __forceinline__ const char* pool_at(const void* pool, int block, uint32_t blk_bytes, uint32_t c_bytes) {
  if constexpr (NARROW) {
    return static_cast<const char*>(pool) + (__umul24(static_cast<uint32_t>(block), blk_bytes) + c_bytes);
  } else {
    return static_cast<const char*>(pool) + (static_cast<int64_t>(block) * blk_bytes + c_bytes);
  }
}

// Reads the physical block of logical block `j` of a sequence.  In checked mode an id outside
// [0, num_blocks) sets PKV_FLAG_BAD_BLOCK and yields -1 so the caller skips the page.
template <bool CHECK>
__device__ __forceinline__ int load_block_id(const int32_t* table_row, int j, int num_blocks, int32_t* err_flag) {
  int b = table_row[j];
  if (CHECK) {
    if (b < 0 || b >= num_blocks) {
      atomicOr(err_flag, PKV_FLAG_BAD_BLOCK);
      return -1;
    }
  }
  return b;
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// 16-byte load marked non-temporal: for data read once (streamed through the caches).
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // round to nearest even
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Largest softmax weight (2^20) before the attention kernels raise their reference max.
constexpr float kMaxWeight = 1048576.f;

// Barrier of the whole workgroup.
struct WgSync {
  __device__ void operator()() const { __syncthreads(); }
};

// Barrier of one 256-thread half (waves 4h .. 4h + 3) of a 512-thread workgroup, so that the two
// halves can run separate programs: each wave adds one arrival to the half's LDS counter (zero at
// start) and waits until all four waves of the current round have arrived.  The wait is bounded
// (about 2^22 polls of 64 cycles, far beyond any real wait) so that a wave can never spin forever;
// a wave that gives up ORs PKV_FLAG_SYNC_TIMEOUT into err_flag (when the call has one): the
// half's staging data can then be corrupt and the outputs are unspecified.
struct HalfSync {
  int* cnt;
  int target;
  int32_t* err_flag;
  __device__ void operator()() {
    target += 4;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    bool arrived = false;
    for (int spins = 0; spins < (1 << 22); ++spins) {
      if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) >= target) {
        arrived = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!arrived && err_flag != nullptr && (threadIdx.x & 63) == 0) atomicOr(err_flag, PKV_FLAG_SYNC_TIMEOUT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
};

// Sixteen E4M3 codes (one 16-byte load, element i in byte i) to sixteen bf16 values in the same
// order.  Exact: every E4M3 value is a bf16 value (the conversion's scale operand is 1).
__device__ __forceinline__ void e4m3x16_to_bf16(uint4 c, uint4& lo, uint4& hi) {
#define PKV_CV(W, H) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(W, 1.0f, H))
  lo = uint4{PKV_CV(c.x, false), PKV_CV(c.x, true), PKV_CV(c.y, false), PKV_CV(c.y, true)};
  hi = uint4{PKV_CV(c.z, false), PKV_CV(c.z, true), PKV_CV(c.w, false), PKV_CV(c.w, true)};
#undef PKV_CV
}

// LDS transpose read of four 16-bit elements.  Within each group of 16 lanes, lane i receives
// element (i % 4) of the 8-byte rows addressed by lanes 4e + i/4 (e = 0..3) of its group.
// `lds_ptr` must point into __shared__ memory and be 8-byte aligned.
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t* lds_ptr) {
  typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
  shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(lds_ptr));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float floatx2;

// Two fp32 values to a packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2{a, b}), bf16x2));
}

// acc + lo + hi of a packed bf16 pair, accumulated in fp32 (one v_dot2c_f32_bf16 with (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float acc) {
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, acc, false);
}

}  // namespace pkv

// Host helpers (defined in status.hip).
namespace pkv_host {
int cu_count();                 // compute units of the current device, cached per device
pkv_status launch_status();     // PKV_OK or PKV_ERR_HIP from hipGetLastError()
}  // namespace pkv_host
