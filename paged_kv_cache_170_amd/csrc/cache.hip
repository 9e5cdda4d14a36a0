// Slot mapping, slot-mapped cache write, block copy (copy-on-write) and the paged gather diagnostic.
//
// Slot mapping follows the block-table definition of "第2章:推理引擎核心技术" (aiinfra.vidrealm.tech)
// §1.2 and the PagedAttention section of "Phase 17 · 04 — vLLM serving internals": the physical
// block of position p is the table entry of logical block p / 16, its row inside the block is
// p % 16.  The write stores new tokens' K/V rows in those slots ("Chunked Prefill", Ultralytics,
// section on prefill and decode); the gather reproduces the figure 按块表取 K of "C13 推理 · 第2课"
// (rows of the pool taken through the table, in logical order).
#include <cmath>

#include "common.hpp"

namespace pkv {

// One thread per new token.  grid = (ceil(max_new_len / 256), num_seqs).
template <bool CHECK>
__global__ __launch_bounds__(256) void slot_mapping_kernel(int32_t* __restrict__ slots,
                                                           const int32_t* __restrict__ block_tables, int max_blocks,
                                                           const int32_t* __restrict__ cu_new_lens,
                                                           const int32_t* __restrict__ start_pos, int num_blocks,
                                                           int32_t* err_flag) {
  const int s = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int lo = cu_new_lens[s];
  const int n = cu_new_lens[s + 1] - lo;
  if (i >= n) return;
  const int p = start_pos[s] + i;
  const int j = p >> 4;
  int slot = -1;
  if (p >= 0 && j < max_blocks) {
    const int b = load_block_id<CHECK>(block_tables + static_cast<int64_t>(s) * max_blocks, j, num_blocks, err_flag);
    if (b >= 0) slot = b * kBlockSize + (p & (kBlockSize - 1));
  } else if (CHECK) {
    atomicOr(err_flag, PKV_FLAG_BAD_LENGTH);
  }
  slots[lo + i] = slot;
}

// Row copy: each thread moves one VEC-byte piece of one token's K row and V row.  Rows are
// `row_bytes` long (head_bytes per KV head, each head's piece going to its own run of the block);
// VEC divides head_bytes and the alignment of every address.
template <int VEC, bool CHECK>
__global__ __launch_bounds__(256) void cache_write_kernel(const char* __restrict__ key, const char* __restrict__ value,
                                                          int64_t key_stride_bytes, int64_t value_stride_bytes,
                                                          char* __restrict__ key_pool, char* __restrict__ value_pool,
                                                          const int32_t* __restrict__ slots, int num_tokens,
                                                          int row_bytes, int head_bytes, int64_t num_slots,
                                                          int32_t* err_flag) {
  const int pieces = row_bytes / VEC;
  const int num_kv_heads = row_bytes / head_bytes;
  const int64_t total = static_cast<int64_t>(num_tokens) * pieces;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int t = static_cast<int>(i / pieces);
    const int c = static_cast<int>(i - static_cast<int64_t>(t) * pieces);
    const int slot = slots[t];
    if (slot < 0) continue;
    if (CHECK && slot >= num_slots) {
      if (c == 0) atomicOr(err_flag, PKV_FLAG_BAD_SLOT);
      continue;
    }
    const int64_t dst = pool_slot_byte(slot, c * VEC, head_bytes, num_kv_heads);
    const char* ks = key + t * key_stride_bytes + c * VEC;
    const char* vs = value + t * value_stride_bytes + c * VEC;
    if constexpr (VEC == 16) {
      st16(key_pool + dst, ld16(ks));
      st16(value_pool + dst, ld16(vs));
    } else if constexpr (VEC == 4) {
      *reinterpret_cast<uint32_t*>(key_pool + dst) = *reinterpret_cast<const uint32_t*>(ks);
      *reinterpret_cast<uint32_t*>(value_pool + dst) = *reinterpret_cast<const uint32_t*>(vs);
    } else {
      *reinterpret_cast<uint16_t*>(key_pool + dst) = *reinterpret_cast<const uint16_t*>(ks);
      *reinterpret_cast<uint16_t*>(value_pool + dst) = *reinterpret_cast<const uint16_t*>(vs);
    }
  }
}

// E4M3 code of an fp32 value (OCP 8-bit floating point, E4M3: bias 7, 3 mantissa bits, no
// infinities, S.1111.111 = NaN): nearest value, ties to the even code; magnitudes >= 448 and
// infinities saturate to +-448; NaN gives 0x7F; the sign of zero is kept.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;          // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // >= 448 or infinite
  if (a >= 0x3c800000u) {                     // >= 2^-6: normal range
    // Rebias the exponent (127 -> 7) and keep 3 mantissa bits; round the 20 dropped bits to
    // nearest even (a carry moves into the exponent field).  |x| < 448 keeps the result <= 0x7E.
    uint32_t t = (a >> 20) - (120u << 3);
    const uint32_t rem = a & 0xfffffu;
    t += (rem > 0x80000u || (rem == 0x80000u && (t & 1u))) ? 1u : 0u;
    return sign | t;
  }
  // Subnormal range: value m * 2^-9 with m = |x| * 2^9 rounded to nearest even (m = 8 is 2^-6,
  // the smallest normal, whose code is also 8).
  return sign | static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.f));
}

// Quantising write: each thread turns 8 consecutive elements of one token's K row and V row into
// codes (an 8-byte store per tensor).  VECIN: 16-byte input loads (aligned rows), else scalar.
template <typename T, bool VECIN, bool CHECK>
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(const T* __restrict__ key, const T* __restrict__ value,
                                                              int64_t key_stride, int64_t value_stride,
                                                              uint8_t* __restrict__ key_pool,
                                                              uint8_t* __restrict__ value_pool,
                                                              const int32_t* __restrict__ slots, int num_tokens,
                                                              int row_elems, int head_dim, int64_t num_slots,
                                                              float inv_k, float inv_v, int32_t* err_flag) {
  const int pieces = row_elems / 8;
  const int num_kv_heads = row_elems / head_dim;
  const int64_t total = static_cast<int64_t>(num_tokens) * pieces;
  auto widen = [](T v) -> float {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(v); else return v;
  };
  auto codes8 = [&](const T* src, float inv) {
    float x[8];
    if constexpr (VECIN && sizeof(T) == 2) {
      const uint4 w = ld16(src);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(ws[i] << 16);
        x[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
      }
    } else if constexpr (VECIN) {
      const float4 a = *reinterpret_cast<const float4*>(src), b = *reinterpret_cast<const float4*>(src + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = widen(src[i]);
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= e4m3_code(x[i] * inv) << (8 * i);
      hi |= e4m3_code(x[4 + i] * inv) << (8 * i);
    }
    return uint2{lo, hi};
  };
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int t = static_cast<int>(i / pieces);
    const int c = static_cast<int>(i - static_cast<int64_t>(t) * pieces);
    const int slot = slots[t];
    if (slot < 0) continue;
    if (CHECK && slot >= num_slots) {
      if (c == 0) atomicOr(err_flag, PKV_FLAG_BAD_SLOT);
      continue;
    }
    const int64_t dst = pool_slot_byte(slot, c * 8, head_dim, num_kv_heads);  // one byte per code
    *reinterpret_cast<uint2*>(key_pool + dst) = codes8(key + t * key_stride + c * 8, inv_k);
    *reinterpret_cast<uint2*>(value_pool + dst) = codes8(value + t * value_stride + c * 8, inv_v);
  }
}

// Block copy for copy-on-write ("第2章:推理引擎核心技术" §1.5): grid = (pieces / 256, num_pairs); each
// thread moves one 16-byte piece of block src[i] to block dst[i] in both pools.  Blocks are
// 16 * Hkv * hd * e bytes, a multiple of 16 * 64 * 2 = 2 KiB, so the pieces divide evenly.
template <bool CHECK>
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ key_pool, char* __restrict__ value_pool,
                                                          const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst, int64_t block_bytes,
                                                          int num_blocks, int32_t* err_flag) {
  const int i = blockIdx.y;
  const int s = src[i], d = dst[i];
  if (CHECK && (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err_flag, PKV_FLAG_BAD_BLOCK);
    return;
  }
  if (s == d) return;
  const int64_t off = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 16;
  if (off >= block_bytes) return;
  st16(key_pool + d * block_bytes + off, ld16(key_pool + s * block_bytes + off));
  st16(value_pool + d * block_bytes + off, ld16(value_pool + s * block_bytes + off));
}

// Gather: grid = (ceil(max_len * pieces / 256), num_seqs); 16-byte pieces of whole token rows.
template <bool CHECK>
__global__ __launch_bounds__(256) void paged_gather_kernel(char* __restrict__ key_out, char* __restrict__ value_out,
                                                           const char* __restrict__ key_pool,
                                                           const char* __restrict__ value_pool,
                                                           const int32_t* __restrict__ block_tables, int max_blocks,
                                                           const int32_t* __restrict__ lengths,
                                                           const int32_t* __restrict__ cu_out, int num_blocks,
                                                           int num_kv_heads, int head_dim, int elem_bytes,
                                                           int32_t* err_flag) {
  const int row_bytes = num_kv_heads * head_dim * elem_bytes;
  const int s = blockIdx.y;
  const int pieces = row_bytes / 16;
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  const int t = static_cast<int>(i / pieces);
  const int c = static_cast<int>(i - static_cast<int64_t>(t) * pieces);
  const int len = lengths[s];
  if (t >= len) return;
  if (CHECK && len > max_blocks * kBlockSize) {
    if (t == 0 && c == 0) atomicOr(err_flag, PKV_FLAG_BAD_LENGTH);
    return;
  }
  const int b = load_block_id<CHECK>(block_tables + static_cast<int64_t>(s) * max_blocks, t >> 4, num_blocks,
                                     err_flag);
  if (b < 0) return;
  // Same row arithmetic as the attention kernels: piece c lies in KV head h's row of the token.
  const int head_bytes = head_dim * elem_bytes;
  const int h = c * 16 / head_bytes;
  const int64_t src = pool_row_offset(b, t & (kBlockSize - 1), num_kv_heads, h, head_dim) * elem_bytes +
                      (c * 16 - h * head_bytes);
  const int64_t dst = (static_cast<int64_t>(cu_out[s]) + t) * row_bytes + c * 16;
  st16(key_out + dst, ld16(key_pool + src));
  st16(value_out + dst, ld16(value_pool + src));
}

}  // namespace pkv

using namespace pkv;

namespace {
int dtype_bytes(pkv_dtype d) { return d == PKV_DTYPE_F32 ? 4 : (d == PKV_DTYPE_BF16 ? 2 : 0); }
// Bytes per element of a pool (the bit-copy calls also take FP8 pools).
int pool_bytes(pkv_dtype d) { return d == PKV_DTYPE_FP8_E4M3 ? 1 : dtype_bytes(d); }
bool scale_ok(float x) { return std::isfinite(x) && x > 0.f; }
bool head_dim_ok(int hd) { return hd == 64 || hd == 128 || hd == 256; }
}  // namespace

extern "C" pkv_status pkv_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* cu_new_lens, const int32_t* start_pos, int32_t num_seqs,
                                       int32_t max_new_len, int32_t num_blocks, int32_t block_size,
                                       int32_t* err_flag, void* stream) {
  if (num_seqs < 0 || max_new_len < 0 || max_blocks_per_seq < 0 || num_blocks < 0) return PKV_ERR_INVALID_ARG;
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_new_len == 0) return PKV_OK;
  if (num_seqs > 65535) return PKV_ERR_UNSUPPORTED;  // grid y limit
  if (!slot_mapping || !block_tables || !cu_new_lens || !start_pos || max_blocks_per_seq == 0)
    return PKV_ERR_INVALID_ARG;
  dim3 grid((max_new_len + 255) / 256, num_seqs);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (err_flag)
    hipLaunchKernelGGL(slot_mapping_kernel<true>, grid, dim3(256), 0, st, slot_mapping, block_tables,
                       max_blocks_per_seq, cu_new_lens, start_pos, num_blocks, err_flag);
  else
    hipLaunchKernelGGL(slot_mapping_kernel<false>, grid, dim3(256), 0, st, slot_mapping, block_tables,
                       max_blocks_per_seq, cu_new_lens, start_pos, num_blocks, err_flag);
  return pkv_host::launch_status();
}

extern "C" pkv_status pkv_cache_write(const void* key, const void* value, int64_t key_tok_stride,
                                      int64_t value_tok_stride, void* key_pool, void* value_pool,
                                      const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_dtype dtype,
                                      int32_t* err_flag, void* stream) {
  const int e = dtype_bytes(dtype);
  if (e == 0 || block_size != kBlockSize || !head_dim_ok(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  const int64_t row_elems = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (key_tok_stride < row_elems || value_tok_stride < row_elems) return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !key_pool || !value_pool || !slot_mapping) return PKV_ERR_INVALID_ARG;
  const int row_bytes = static_cast<int>(row_elems * e);
  const int64_t ks = key_tok_stride * e, vs = value_tok_stride * e;
  auto aligned = [](const void* p, int a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  const bool a16 = aligned(key, 16) && aligned(value, 16) && aligned(key_pool, 16) && aligned(value_pool, 16) &&
                   ks % 16 == 0 && vs % 16 == 0;
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * kBlockSize;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int vec = a16 ? 16 : e;
  const int64_t total = static_cast<int64_t>(num_tokens) * (row_bytes / vec);
  const int64_t want = (total + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
#define PKV_LAUNCH_WRITE(V, C)                                                                                   \
  hipLaunchKernelGGL((cache_write_kernel<V, C>), dim3(blocks), dim3(256), 0, st, static_cast<const char*>(key),  \
                     static_cast<const char*>(value), ks, vs, static_cast<char*>(key_pool),                      \
                     static_cast<char*>(value_pool), slot_mapping, num_tokens, row_bytes, head_dim * e, num_slots, \
                     err_flag)
  if (vec == 16) {
    if (err_flag) PKV_LAUNCH_WRITE(16, true); else PKV_LAUNCH_WRITE(16, false);
  } else if (vec == 4) {
    if (err_flag) PKV_LAUNCH_WRITE(4, true); else PKV_LAUNCH_WRITE(4, false);
  } else {
    if (err_flag) PKV_LAUNCH_WRITE(2, true); else PKV_LAUNCH_WRITE(2, false);
  }
#undef PKV_LAUNCH_WRITE
  return pkv_host::launch_status();
}

extern "C" pkv_status pkv_cache_write_fp8(const void* key, const void* value, int64_t key_tok_stride,
                                          int64_t value_tok_stride, void* key_pool, void* value_pool,
                                          const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                          pkv_dtype in_dtype, float k_scale, float v_scale, int32_t* err_flag,
                                          void* stream) {
  const int e = dtype_bytes(in_dtype);
  if (e == 0 || block_size != kBlockSize || !head_dim_ok(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || !scale_ok(k_scale) || !scale_ok(v_scale))
    return PKV_ERR_INVALID_ARG;
  const int64_t row_elems = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (key_tok_stride < row_elems || value_tok_stride < row_elems) return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !key_pool || !value_pool || !slot_mapping) return PKV_ERR_INVALID_ARG;
  for (const void* p : {static_cast<const void*>(key_pool), static_cast<const void*>(value_pool)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return PKV_ERR_INVALID_ARG;
  auto aligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; };
  const bool vec = aligned(key) && aligned(value) && (key_tok_stride * e) % 16 == 0 && (value_tok_stride * e) % 16 == 0;
  // The reciprocals are rounded to nearest in fp32 here, on the host.
  const float inv_k = 1.0f / k_scale, inv_v = 1.0f / v_scale;
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * kBlockSize;
  const int64_t total = static_cast<int64_t>(num_tokens) * (row_elems / 8);
  const int64_t want = (total + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipStream_t st = static_cast<hipStream_t>(stream);
#define PKV_LAUNCH_W8(T, V, C)                                                                                  \
  hipLaunchKernelGGL((cache_write_fp8_kernel<T, V, C>), dim3(blocks), dim3(256), 0, st,                         \
                     static_cast<const T*>(key), static_cast<const T*>(value), key_tok_stride, value_tok_stride, \
                     static_cast<uint8_t*>(key_pool), static_cast<uint8_t*>(value_pool), slot_mapping,          \
                     num_tokens, static_cast<int>(row_elems), head_dim, num_slots, inv_k, inv_v, err_flag)
#define PKV_LAUNCH_W8_C(T, V) \
  if (err_flag) PKV_LAUNCH_W8(T, V, true); else PKV_LAUNCH_W8(T, V, false);
  if (in_dtype == PKV_DTYPE_BF16) {
    if (vec) { PKV_LAUNCH_W8_C(uint16_t, true) } else { PKV_LAUNCH_W8_C(uint16_t, false) }
  } else {
    if (vec) { PKV_LAUNCH_W8_C(float, true) } else { PKV_LAUNCH_W8_C(float, false) }
  }
#undef PKV_LAUNCH_W8_C
#undef PKV_LAUNCH_W8
  return pkv_host::launch_status();
}

extern "C" pkv_status pkv_paged_gather(void* key_out, void* value_out, const void* key_pool, const void* value_pool,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* lengths, const int32_t* cu_out, int32_t num_seqs,
                                       int32_t max_len, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, pkv_dtype dtype, int32_t* err_flag, void* stream) {
  const int e = pool_bytes(dtype);
  if (e == 0 || block_size != kBlockSize || !head_dim_ok(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_len < 0 || num_blocks < 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_len == 0) return PKV_OK;
  if (num_seqs > 65535) return PKV_ERR_UNSUPPORTED;  // grid y limit
  if (!key_out || !value_out || !key_pool || !value_pool || !block_tables || !lengths || !cu_out ||
      max_blocks_per_seq == 0)
    return PKV_ERR_INVALID_ARG;
  const int row_bytes = num_kv_heads * head_dim * e;
  const int64_t threads = static_cast<int64_t>(max_len) * (row_bytes / 16);
  dim3 grid(static_cast<unsigned>((threads + 255) / 256), num_seqs);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (err_flag)
    hipLaunchKernelGGL(paged_gather_kernel<true>, grid, dim3(256), 0, st, static_cast<char*>(key_out),
                       static_cast<char*>(value_out), static_cast<const char*>(key_pool),
                       static_cast<const char*>(value_pool), block_tables, max_blocks_per_seq, lengths, cu_out,
                       num_blocks, num_kv_heads, head_dim, e, err_flag);
  else
    hipLaunchKernelGGL(paged_gather_kernel<false>, grid, dim3(256), 0, st, static_cast<char*>(key_out),
                       static_cast<char*>(value_out), static_cast<const char*>(key_pool),
                       static_cast<const char*>(value_pool), block_tables, max_blocks_per_seq, lengths, cu_out,
                       num_blocks, num_kv_heads, head_dim, e, err_flag);
  return pkv_host::launch_status();
}

extern "C" pkv_status pkv_copy_blocks(void* key_pool, void* value_pool, const int32_t* src, const int32_t* dst,
                                      int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, pkv_dtype dtype, int32_t* err_flag, void* stream) {
  const int e = pool_bytes(dtype);
  if (e == 0 || block_size != kBlockSize || !head_dim_ok(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_pairs < 0 || num_blocks < 0 || num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (num_pairs == 0) return PKV_OK;
  if (num_pairs > 65535) return PKV_ERR_UNSUPPORTED;  // grid y limit
  if (!key_pool || !value_pool || !src || !dst) return PKV_ERR_INVALID_ARG;
  for (const void* p : {static_cast<const void*>(key_pool), static_cast<const void*>(value_pool)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return PKV_ERR_INVALID_ARG;
  const int64_t block_bytes = static_cast<int64_t>(kBlockSize) * num_kv_heads * head_dim * e;
  const dim3 grid(static_cast<unsigned>((block_bytes / 16 + 255) / 256), static_cast<unsigned>(num_pairs));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (err_flag)
    hipLaunchKernelGGL(copy_blocks_kernel<true>, grid, dim3(256), 0, st, static_cast<char*>(key_pool),
                       static_cast<char*>(value_pool), src, dst, block_bytes, num_blocks, err_flag);
  else
    hipLaunchKernelGGL(copy_blocks_kernel<false>, grid, dim3(256), 0, st, static_cast<char*>(key_pool),
                       static_cast<char*>(value_pool), src, dst, block_bytes, num_blocks, err_flag);
  return pkv_host::launch_status();
}
