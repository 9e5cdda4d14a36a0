// Chunked-prefill attention over the paged cache (bf16 MFMA, fp32 accumulation).
//
// What is computed ("Chunked Prefill", Ultralytics, section on how chunked prefill works, and its
// PyTorch example): a chunk row at absolute position P attends to every cached key at a position
// <= P (causal) — the earlier chunks and its own chunk, which the cache write stored first — so
// the chunked result equals one-pass causal prefill.  Non-causal rows see the whole chunk end.
//
// Design (gfx950, wave64):
//   * a work item is 256 rows (eight waves of 32 rows) and one key split.  The rows are the chunk
//     positions of one query head, or, when that gives fewer row tiles (chunks short of 256
//     positions, or well short of a multiple of it), the (position, query head) pairs of one KV
//     head's group (row R = position R / G, query head g*G + R % G), so that each K/V tile an item
//     stages serves all G heads; the 1-D grid is remapped so that each XCD (workgroups are dealt
//     round-robin over the 8 XCDs) gets a contiguous run of items, whose K/V streams then meet in
//     the XCD's L2.
//   * when there are fewer row tiles than compute units, a row tile's key range is cut into up to
//     eight splits of whole tile pairs, one workgroup each; every split writes its (o, m, l) partial
//     to the workspace and prefill_merge_kernel combines them in split order after the launch.
//   * key tiles (64 positions = 4 blocks; 32 for head_dim 256) are gathered through the block
//     table by all 512 threads, a pair at a time, into double-buffered LDS; all eight waves compute
//     on both tiles of a pair; the next pair's loads are in flight while the current pair is
//     computed, with one barrier per pair.  Block ids are staged in an LDS window.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q rows in registers);
//     the accumulator layout gives each lane 16 keys of one query.  Only tiles crossing the causal
//     diagonal or the key end are masked.  The reference max the exponentials subtract trails the
//     running max: it is raised (with the accumulator rescale) only when a weight would exceed
//     2^20, on edge tiles, or before the first key, so the common path computes no row max.
//   * P stays in registers and is exactly the B operand of O^T = V^T P^T; V^T comes from the
//     natural-layout V tile through ds_read_b64_tr_b16.
//   * consecutive MFMAs work on different accumulators, and the LDS operand reads are scheduled
//     four (K) or eight (V) reads ahead of the MFMAs that use them, so MFMA issue does not wait on
//     LDS latency.
#include "prefill_dev.hpp"

namespace pkv {

// Log-sum-exp merge of a row tile's key splits: grid = (row items, kPreTile / 32), 256 threads per
// 32-row slice.  First 32 threads turn their row's (m, l) pairs into split weights (in split order,
// so the result does not depend on which split finished first); then the threads sweep the slice's
// partial rows with 16-byte loads, consecutive threads on consecutive columns of one row.
constexpr int kMergeRows = 32;

template <int HD>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PreArgs a) {
  __shared__ float wgt[kMergeRows][kPreMaxSplit];
  __shared__ float inv_s[kMergeRows];
  const int w = blockIdx.x, r0 = blockIdx.y * kMergeRows;
  const int t = w % a.q_tiles;
  int q = w / a.q_tiles;
  const int hp = a.pack ? a.group : 1;  // query heads sharing the rows
  const int hi = a.pack ? 0 : q % a.group;
  q = a.pack ? q : q / a.group;
  const int g = q % a.num_kv_heads;
  const int s = q / a.num_kv_heads;
  const int qlo = a.cu_q_lens[s];
  const int nrows = (a.cu_q_lens[s + 1] - qlo) * hp;
  const int rows = min(kMergeRows, nrows - t * kPreTile - r0);
  if (rows <= 0) return;
  const int ks = a.ksplit;
  const int64_t base = static_cast<int64_t>(w) * ks * kPreTile + r0;
  if (threadIdx.x < kMergeRows) {
    const int r = threadIdx.x;
    float M = -INFINITY;
    for (int k = 0; k < ks; ++k) M = fmaxf(M, a.ws_ml[(base + static_cast<int64_t>(k) * kPreTile + r) * 2]);
    float Ls = 0.f;
    for (int k = 0; k < ks; ++k) {
      const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + (base + static_cast<int64_t>(k) * kPreTile + r) * 2);
      const float f = (ml.x == -INFINITY) ? 0.f : fast_exp2(ml.x - M);
      wgt[r][k] = f;
      Ls += f * ml.y;
    }
    inv_s[r] = Ls > 0.f ? a.v_scale / Ls : 0.f;
  }
  __syncthreads();
  constexpr int Q = HD / 4;  // 16-byte pieces per row
  for (int i = threadIdx.x; i < rows * Q; i += 256) {
    const int r = i / Q, d = (i % Q) * 4;
    float4 o = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < ks; ++k) {
      const float f = wgt[r][k];
      const float4 p = *reinterpret_cast<const float4*>(a.ws_o + (base + static_cast<int64_t>(k) * kPreTile + r) * HD + d);
      o.x += f * p.x;
      o.y += f * p.y;
      o.z += f * p.z;
      o.w += f * p.w;
    }
    const float inv = inv_s[r];
    o.x *= inv;
    o.y *= inv;
    o.z *= inv;
    o.w *= inv;
    const int R = t * kPreTile + r0 + r;  // row: position R / hp, query head g*G + hi + R % hp
    const int64_t oi = (static_cast<int64_t>(qlo + R / hp) * a.num_q_heads + g * a.group + hi + R % hp) * HD + d;
    if (a.out_bf16)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + oi) = uint2{pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
    else
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + oi) = o;
  }
}

template <int HD, bool CHECK, bool NARROW, bool KV8, bool PACK>
__global__ __launch_bounds__(kPreThreads) void prefill_bf16_kernel(PreArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[PreCfg<HD>::LDS];
  __shared__ int ids[kIdWindow];
  prefill_body<HD, CHECK, NARROW, KV8, PACK>(a, blockIdx.x, gridDim.x, smem, ids);
}

}  // namespace pkv

using namespace pkv;

void pkv_pre::launch_merge(const PreArgs& a, int64_t row_items, int32_t head_dim, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(row_items), kPreTile / kMergeRows);
  if (head_dim == 64)
    hipLaunchKernelGGL(prefill_merge_kernel<64>, grid, dim3(kPreTile), 0, st, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL(prefill_merge_kernel<128>, grid, dim3(kPreTile), 0, st, a);
  else
    hipLaunchKernelGGL(prefill_merge_kernel<256>, grid, dim3(kPreTile), 0, st, a);
}

namespace {

// Shared body of the bf16 and FP8 prefill calls (dtype = pool dtype; queries are bf16).
pkv_status prefill_impl(void* out, pkv_dtype out_dtype, const void* query, const int32_t* cu_q_lens,
                        const int32_t* chunk_offsets, const void* key_pool, const void* value_pool,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs, int32_t max_q_len,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                        int32_t causal, float scale, pkv_dtype dtype, float k_scale, float v_scale,
                        void* workspace, size_t workspace_bytes, int32_t* err_flag, void* stream) {
  const bool kv8 = dtype == PKV_DTYPE_FP8_E4M3;
  if (kv8 && (!std::isfinite(k_scale) || !(k_scale > 0.f) || !std::isfinite(v_scale) || !(v_scale > 0.f)))
    return PKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || max_q_len < 0 || num_blocks < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || !std::isfinite(scale) || !(scale > 0.f))
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (dtype != PKV_DTYPE_BF16 && !kv8) return PKV_ERR_UNSUPPORTED;
  if (out_dtype != PKV_DTYPE_F32 && out_dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  if (num_blocks == 0) return PKV_ERR_INVALID_ARG;  // a non-empty chunk needs cached positions
  if (!out || !query || !cu_q_lens || !chunk_offsets || !key_pool || !value_pool || !block_tables)
    return PKV_ERR_INVALID_ARG;
  for (const void* p : {static_cast<const void*>(out), query, key_pool, value_pool})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return PKV_ERR_INVALID_ARG;
  const int group = num_q_heads / num_kv_heads;
  const bool pack = pkv_pre::pack_rows(max_q_len, num_q_heads, num_kv_heads);
  const int64_t q_tiles64 = pkv_pre::row_tiles(max_q_len, pack ? group : 1);
  if (q_tiles64 > (1 << 22)) return PKV_ERR_UNSUPPORTED;
  const int q_tiles = static_cast<int>(q_tiles64);
  const int64_t row_items = static_cast<int64_t>(num_seqs) * (pack ? num_kv_heads : num_q_heads) * q_tiles;
  const int ksplit = pkv_pre::ksplit_for(row_items, max_blocks_per_seq, head_dim, pkv_host::cu_count());
  const int64_t items = row_items * ksplit;
  if (items > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  const pkv_pre::Layout lay = pkv_pre::layout(row_items, ksplit, head_dim);
  if (ksplit > 1 && (!workspace || workspace_bytes < lay.total)) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (ksplit > 1 && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return PKV_ERR_INVALID_ARG;
  char* ws = static_cast<char*>(workspace);
  const float scale_log2 = kv8 ? scale * kLog2e * k_scale : scale * kLog2e;
  const float vs = kv8 ? v_scale : 1.f;
  const int ob = out_dtype == PKV_DTYPE_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool narrow = pkv_host::narrow_addressing(num_blocks, num_kv_heads, head_dim, kv8 ? 1 : 2);
  PreArgs pa{static_cast<const uint16_t*>(query), cu_q_lens, chunk_offsets, key_pool, value_pool, block_tables,
                   max_blocks_per_seq, q_tiles, num_q_heads, num_kv_heads, group, num_blocks, causal != 0,
                   scale_log2, vs, out, ob, err_flag, ksplit,
                   ksplit > 1 ? reinterpret_cast<float*>(ws + lay.o) : nullptr,
                   ksplit > 1 ? reinterpret_cast<float*>(ws + lay.ml) : nullptr};
  pa.pack = pack;
#define PKV_PRE(HD, CHECK, NARROW, KV8, PACK)                                                                  \
  hipLaunchKernelGGL((prefill_bf16_kernel<HD, CHECK, NARROW, KV8, PACK>), dim3(static_cast<unsigned>(items)), \
                     dim3(kPreThreads), 0, st, pa)
#define PKV_PRE_P(HD, CHECK, NARROW, KV8) \
  if (pack) PKV_PRE(HD, CHECK, NARROW, KV8, true); else PKV_PRE(HD, CHECK, NARROW, KV8, false);
#define PKV_PRE_K(HD, CHECK, NARROW) \
  if (kv8) { PKV_PRE_P(HD, CHECK, NARROW, true) } else { PKV_PRE_P(HD, CHECK, NARROW, false) }
#define PKV_PRE_N(HD, CHECK) \
  if (narrow) { PKV_PRE_K(HD, CHECK, true) } else { PKV_PRE_K(HD, CHECK, false) }
#define PKV_PRE_HD(CHECK)                         \
  switch (head_dim) {                             \
    case 64: PKV_PRE_N(64, CHECK) break;          \
    case 128: PKV_PRE_N(128, CHECK) break;        \
    default: PKV_PRE_N(256, CHECK) break;         \
  }
  if (err_flag) { PKV_PRE_HD(true) } else { PKV_PRE_HD(false) }
#undef PKV_PRE_HD
#undef PKV_PRE_N
#undef PKV_PRE_K
#undef PKV_PRE_P
#undef PKV_PRE
  if (pkv_host::launch_status() != PKV_OK) return PKV_ERR_HIP;
  if (ksplit > 1) {
    pkv_pre::launch_merge(pa, row_items, head_dim, st);
    return pkv_host::launch_status();
  }
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_paged_attn_prefill_chunk(void* out, pkv_dtype out_dtype, const void* query,
                                                   const int32_t* cu_q_lens, const int32_t* chunk_offsets,
                                                   const void* key_pool, const void* value_pool,
                                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                   int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                                   int32_t causal, float scale, pkv_dtype dtype, void* workspace,
                                                   size_t workspace_bytes, int32_t* err_flag, void* stream) {
  if (dtype == PKV_DTYPE_FP8_E4M3) return PKV_ERR_UNSUPPORTED;  // FP8 pools need their scales
  return prefill_impl(out, out_dtype, query, cu_q_lens, chunk_offsets, key_pool, value_pool, block_tables,
                      max_blocks_per_seq, num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim, num_blocks, causal,
                      scale, dtype, 1.f, 1.f, workspace, workspace_bytes, err_flag, stream);
}

extern "C" size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads,
                                              int32_t head_dim, int32_t max_blocks_per_seq) {
  if (num_seqs < 0 || max_q_len < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 ||
      (head_dim != 64 && head_dim != 128 && head_dim != 256))
    return 0;
  // The row layout depends on the KV head count, which this query does not take: the bound over
  // every count that divides num_q_heads.
  size_t most = 0;
  for (int32_t hkv = 1; hkv <= num_q_heads; ++hkv) {
    if (num_q_heads % hkv != 0) continue;
    const bool pack = pkv_pre::pack_rows(max_q_len, num_q_heads, hkv);
    const int64_t row_items = static_cast<int64_t>(num_seqs) * (pack ? hkv : num_q_heads) *
                              pkv_pre::row_tiles(max_q_len, pack ? num_q_heads / hkv : 1);
    const int ksplit = pkv_pre::ksplit_for(row_items, max_blocks_per_seq, head_dim, pkv_host::cu_count());
    const size_t b = pkv_pre::layout(row_items, ksplit, head_dim).total;
    most = b > most ? b : most;
  }
  return most;
}

extern "C" pkv_status pkv_paged_attn_prefill_chunk_fp8(void* out, pkv_dtype out_dtype, const void* query,
                                                       const int32_t* cu_q_lens, const int32_t* chunk_offsets,
                                                       const void* key_pool, const void* value_pool,
                                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                       int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads,
                                                       int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                                       int32_t causal, float scale, float k_scale, float v_scale,
                                                       void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                                       void* stream) {
  return prefill_impl(out, out_dtype, query, cu_q_lens, chunk_offsets, key_pool, value_pool, block_tables,
                      max_blocks_per_seq, num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim, num_blocks, causal,
                      scale, PKV_DTYPE_FP8_E4M3, k_scale, v_scale, workspace, workspace_bytes, err_flag, stream);
}
