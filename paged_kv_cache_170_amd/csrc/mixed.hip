// Fused mixed-batch step: the decode tokens and the prefill chunks of one scheduler step in one
// attention launch.
//
// What is computed: exactly what pkv_paged_attn_decode and pkv_paged_attn_prefill_chunk compute
// for the two halves of the batch ("Phase 17 · 04 — vLLM serving internals", scheduler-loop
// section: one step carries decode tokens and prefill chunks through one forward call; "Chunked
// Prefill", Ultralytics, token-budget section: decode tokens first, then chunks).
//
// Design (gfx950): one 512-thread launch whose first workgroups are decode workers and whose
// remaining workgroups are prefill items.  A decode workgroup runs two independent persistent
// decode workers (threads 0-255 and 256-511), each with its own LDS area and an LDS-counter
// barrier, so the decode part keeps eight waves per CU as in the decode launch.  The dispatcher
// starts workgroups in index order as CUs free up (one workgroup per CU: both kinds use most of the
// LDS), so prefill items start on the CUs that the decode workers leave, with no kernel boundary
// and no drain between the two parts.  The device code is the decode and prefill kernels' own
// (decode_dev.hpp, prefill_dev.hpp): results are bit-identical to the two separate launches.
#include "decode_dev.hpp"
#include "prefill_dev.hpp"

namespace pkv {

template <int HD>
struct MixCfg {
  static constexpr int DEC = (DecCfg<HD>::LDS + 255) / 256 * 256;  // one decode worker's area
  static constexpr int PRE = PreCfg<HD>::LDS + kIdWindow * 4;      // one prefill item's area
  static constexpr int LDS = (2 * DEC + 64 > PRE ? 2 * DEC + 64 : PRE);
};

// PACK: the prefill items' row layout (prefill_body); the shared-prefix rows do not depend on it.
template <int HD, bool CHECK, bool NARROW, bool KV8, bool PACK>
__global__ __launch_bounds__(kPreThreads) void mixed_step_kernel(DecArgs da, const int2* __restrict__ pieces,
                                                                 int32_t* __restrict__ plan, int queues, int dec_wgs,
                                                                 PreArgs pa, int pre_items, int pre_first) {
  using M = MixCfg<HD>;
  __shared__ __attribute__((aligned(16))) char smem[M::LDS];
  // pre_first = 0: decode workgroups [0, dec_wgs), then the prefill items.  pre_first > 0 (a
  // multiple of 8, >= pre_items): the prefill items first, in workgroups [0, pre_first), then the
  // decode workgroups, so the dispatcher places the items before the decode workers take the CUs.
  const int b = static_cast<int>(blockIdx.x) - pre_first;  // decode workgroup index
  if (pre_first > 0 ? b >= 0 : b < dec_wgs) {
    // Two decode workers: worker h of workgroup b is worker h * dec_wgs + b of a 2 * dec_wgs grid,
    // so (dec_wgs being a multiple of 8) its index modulo 8 is still its XCD.
    const int half = threadIdx.x >> 8;
    int* tail = reinterpret_cast<int*>(smem + 2 * M::DEC);  // [counter, fetched0, fetched1, pad] per half
    if ((threadIdx.x & 255) == 0) tail[4 * half] = 0;
    __syncthreads();  // both halves pass this once, before they go separate ways
    HalfSync sync{tail + 4 * half, 0, da.err_flag};
    decode_worker<HD, CHECK, NARROW, KV8>(da, pieces, plan, queues, half * dec_wgs + b, 2 * dec_wgs,
                                          smem + half * M::DEC, tail + 4 * half + 1, sync);
  } else {
    const int id = pre_first > 0 ? static_cast<int>(blockIdx.x) : b - dec_wgs;
    if (id < pre_items)
      prefill_body<HD, CHECK, NARROW, KV8, PACK>(pa, id, pre_items, smem,
                                                 reinterpret_cast<int*>(smem + PreCfg<HD>::LDS));
  }
}

}  // namespace pkv

using namespace pkv;
using namespace pkv_dec;

void pkv_dec::launch_prefix_decode(const DecArgs& da, const int2* pieces, int32_t* plan, int queues, int dec_wgs,
                                   const PreArgs& pa, int pre_items, int32_t head_dim, bool check, bool narrow,
                                   bool kv8, hipStream_t st) {
  const int pre_first = (pre_items + 7) / 8 * 8;
  const unsigned grid = static_cast<unsigned>(pre_first + dec_wgs);
#define PKV_PXD(HD, CHECK, NARROW, KV8)                                                                        \
  hipLaunchKernelGGL((mixed_step_kernel<HD, CHECK, NARROW, KV8, false>), dim3(grid), dim3(kPreThreads), 0, st, da, \
                     pieces, plan, queues, dec_wgs, pa, pre_items, pre_first)
#define PKV_PXD_K(HD, CHECK, NARROW) \
  if (kv8) PKV_PXD(HD, CHECK, NARROW, true); else PKV_PXD(HD, CHECK, NARROW, false);
#define PKV_PXD_N(HD, CHECK) \
  if (narrow) { PKV_PXD_K(HD, CHECK, true) } else { PKV_PXD_K(HD, CHECK, false) }
#define PKV_PXD_C(HD) \
  if (check) { PKV_PXD_N(HD, true) } else { PKV_PXD_N(HD, false) }
  if (head_dim == 64) { PKV_PXD_C(64) } else { PKV_PXD_C(128) }
#undef PKV_PXD_C
#undef PKV_PXD_N
#undef PKV_PXD_K
#undef PKV_PXD
}

namespace {

bool scale_ok(float x) { return std::isfinite(x) && x > 0.f; }

}  // namespace

extern "C" pkv_status pkv_paged_attn_mixed(
    void* dec_out, const void* dec_query, const int32_t* dec_block_tables, int32_t dec_max_blocks,
    const int32_t* context_lens, int32_t num_dec_seqs, void* pre_out, const void* pre_query, const int32_t* cu_q_lens,
    const int32_t* chunk_offsets, const int32_t* pre_block_tables, int32_t pre_max_blocks, int32_t num_pre_seqs,
    int32_t max_q_len, int32_t causal, const void* key_pool, const void* value_pool, int32_t num_blocks,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale, pkv_dtype dtype, float k_scale,
    float v_scale, pkv_dtype out_dtype, int32_t split_tokens, void* workspace, size_t workspace_bytes,
    void* pre_workspace, size_t pre_workspace_bytes, int32_t* err_flag, void* stream) {
  const bool kv8 = dtype == PKV_DTYPE_FP8_E4M3;
  if (dtype != PKV_DTYPE_BF16 && !kv8) return PKV_ERR_UNSUPPORTED;
  if (kv8 && (!scale_ok(k_scale) || !scale_ok(v_scale))) return PKV_ERR_INVALID_ARG;
  if (out_dtype != PKV_DTYPE_F32 && out_dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_dec_seqs < 0 || num_pre_seqs < 0 || max_q_len < 0 || num_blocks < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || !scale_ok(scale) || num_q_heads % num_kv_heads != 0)
    return PKV_ERR_INVALID_ARG;
  if (split_tokens < 0 || split_tokens % 128 != 0 || split_tokens > 2048) return PKV_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;  // two decode workers need HD <= 128
  if (num_q_heads / num_kv_heads > kMaxGroup) return PKV_ERR_UNSUPPORTED;
  const bool has_dec = num_dec_seqs > 0, has_pre = num_pre_seqs > 0 && max_q_len > 0;
  if (!has_dec && !has_pre) return PKV_OK;
  if (!key_pool || !value_pool || num_blocks == 0) return PKV_ERR_INVALID_ARG;
  if (has_dec && (!dec_out || !dec_query || !dec_block_tables || !context_lens || dec_max_blocks <= 0))
    return PKV_ERR_INVALID_ARG;
  if (has_pre && (!pre_out || !pre_query || !cu_q_lens || !chunk_offsets || !pre_block_tables || pre_max_blocks <= 0))
    return PKV_ERR_INVALID_ARG;
  for (const void* p : {static_cast<const void*>(dec_out), dec_query, static_cast<const void*>(pre_out), pre_query,
                        key_pool, value_pool, static_cast<const void*>(workspace)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return PKV_ERR_INVALID_ARG;
  if (num_dec_seqs > 65535 || num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;

  const int group = num_q_heads / num_kv_heads;
  const float base_log2 = scale * kLog2e;
  const float scale_log2 = kv8 ? base_log2 * k_scale : base_log2;
  const float vs = kv8 ? v_scale : 1.f;
  const int ob = out_dtype == PKV_DTYPE_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool narrow = pkv_host::narrow_addressing(num_blocks, num_kv_heads, head_dim, kv8 ? 1 : 2);

  // Decode part: the same plan, workspace layout and split size as pkv_paged_attn_decode.
  int dec_wgs = 0, queues = 1, S = 0, max_splits = 1;
  DecArgs da{};
  int2* pieces = nullptr;
  int32_t* plan = nullptr;
  float *ws_o = nullptr, *ws_ml = nullptr;
  if (has_dec) {
    S = split_tokens > 0 ? split_tokens
                         : pkv_decode_split_tokens(num_dec_seqs, num_q_heads, num_kv_heads, head_dim, dec_max_blocks);
    const int64_t ms = (static_cast<int64_t>(dec_max_blocks) * kBlockSize + S - 1) / S;
    if (ms > 65535) return PKV_ERR_UNSUPPORTED;
    max_splits = static_cast<int>(ms);
    if (static_cast<int64_t>(num_dec_seqs) * max_splits * num_kv_heads > INT32_MAX / 2) return PKV_ERR_UNSUPPORTED;
    const WsLayout lay = ws_layout(num_dec_seqs, num_q_heads, head_dim, max_splits);
    if (!workspace || workspace_bytes < lay.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
    char* ws = static_cast<char*>(workspace);
    plan = reinterpret_cast<int32_t*>(ws);
    pieces = reinterpret_cast<int2*>(ws + lay.pieces);
    ws_o = max_splits > 1 ? reinterpret_cast<float*>(ws + lay.o) : nullptr;
    ws_ml = max_splits > 1 ? reinterpret_cast<float*>(ws + lay.ml) : nullptr;
    da = DecArgs{static_cast<const uint16_t*>(dec_query), key_pool, value_pool, dec_block_tables, context_lens, ws_o,
                 ws_ml, dec_out, err_flag, dec_max_blocks, num_q_heads, num_kv_heads, group, num_blocks, S,
                 max_splits, ob, scale_log2, vs, num_dec_seqs, nullptr, 0, max_splits};
    // As many workers as the decode launch has workgroups (two per CU), two per workgroup; the
    // workgroup count is a multiple of 8 so that worker indices keep their XCD.
    const int64_t max_items = static_cast<int64_t>(num_dec_seqs) * num_kv_heads * max_splits;
    const int64_t want = 2 * static_cast<int64_t>(pkv_host::cu_count());
    const int64_t workers = max_items < want ? max_items : want;
    dec_wgs = static_cast<int>((workers + 15) / 16 * 8);
    const int nworkers = 2 * dec_wgs;
    queues = nworkers % kMaxQueues == 0 ? kMaxQueues : 8;
    launch_plan(err_flag != nullptr, context_lens, num_dec_seqs, dec_max_blocks, S, pieces, plan, nworkers, queues,
                err_flag, st);
    if (pkv_host::launch_status() != PKV_OK) return PKV_ERR_HIP;
  }

  // Prefill part: the items (row tiles x key splits) of pkv_paged_attn_prefill_chunk.
  int pre_items = 0;
  int64_t pre_row_items = 0;
  bool pack = false;
  PreArgs pa{};
  if (has_pre) {
    pack = pkv_pre::pack_rows(max_q_len, num_q_heads, num_kv_heads);
    const int64_t q_tiles64 = pkv_pre::row_tiles(max_q_len, pack ? group : 1);
    if (q_tiles64 > (1 << 22)) return PKV_ERR_UNSUPPORTED;
    const int q_tiles = static_cast<int>(q_tiles64);
    const int64_t row_items = static_cast<int64_t>(num_pre_seqs) * (pack ? num_kv_heads : num_q_heads) * q_tiles;
    const int ksplit = pkv_pre::ksplit_for(row_items, pre_max_blocks, head_dim, pkv_host::cu_count());
    const int64_t items = row_items * ksplit;
    if (items + dec_wgs > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
    const pkv_pre::Layout lay = pkv_pre::layout(row_items, ksplit, head_dim);
    if (ksplit > 1 && (!pre_workspace || pre_workspace_bytes < lay.total)) return PKV_ERR_WORKSPACE_TOO_SMALL;
    if (ksplit > 1 && reinterpret_cast<uintptr_t>(pre_workspace) % 16 != 0) return PKV_ERR_INVALID_ARG;
    char* pw = static_cast<char*>(pre_workspace);
    pre_items = static_cast<int>(items);
    pa = PreArgs{static_cast<const uint16_t*>(pre_query), cu_q_lens, chunk_offsets, key_pool, value_pool,
                 pre_block_tables, pre_max_blocks, q_tiles, num_q_heads, num_kv_heads, group, num_blocks,
                 causal != 0, scale_log2, vs, pre_out, ob, err_flag, ksplit,
                 ksplit > 1 ? reinterpret_cast<float*>(pw + lay.o) : nullptr,
                 ksplit > 1 ? reinterpret_cast<float*>(pw + lay.ml) : nullptr};
    pa.pack = pack;
    pre_row_items = row_items;
  }

  const unsigned grid = static_cast<unsigned>(dec_wgs + pre_items);
#define PKV_MIX(HD, CHECK, NARROW, KV8, PACK)                                                                   \
  hipLaunchKernelGGL((mixed_step_kernel<HD, CHECK, NARROW, KV8, PACK>), dim3(grid), dim3(kPreThreads), 0, st, da, \
                     pieces, plan, queues, dec_wgs, pa, pre_items, 0)
#define PKV_MIX_P(HD, CHECK, NARROW, KV8) \
  if (pack) PKV_MIX(HD, CHECK, NARROW, KV8, true); else PKV_MIX(HD, CHECK, NARROW, KV8, false);
#define PKV_MIX_K(HD, CHECK, NARROW) \
  if (kv8) { PKV_MIX_P(HD, CHECK, NARROW, true) } else { PKV_MIX_P(HD, CHECK, NARROW, false) }
#define PKV_MIX_N(HD, CHECK) \
  if (narrow) { PKV_MIX_K(HD, CHECK, true) } else { PKV_MIX_K(HD, CHECK, false) }
#define PKV_MIX_C(HD) \
  if (err_flag) { PKV_MIX_N(HD, true) } else { PKV_MIX_N(HD, false) }
  if (head_dim == 64) { PKV_MIX_C(64) } else { PKV_MIX_C(128) }
#undef PKV_MIX_C
#undef PKV_MIX_N
#undef PKV_MIX_K
#undef PKV_MIX_P
#undef PKV_MIX
  if (pkv_host::launch_status() != PKV_OK) return PKV_ERR_HIP;
  if (has_dec && max_splits > 1) {
    launch_reduce(ws_o, ws_ml, context_lens, dec_max_blocks, num_dec_seqs, num_q_heads, num_kv_heads, head_dim, S,
                  max_splits, dec_out, ob, st);
    if (pkv_host::launch_status() != PKV_OK) return PKV_ERR_HIP;
  }
  if (has_pre && pa.ksplit > 1) {
    pkv_pre::launch_merge(pa, pre_row_items, head_dim, st);
    return pkv_host::launch_status();
  }
  return PKV_OK;
}
