// One-token paged decode with split-KV partition and log-sum-exp combine.
//
// What is computed: for each sequence s and query head h, softmax attention of q[s][h] over the
// sequence's cached positions 0 .. ctx_s - 1 of KV head h / G ("Chunked Prefill", Ultralytics,
// section on prefill and decode: decode reads the whole cache every step).  The pages' paged
// kernel ("第2章:推理引擎核心技术", §1.4) walks the request's pages through its table and keeps an
// online softmax; here the walk is split over workgroups and the partial states are merged.
//
// Design (gfx950, wave64):
//   * a persistent grid walks the compact list of (sequence, split, KV head) items (built on the
//     device from context_lens, so no workgroup is launched idle); a workgroup of 4 waves owns
//     `split_tokens` positions of one (sequence, KV head) and serves all G query heads of that
//     group from each loaded page.
//   * a wave step covers 32 positions = two 16-token blocks.  K and V rows are fetched whole
//     (every wave-wide load covers complete rows of the KV head) with non-temporal loads, except
//     blocks the neighbouring sequence also holds at the same logical index (a shared prefix,
//     "第2章:推理引擎核心技术" §1.5), which are read normally so that they stay in L2 for the other
//     sequences; rows are staged in LDS;
//     S^T = K Q^T uses v_mfma_f32_16x16x32_bf16 with the 16 MFMA columns holding the G query
//     heads (zero-padded), and V is read back transposed with ds_read_b64_tr_b16 as the A operand
//     of O^T = V^T P^T.
//   * the online softmax runs in the log2 domain on the MFMA accumulator layout against a
//     reference max that is raised only when a weight would pass 2^20 (so the common step needs
//     no cross-lane max); the 4 waves' states merge in LDS, and a split's (o, m, l) goes to the workspace unless the sequence
//     fits one split, in which case the normalised row is written directly.
//   * fp32 pools take a plain VALU kernel with the same split/merge structure.
//   * pkv_paged_attn_decode_prefix: the members of a shared prefix (§1.5) get the prefix attended
//     once per KV head by MFMA prefix items placed in front of the decode workers of the same
//     launch (mixed.hip); the reduce merges those partials with the members' own splits.
#include <atomic>
#include <mutex>

#include "decode_dev.hpp"
#include "prefill_dev.hpp"

namespace pkv {

// Shared-prefix decode (members != null): the plan first marks the member sequences in
// member_out; a member's pieces then cover its positions after the prefix_blocks shared blocks
// (a member whose context ends with the prefix gets no piece: the prefix partial is its result).
template <bool CHECK>
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(const int32_t* __restrict__ context_lens,
                                                                   int num_seqs, int max_blocks, int split_tokens,
                                                                   int2* __restrict__ pieces,
                                                                   int32_t* __restrict__ plan, int grid, int queues,
                                                                   int32_t* err_flag, const int32_t* __restrict__ members,
                                                                   int num_members, int prefix_blocks,
                                                                   uint8_t* __restrict__ member_out) {
  __shared__ int count[kMaxClasses];
  __shared__ int cursor[kMaxClasses];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int top = split_tokens / 32;  // class of a full split (<= 64)
  if (tid < kMaxClasses) count[tid] = 0;
  if (members != nullptr) {
    for (int s = tid; s < num_seqs; s += kPlanThreads) member_out[s] = 0;
    __syncthreads();
    for (int i = tid; i < num_members; i += kPlanThreads) {
      const int m = members[i];
      if (m >= 0 && m < num_seqs) member_out[m] = 1;
    }
  }
  __syncthreads();
  // Context of the pieces: the whole context, or a member's positions past the prefix.
  auto piece_ctx = [&](int s, bool report, bool& member) {
    int ctx = clamp_ctx<CHECK>(context_lens[s], max_blocks, err_flag, report);
    member = members != nullptr && member_out[s];
    if (member) {
      ctx -= prefix_blocks * kBlockSize;
      if (ctx < 0) {
        if (CHECK && report) atomicOr(err_flag, PKV_FLAG_BAD_LENGTH);
        ctx = 0;
      }
    }
    return ctx;
  };
  for (int s = tid; s < num_seqs; s += kPlanThreads) {
    bool member;
    const int ctx = piece_ctx(s, true, member);
    const int full = ctx / split_tokens, rem = ctx - full * split_tokens;
    if (full) atomicAdd(&count[top], full);
    if (rem || (!ctx && !member)) atomicAdd(&count[rem ? (rem + 31) / 32 : 1], 1);
  }
  __syncthreads();
  if (tid < kWave) {
    // Classes top, top - 1, ..., 1 on lanes 0, 1, ...: exclusive prefix sum over the wave.
    const int c = top - lane;
    const int n = c >= 1 ? count[c] : 0;
    int incl = n;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (c >= 1) cursor[c] = incl - n;
    if (lane == kWave - 1) plan[kPlanTotal] = incl;
  }
  if (tid < queues) plan[tid * kCounterStride] = 2 * (grid / queues);
  __syncthreads();
  for (int s = tid; s < num_seqs; s += kPlanThreads) {
    bool member;
    const int ctx = piece_ctx(s, false, member);
    const int full = ctx / split_tokens, rem = ctx - full * split_tokens;
    const int tag = static_cast<int>(static_cast<uint32_t>(s) << 16);
    if (full) {
      const int at = atomicAdd(&cursor[top], full);
      for (int k = 0; k < full; ++k) pieces[at + k] = int2{tag | k, ctx};
    }
    if (rem || (!ctx && !member)) pieces[atomicAdd(&cursor[rem ? (rem + 31) / 32 : 1], 1)] = int2{tag | full, ctx};
  }
}

// Persistent decode kernel: one worker per workgroup (see decode_worker).
// PLANNED false: a small batch without a plan pass (see decode_worker).
template <int HD, bool CHECK, bool NARROW, bool KV8, bool PLANNED>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(HD > 128 ? 1 : 2))) void decode_bf16_kernel(DecArgs a, const int2* __restrict__ pieces,
                                                                  int32_t* __restrict__ plan, int queues) {
  __shared__ __attribute__((aligned(16))) char smem[DecCfg<HD>::LDS];
  __shared__ int fetched[2];
  WgSync sync;
  if constexpr (PLANNED) {
    decode_worker<HD, CHECK, NARROW, KV8>(a, pieces, plan, queues, blockIdx.x, gridDim.x, smem, fetched, sync);
  } else {
    __shared__ int scan[2 * kWave];
    decode_worker<HD, CHECK, NARROW, KV8, false>(a, pieces, plan, queues, blockIdx.x, gridDim.x, smem, fetched, sync,
                                                 scan);
  }
}

// fp32 pools: VALU kernel.  A wave step covers 32 positions; lanes 0-31 and 32-63 each take one
// position and half of head_dim for the scores, then lanes span head_dim for P V.
template <int HD, bool CHECK>
__global__ __launch_bounds__(kDecThreads) void decode_f32_kernel(
    const float* __restrict__ query, const float* __restrict__ key_pool, const float* __restrict__ value_pool,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ context_lens,
    int num_q_heads, int num_kv_heads, int group, int num_blocks, float scale_log2, int split_tokens, int max_splits,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, void* __restrict__ out, int out_bf16, int32_t* err_flag) {
  constexpr int DPL = HD / kWave;  // head_dim elements per lane in P V
  constexpr int HALF = HD / 2;
  constexpr int CP = DecCfg<HD>::CPITCH;  // merge row pitch in floats (merge_waves reads this layout)
  constexpr int COMB = kMaxGroup * CP * 4 * kDecWaves;
  __shared__ __attribute__((aligned(16))) char smem[COMB + kDecWaves * kMaxGroup * 2 * 4 + kMaxGroup * HD * 4];
  float* q_lds = reinterpret_cast<float*>(smem + COMB + kDecWaves * kMaxGroup * 2 * 4);

  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int ctx = clamp_ctx<CHECK>(context_lens[s], max_blocks, err_flag, split == 0 && g == 0 && threadIdx.x == 0);
  const int nsplit = (ctx + split_tokens - 1) / split_tokens;
  if (ctx == 0) {
    if (split != 0) return;
    for (int i = threadIdx.x; i < group * HD; i += kDecThreads)
      store_out(out, (static_cast<int64_t>(s) * num_q_heads + g * group) * HD + i, 0.f, out_bf16);
    return;
  }
  if (split >= nsplit) return;
  for (int i = threadIdx.x; i < group * HD; i += kDecThreads)
    q_lds[i] = query[(static_cast<int64_t>(s) * num_q_heads + g * group) * HD + i];
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int tl = lane & 31, half = lane >> 5;
  const int tok0 = split * split_tokens;
  const int tok_end = min(tok0 + split_tokens, ctx);
  const int32_t* table = block_tables + static_cast<int64_t>(s) * max_blocks;

  float m_run[kMaxGroup], l_run[kMaxGroup], o[kMaxGroup][DPL];
#pragma unroll
  for (int hn = 0; hn < kMaxGroup; ++hn) {
    m_run[hn] = -INFINITY;
    l_run[hn] = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[hn][k] = 0.f;
  }

  const int units = (tok_end - tok0 + 31) / 32;
  for (int u = wave; u < units; u += kDecWaves) {
    const int t0 = tok0 + 32 * u;
    const int j0 = t0 / kBlockSize;
    const bool has1 = t0 + kBlockSize < ctx;
    const int b0 = load_block_id<CHECK>(table, j0, num_blocks, err_flag);
    const int b1 = has1 ? load_block_id<CHECK>(table, j0 + 1, num_blocks, err_flag) : -1;
    const int tok = t0 + tl;
    const int bt = tl < kBlockSize ? b0 : b1;
    const bool valid = tok < ctx && bt >= 0;

    float sc[kMaxGroup];
#pragma unroll
    for (int hn = 0; hn < kMaxGroup; ++hn) sc[hn] = 0.f;
    if (valid) {
      const float* krow = key_pool + pool_row_offset(bt, tok % kBlockSize, num_kv_heads, g, HD) + half * HALF;
      for (int d = 0; d < HALF; d += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(krow + d);
#pragma unroll
        for (int hn = 0; hn < kMaxGroup; ++hn) {
          if (hn < group) {
            const float* qv = q_lds + hn * HD + half * HALF + d;
            sc[hn] += qv[0] * kv.x + qv[1] * kv.y + qv[2] * kv.z + qv[3] * kv.w;
          }
        }
      }
    }
    float p[kMaxGroup];
#pragma unroll
    for (int hn = 0; hn < kMaxGroup; ++hn) {
      if (hn >= group) continue;
      const float full = sc[hn] + __shfl_xor(sc[hn], 32);
      const float xv = valid ? full * scale_log2 : -INFINITY;
      float mx = xv;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_new = fmaxf(m_run[hn], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[hn] - m_use);
      const float pv = fast_exp2(xv - m_use);
      float ps = pv;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) ps += __shfl_xor(ps, off);
      l_run[hn] = l_run[hn] * alpha + ps;
      m_run[hn] = m_new;
      p[hn] = pv;
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[hn][k] *= alpha;
    }
    const int nt = min(32, ctx - t0);
    for (int tt = 0; tt < nt; ++tt) {
      const int b = tt < kBlockSize ? b0 : b1;
      if (b < 0) continue;
      const float* vrow = value_pool + pool_row_offset(b, (t0 + tt) % kBlockSize, num_kv_heads, g, HD);
      float vv[DPL];
#pragma unroll
      for (int k = 0; k < DPL; ++k) vv[k] = vrow[lane + kWave * k];
#pragma unroll
      for (int hn = 0; hn < kMaxGroup; ++hn) {
        if (hn >= group) continue;
        const float w = __shfl(p[hn], tt);
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[hn][k] += w * vv[k];
      }
    }
  }

  __syncthreads();
  float* comb_o = reinterpret_cast<float*>(smem);
  float* comb_ml = reinterpret_cast<float*>(smem + COMB);
#pragma unroll
  for (int hn = 0; hn < kMaxGroup; ++hn) {
    if (hn >= group) continue;
#pragma unroll
    for (int k = 0; k < DPL; ++k) comb_o[(wave * kMaxGroup + hn) * CP + lane + kWave * k] = o[hn][k];
    if (lane == 0) {
      comb_ml[(wave * kMaxGroup + hn) * 2] = m_run[hn];
      comb_ml[(wave * kMaxGroup + hn) * 2 + 1] = l_run[hn];
    }
  }
  __syncthreads();
  merge_waves<HD>(comb_o, comb_ml, group, s, g, split, nsplit == 1, max_splits, num_q_heads, ws_o, ws_ml, out,
                  out_bf16, 1.f);
}

// Log-sum-exp merge of split partials: grid (num_kv_heads, num_seqs); the 256 threads cover the
// group's query heads x head_dim.  Sequences that fit one split were finished by the main kernel.
// Shared-prefix decode (member != null): a member's parts are its splits past the prefix (slots
// 0 .. nsplit - 1) and the prefix_parts prefix partials (slots prefix_slot0 ..), always merged.
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ ws_o,
                                                            const float* __restrict__ ws_ml,
                                                            const int32_t* __restrict__ context_lens, int max_blocks,
                                                            int num_q_heads, int group, int head_dim,
                                                            int split_tokens, int slots, void* __restrict__ out,
                                                            int out_bf16, const uint8_t* __restrict__ member,
                                                            int prefix_blocks, int prefix_slot0, int prefix_parts) {
  const int g = blockIdx.x, s = blockIdx.y;
  int ctx = context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > max_blocks * kBlockSize ? max_blocks * kBlockSize : ctx);
  const bool is_member = member != nullptr && member[s];
  if (is_member) ctx = max(ctx - prefix_blocks * kBlockSize, 0);
  const int nsplit = (ctx + split_tokens - 1) / split_tokens;
  if (!is_member && nsplit <= 1) return;
  const int nparts = nsplit + (is_member ? prefix_parts : 0);
  // Each thread owns four consecutive head_dim elements of one query head (16-byte loads).
  const int quads = head_dim / 4;
  for (int i = threadIdx.x; i < group * quads; i += blockDim.x) {
    const int hn = i / quads, d = 4 * (i - hn * quads);
    const int h = g * group + hn;
    const int64_t base = (static_cast<int64_t>(s) * num_q_heads + h) * slots;
    // One pass with a running max; the loads of a batch of parts are independent and issue together.
    float M = -INFINITY, L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < nparts; p0 += 8) {
      float2 ml[8];
      float4 op[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool live = p0 + k < nparts;
        const int pk = live ? p0 + k : p0;
        const int64_t part = base + (pk < nsplit ? pk : prefix_slot0 + pk - nsplit);
        ml[k] = *reinterpret_cast<const float2*>(ws_ml + part * 2);
        if (!live) ml[k].x = -INFINITY;
        op[k] = *reinterpret_cast<const float4*>(ws_o + part * head_dim + d);
      }
      float Mn = M;
#pragma unroll
      for (int k = 0; k < 8; ++k) Mn = fmaxf(Mn, ml[k].x);
      if (Mn == -INFINITY) continue;
      const float sc = (M == -INFINITY) ? 0.f : fast_exp2(M - Mn);
      O.x *= sc;
      O.y *= sc;
      O.z *= sc;
      O.w *= sc;
      L *= sc;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float f = (ml[k].x == -INFINITY) ? 0.f : fast_exp2(ml[k].x - Mn);
        O.x += f * op[k].x;
        O.y += f * op[k].y;
        O.z += f * op[k].z;
        O.w += f * op[k].w;
        L += f * ml[k].y;
      }
      M = Mn;
    }
    if (L > 0.f) {
      O.x /= L;
      O.y /= L;
      O.z /= L;
      O.w /= L;
    } else {
      O = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int64_t o = (static_cast<int64_t>(s) * num_q_heads + h) * head_dim + d;
    if (out_bf16)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = uint2{pack_bf16x2(O.x, O.y), pack_bf16x2(O.z, O.w)};
    else
      *reinterpret_cast<float4*>(static_cast<float*>(out) + o) = O;
  }
}

}  // namespace pkv

using namespace pkv;
using namespace pkv_dec;

void pkv_dec::launch_plan(bool check, const int32_t* context_lens, int num_seqs, int max_blocks, int split_tokens,
                          int2* pieces, int32_t* plan, int grid, int queues, int32_t* err_flag, hipStream_t st,
                          const int32_t* members, int num_members, int prefix_blocks, uint8_t* member_out) {
  if (check)
    hipLaunchKernelGGL((decode_plan_kernel<true>), dim3(1), dim3(kPlanThreads), 0, st, context_lens, num_seqs,
                       max_blocks, split_tokens, pieces, plan, grid, queues, err_flag, members, num_members,
                       prefix_blocks, member_out);
  else
    hipLaunchKernelGGL((decode_plan_kernel<false>), dim3(1), dim3(kPlanThreads), 0, st, context_lens, num_seqs,
                       max_blocks, split_tokens, pieces, plan, grid, queues, err_flag, members, num_members,
                       prefix_blocks, member_out);
}

void pkv_dec::launch_reduce(const float* ws_o, const float* ws_ml, const int32_t* context_lens, int max_blocks,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int split_tokens,
                            int slots, void* out, int out_bf16, hipStream_t st, const uint8_t* member,
                            int prefix_blocks, int prefix_slot0, int prefix_parts) {
  hipLaunchKernelGGL(decode_reduce_kernel, dim3(num_kv_heads, num_seqs), dim3(256), 0, st, ws_o, ws_ml, context_lens,
                     max_blocks, num_q_heads, num_q_heads / num_kv_heads, head_dim, split_tokens, slots, out,
                     out_bf16, member, prefix_blocks, prefix_slot0, prefix_parts);
}

namespace {

int env_split_tokens() {
  static const int v = [] {
    const char* e = std::getenv("PKV_SPLIT_TOKENS");
    if (!e) return 0;
    const int x = std::atoi(e);
    return (x > 0 && x % 128 == 0 && x <= 2048) ? x : 0;
  }();
  return v;
}

int32_t resolve_split(int32_t requested, int32_t num_seqs, int32_t hq, int32_t hkv, int32_t hd, int32_t max_blocks) {
  if (requested > 0) return requested;
  return pkv_decode_split_tokens(num_seqs, hq, hkv, hd, max_blocks);
}

}  // namespace

extern "C" int32_t pkv_decode_split_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t max_blocks_per_seq) {
  if (const int e = env_split_tokens()) return e;
  if (!shapes_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq)) return 512;
  const int64_t max_ctx = static_cast<int64_t>(max_blocks_per_seq) * kBlockSize;
  const int64_t pairs = static_cast<int64_t>(num_seqs) * num_kv_heads;
  // Prefer long splits (fewer partials, fewer merges; the longest-first dynamic schedule evens
  // out the workgroups) while the largest possible number of work items still covers every
  // resident workgroup of a 256-CU device (two per CU at head_dim <= 128, one at 256).
  const int64_t resident = head_dim <= 128 ? 512 : 256;
  for (int S : {2048, 1024, 512, 256})
    if (pairs * ((max_ctx + S - 1) / S) >= resident) return S;
  return 128;
}

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t max_blocks_per_seq, int32_t split_tokens) {
  if (!shapes_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq)) return 0;
  if (split_tokens < 0 || split_tokens % 128 != 0 || split_tokens > 2048) return 0;
  const int32_t S = resolve_split(split_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq);
  const int64_t max_splits = (static_cast<int64_t>(max_blocks_per_seq) * kBlockSize + S - 1) / S;
  return ws_layout(num_seqs, num_q_heads, head_dim, max_splits).total;
}

namespace {

// Shared body of the bf16 / fp32 and FP8 decode calls.  dtype is the pool dtype (FP8_E4M3 pools take
// bf16 queries and the two scales).
pkv_status decode_impl(void* out, pkv_dtype out_dtype, const void* query, const void* key_pool,
                       const void* value_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t num_blocks, float scale, pkv_dtype dtype, float k_scale,
                       float v_scale, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                       int32_t* err_flag, void* stream) {
  const bool kv8 = dtype == PKV_DTYPE_FP8_E4M3;
  if (kv8 && (!std::isfinite(k_scale) || !(k_scale > 0.f) || !std::isfinite(v_scale) || !(v_scale > 0.f)))
    return PKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0 || num_kv_heads <= 0)
    return PKV_ERR_INVALID_ARG;
  if (split_tokens < 0 || split_tokens % 128 != 0 || split_tokens > 2048) return PKV_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return PKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (!shapes_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq)) return PKV_ERR_UNSUPPORTED;
  if (dtype != PKV_DTYPE_F32 && dtype != PKV_DTYPE_BF16 && !kv8) return PKV_ERR_UNSUPPORTED;
  if (out_dtype != PKV_DTYPE_F32 && out_dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (num_seqs > 65535 || num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;  // grid y/z limits
  if (!out || !query || !key_pool || !value_pool || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  for (const void* p : {static_cast<const void*>(out), query, key_pool, value_pool, static_cast<const void*>(workspace)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return PKV_ERR_INVALID_ARG;
  const int32_t S = resolve_split(split_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq);
  const int64_t max_splits64 = (static_cast<int64_t>(max_blocks_per_seq) * kBlockSize + S - 1) / S;
  if (max_splits64 > 65535) return PKV_ERR_UNSUPPORTED;
  const int max_splits = static_cast<int>(max_splits64);
  // Work items index pieces x KV heads in int32.
  if (static_cast<int64_t>(num_seqs) * max_splits * num_kv_heads > INT32_MAX / 2) return PKV_ERR_UNSUPPORTED;
  const WsLayout lay = ws_layout(num_seqs, num_q_heads, head_dim, max_splits);
  if (!workspace || workspace_bytes < lay.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  char* ws = static_cast<char*>(workspace);
  int32_t* plan = reinterpret_cast<int32_t*>(ws);
  int2* pieces = reinterpret_cast<int2*>(ws + lay.pieces);
  float* ws_o = max_splits > 1 ? reinterpret_cast<float*>(ws + lay.o) : nullptr;
  float* ws_ml = max_splits > 1 ? reinterpret_cast<float*>(ws + lay.ml) : nullptr;
  const int group = num_q_heads / num_kv_heads;
  const float scale_log2 = kv8 ? scale * kLog2e * k_scale : scale * kLog2e;
  const int ob = out_dtype == PKV_DTYPE_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  dim3 grid(max_splits, num_kv_heads, num_seqs);

#define PKV_DEC(KERNEL, T, HD, CHECK)                                                                              \
  hipLaunchKernelGGL((KERNEL<HD, CHECK>), grid, dim3(kDecThreads), 0, st, static_cast<const T*>(query),            \
                     static_cast<const T*>(key_pool), static_cast<const T*>(value_pool), block_tables,             \
                     max_blocks_per_seq, context_lens, num_q_heads, num_kv_heads, group, num_blocks, scale_log2, S, \
                     max_splits, ws_o, ws_ml, out, ob, err_flag)
#define PKV_DEC_HD(KERNEL, T, CHECK)                 \
  switch (head_dim) {                                \
    case 64: PKV_DEC(KERNEL, T, 64, CHECK); break;   \
    case 128: PKV_DEC(KERNEL, T, 128, CHECK); break; \
    default: PKV_DEC(KERNEL, T, 256, CHECK); break;  \
  }
  if (dtype == PKV_DTYPE_BF16 || kv8) {
    DecArgs a{static_cast<const uint16_t*>(query), key_pool, value_pool, block_tables, context_lens, ws_o, ws_ml, out,
              err_flag, max_blocks_per_seq, num_q_heads, num_kv_heads, group, num_blocks, S, max_splits, ob,
              scale_log2, kv8 ? v_scale : 1.f, num_seqs, nullptr, 0, max_splits};
    // Two resident workgroups per CU at head_dim <= 128 (register bound), one at 256; never more
    // workgroups than the largest possible number of items.
    const int64_t max_items = static_cast<int64_t>(num_seqs) * num_kv_heads * max_splits;
    const int64_t resident = static_cast<int64_t>(pkv_host::cu_count()) * (head_dim <= 128 ? 2 : 1);
    const unsigned nwg = static_cast<unsigned>(max_items < resident ? max_items : resident);
    const int queues = nwg % kMaxQueues == 0 ? kMaxQueues : (nwg % 8 == 0 ? 8 : 1);
    const bool narrow = pkv_host::narrow_addressing(num_blocks, num_kv_heads, head_dim, kv8 ? 1 : 2);
    // A small batch whose every possible item has a workgroup of its own needs no plan: each
    // workgroup finds its item from the context lengths, and the plan launch is saved.
    const bool planned = !(num_seqs <= kWave && max_items <= resident);
    if (planned) {
      launch_plan(err_flag != nullptr, context_lens, num_seqs, max_blocks_per_seq, S, pieces, plan,
                  static_cast<int>(nwg), queues, err_flag, st);
      if (pkv_host::launch_status() != PKV_OK) return PKV_ERR_HIP;
    }
#define PKV_DEC_BF16P(HD, CHECK, NARROW, KV8, PLANNED)                                                            \
  hipLaunchKernelGGL((decode_bf16_kernel<HD, CHECK, NARROW, KV8, PLANNED>), dim3(nwg), dim3(kDecThreads), 0, st, a, \
                     pieces, plan, queues)
#define PKV_DEC_BF16(HD, CHECK, NARROW, KV8) \
  if (planned) PKV_DEC_BF16P(HD, CHECK, NARROW, KV8, true); else PKV_DEC_BF16P(HD, CHECK, NARROW, KV8, false);
#define PKV_DEC_BF16_K(HD, CHECK, NARROW) \
  if (kv8) { PKV_DEC_BF16(HD, CHECK, NARROW, true) } else { PKV_DEC_BF16(HD, CHECK, NARROW, false) }
#define PKV_DEC_BF16_N(HD, CHECK) \
  if (narrow) { PKV_DEC_BF16_K(HD, CHECK, true) } else { PKV_DEC_BF16_K(HD, CHECK, false) }
#define PKV_DEC_BF16_C(HD) \
  if (err_flag) { PKV_DEC_BF16_N(HD, true) } else { PKV_DEC_BF16_N(HD, false) }
    switch (head_dim) {
      case 64: PKV_DEC_BF16_C(64) break;
      case 128: PKV_DEC_BF16_C(128) break;
      default: PKV_DEC_BF16_C(256) break;
    }
#undef PKV_DEC_BF16_C
#undef PKV_DEC_BF16_N
#undef PKV_DEC_BF16_K
#undef PKV_DEC_BF16
#undef PKV_DEC_BF16P
  } else {
    if (err_flag) { PKV_DEC_HD(decode_f32_kernel, float, true) } else { PKV_DEC_HD(decode_f32_kernel, float, false) }
  }
#undef PKV_DEC_HD
#undef PKV_DEC
  if (pkv_host::launch_status() != PKV_OK) return PKV_ERR_HIP;
  if (max_splits > 1) {
    launch_reduce(ws_o, ws_ml, context_lens, max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim, S,
                  max_splits, out, ob, st);
    return pkv_host::launch_status();
  }
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_paged_attn_decode(void* out, pkv_dtype out_dtype, const void* query, const void* key_pool,
                                            const void* value_pool, const int32_t* block_tables,
                                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t num_blocks, float scale, pkv_dtype dtype,
                                            int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                            int32_t* err_flag, void* stream) {
  if (dtype == PKV_DTYPE_FP8_E4M3) return PKV_ERR_UNSUPPORTED;  // FP8 pools need their scales
  return decode_impl(out, out_dtype, query, key_pool, value_pool, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, scale, dtype, 1.f, 1.f, split_tokens,
                     workspace, workspace_bytes, err_flag, stream);
}

extern "C" pkv_status pkv_paged_attn_decode_fp8(void* out, pkv_dtype out_dtype, const void* query,
                                                const void* key_pool, const void* value_pool,
                                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                                float scale, float k_scale, float v_scale, int32_t split_tokens,
                                                void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                                void* stream) {
  return decode_impl(out, out_dtype, query, key_pool, value_pool, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, scale, PKV_DTYPE_FP8_E4M3, k_scale,
                     v_scale, split_tokens, workspace, workspace_bytes, err_flag, stream);
}

// ---------------------------------------------------------------------------------------------
// Shared-prefix decode.  Member sequences share their first prefix_blocks physical blocks (a
// cached prefix, [Engine-core] §1.5 / §3.2).  The prefix is attended once per KV head for all
// members together: the prefill kernel in shared-prefix mode takes the (member, query head) pairs
// as its rows and writes one (o, m, l) partial per key split; the decode then covers each member's
// positions past the prefix, and the reduce merges both (log-sum-exp combine, the same identity
// as the split reduce).  Non-members are decoded as by pkv_paged_attn_decode.

namespace {

struct PfxLayout {
  WsLayout base;
  size_t member, total;
  int slots, max_splits;
};

PfxLayout pfx_layout(int32_t num_seqs, int32_t hq, int32_t hd, int32_t max_blocks, int32_t S) {
  PfxLayout l;
  l.max_splits = static_cast<int>((static_cast<int64_t>(max_blocks) * kBlockSize + S - 1) / S);
  l.slots = l.max_splits + kPreMaxSplit;
  l.base = ws_layout(num_seqs, hq, hd, l.slots);
  l.member = round256(l.base.total);
  l.total = l.member + round256(static_cast<size_t>(num_seqs));
  return l;
}

}  // namespace

extern "C" size_t pkv_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                    int32_t head_dim, int32_t max_blocks_per_seq,
                                                    int32_t split_tokens) {
  if (!shapes_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq)) return 0;
  if (split_tokens < 0 || split_tokens % 128 != 0 || split_tokens > 2048) return 0;
  const int32_t S = resolve_split(split_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq);
  return pfx_layout(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, S).total;
}

namespace {

// Body of the bf16 and FP8 shared-prefix calls (dtype = pool dtype; queries are bf16; the scales
// are 1 for bf16 pools).
pkv_status decode_prefix_impl(void* out, pkv_dtype out_dtype, const void* query, const void* key_pool,
                              const void* value_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, float scale, pkv_dtype dtype,
                              float k_scale, float v_scale, const int32_t* prefix_members, int32_t num_members,
                              int32_t prefix_blocks, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                              int32_t* err_flag, void* stream) {
  const bool kv8 = dtype == PKV_DTYPE_FP8_E4M3;
  if (out_dtype != PKV_DTYPE_F32 && out_dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_blocks < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_members < 0 || prefix_blocks < 0 || prefix_blocks > max_blocks_per_seq || num_members > num_seqs)
    return PKV_ERR_INVALID_ARG;
  if (split_tokens < 0 || split_tokens % 128 != 0 || split_tokens > 2048) return PKV_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return PKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (!shapes_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq)) return PKV_ERR_UNSUPPORTED;
  if (head_dim > 128) return PKV_ERR_UNSUPPORTED;  // the prefix pass uses the prefill kernel's key splits
  if (num_seqs == 0) return PKV_OK;
  if (num_seqs > 65535 || num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;
  if (!out || !query || !key_pool || !value_pool || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  if (num_members > 0 && prefix_blocks > 0 && !prefix_members) return PKV_ERR_INVALID_ARG;
  for (const void* p : {static_cast<const void*>(out), query, key_pool, value_pool, static_cast<const void*>(workspace)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return PKV_ERR_INVALID_ARG;
  const int32_t S = resolve_split(split_tokens, num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq);
  const PfxLayout lay = pfx_layout(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, S);
  if (!workspace || workspace_bytes < lay.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  // No shared prefix: the ordinary decode (its layout fits in this one).
  if (num_members == 0 || prefix_blocks == 0)
    return kv8 ? pkv_paged_attn_decode_fp8(out, out_dtype, query, key_pool, value_pool, block_tables,
                                           max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                                           head_dim, num_blocks, scale, k_scale, v_scale, S, workspace,
                                           workspace_bytes, err_flag, stream)
               : pkv_paged_attn_decode(out, out_dtype, query, key_pool, value_pool, block_tables,
                                       max_blocks_per_seq, context_lens, num_seqs, num_q_heads, num_kv_heads,
                                       head_dim, num_blocks, scale, dtype, S, workspace, workspace_bytes, err_flag,
                                       stream);
  if (static_cast<int64_t>(num_seqs) * lay.max_splits * num_kv_heads > INT32_MAX / 2) return PKV_ERR_UNSUPPORTED;
  char* ws = static_cast<char*>(workspace);
  int32_t* plan = reinterpret_cast<int32_t*>(ws);
  int2* pieces = reinterpret_cast<int2*>(ws + lay.base.pieces);
  float* ws_o = reinterpret_cast<float*>(ws + lay.base.o);
  float* ws_ml = reinterpret_cast<float*>(ws + lay.base.ml);
  uint8_t* member = reinterpret_cast<uint8_t*>(ws + lay.member);
  const int group = num_q_heads / num_kv_heads;
  const float scale_log2 = scale * kLog2e * k_scale;  // the K scale folds into the exponent
  const int ob = out_dtype == PKV_DTYPE_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool check = err_flag != nullptr;
  const bool narrow = pkv_host::narrow_addressing(num_blocks, num_kv_heads, head_dim, kv8 ? 1 : 2);

  // Prefix pass: rows (member, query head) of each KV head, key splits of the prefix.
  const int q_tiles = static_cast<int>((static_cast<int64_t>(num_members) * group + kPreTile - 1) / kPreTile);
  const int64_t row_items = static_cast<int64_t>(q_tiles) * num_kv_heads;
  // Key splits of the prefix: enough items to fill the chip, but each split adds a partial per
  // (member, query head) that is written and read back (M*G*hd*8 bytes per KV head against the
  // prefix's 64*P*hd); halve the splits while that traffic exceeds four times the prefix's.
  int kp = pkv_pre::ksplit_for(row_items, prefix_blocks, head_dim, pkv_host::cu_count());
  while (kp > 1 && static_cast<int64_t>(kp) * num_members * group > 32 * static_cast<int64_t>(prefix_blocks)) kp /= 2;
  PreArgs pa{};
  pa.query = static_cast<const uint16_t*>(query);
  pa.key_pool = key_pool;
  pa.value_pool = value_pool;
  pa.block_tables = block_tables;
  pa.max_blocks = max_blocks_per_seq;
  pa.q_tiles = q_tiles;
  pa.num_q_heads = num_q_heads;
  pa.num_kv_heads = num_kv_heads;
  pa.group = group;
  pa.num_blocks = num_blocks;
  pa.causal = 0;
  pa.scale_log2 = scale_log2;
  pa.v_scale = v_scale;
  pa.err_flag = err_flag;
  pa.ksplit = kp;
  pa.ws_o = ws_o;
  pa.ws_ml = ws_ml;
  pa.prefix_members = prefix_members;
  pa.num_members = num_members;
  pa.prefix_blocks = prefix_blocks;
  pa.prefix_slots = lay.slots;
  pa.prefix_slot0 = lay.max_splits;
  pa.prefix_num_seqs = num_seqs;
  // Plan: members marked, their pieces past the prefix; as many decode workers as the decode
  // launch has workgroups (two per CU), two per 512-thread workgroup, the workgroup count a
  // multiple of 8 so that worker indices keep their XCD.
  const int64_t max_items = static_cast<int64_t>(num_seqs) * num_kv_heads * lay.max_splits;
  const int64_t want = 2 * static_cast<int64_t>(pkv_host::cu_count());
  const int64_t workers = max_items < want ? max_items : want;
  const int dec_wgs = static_cast<int>((workers + 15) / 16 * 8);
  const int nworkers = 2 * dec_wgs;
  const int queues = nworkers % kMaxQueues == 0 ? kMaxQueues : 8;
  launch_plan(check, context_lens, num_seqs, max_blocks_per_seq, S, pieces, plan, nworkers, queues, err_flag, st,
              prefix_members, num_members, prefix_blocks, member);
  if (pkv_host::launch_status() != PKV_OK) return PKV_ERR_HIP;

  // One launch: the prefix items, then the decode of everything else (every member item leaves a
  // partial), then the reduce merges both.
  const DecArgs a{static_cast<const uint16_t*>(query), key_pool, value_pool, block_tables, context_lens, ws_o, ws_ml,
                  out, err_flag, max_blocks_per_seq, num_q_heads, num_kv_heads, group, num_blocks, S, lay.max_splits,
                  ob, scale_log2, v_scale, num_seqs, member, prefix_blocks, lay.slots};
  const int64_t pre_items = row_items * kp;
  if (pre_items + dec_wgs + 8 > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  launch_prefix_decode(a, pieces, plan, queues, dec_wgs, pa, static_cast<int>(pre_items), head_dim, check, narrow,
                       kv8, st);
  if (pkv_host::launch_status() != PKV_OK) return PKV_ERR_HIP;
  launch_reduce(ws_o, ws_ml, context_lens, max_blocks_per_seq, num_seqs, num_q_heads, num_kv_heads, head_dim, S,
                lay.slots, out, ob, st, member, prefix_blocks, lay.max_splits, kp);
  return pkv_host::launch_status();
}

}  // namespace

extern "C" pkv_status pkv_paged_attn_decode_prefix(void* out, pkv_dtype out_dtype, const void* query,
                                                   const void* key_pool, const void* value_pool,
                                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                   const int32_t* context_lens, int32_t num_seqs,
                                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                   int32_t num_blocks, float scale, pkv_dtype dtype,
                                                   const int32_t* prefix_members, int32_t num_members,
                                                   int32_t prefix_blocks, int32_t split_tokens, void* workspace,
                                                   size_t workspace_bytes, int32_t* err_flag, void* stream) {
  if (dtype != PKV_DTYPE_BF16) return PKV_ERR_UNSUPPORTED;
  return decode_prefix_impl(out, out_dtype, query, key_pool, value_pool, block_tables, max_blocks_per_seq,
                            context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, scale, dtype,
                            1.f, 1.f, prefix_members, num_members, prefix_blocks, split_tokens, workspace,
                            workspace_bytes, err_flag, stream);
}

extern "C" pkv_status pkv_paged_attn_decode_prefix_fp8(void* out, pkv_dtype out_dtype, const void* query,
                                                       const void* key_pool, const void* value_pool,
                                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                       const int32_t* context_lens, int32_t num_seqs,
                                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                       int32_t num_blocks, float scale, float k_scale, float v_scale,
                                                       const int32_t* prefix_members, int32_t num_members,
                                                       int32_t prefix_blocks, int32_t split_tokens, void* workspace,
                                                       size_t workspace_bytes, int32_t* err_flag, void* stream) {
  if (!std::isfinite(k_scale) || !(k_scale > 0.f) || !std::isfinite(v_scale) || !(v_scale > 0.f))
    return PKV_ERR_INVALID_ARG;
  return decode_prefix_impl(out, out_dtype, query, key_pool, value_pool, block_tables, max_blocks_per_seq,
                            context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, scale,
                            PKV_DTYPE_FP8_E4M3, k_scale, v_scale, prefix_members, num_members, prefix_blocks,
                            split_tokens, workspace, workspace_bytes, err_flag, stream);
}

// ---------------------------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).  The work plan and the split
// partials live in `scratch`, a file-scope device array of PKV_NOALLOC_SCRATCH_BYTES: every GPU the
// library runs on holds its own copy until the process ends, and every call on that GPU shares it.
// Host code never passes `scratch` itself (its host-side name is not a device address): the
// array's address on each device is resolved once, with that device current, on the first call
// there, and that pointer is what the kernels receive.  Nothing in it must start at zero: the plan
// pass rewrites the header, the counters and the piece list on every call.

static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (resolved once per device).
pkv_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return PKV_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
        (void)hipGetLastError();  // leave no error behind for the caller's next HIP call
        return PKV_ERR_HIP;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_paged_attn_decode_noalloc(void* out, pkv_dtype out_dtype, const void* query,
                                                    const void* key_pool, const void* value_pool,
                                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                    const int32_t* context_lens, int32_t num_seqs,
                                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t num_blocks, float scale, pkv_dtype dtype,
                                                    int32_t split_tokens, int32_t* err_flag, void* stream) {
  if (dtype == PKV_DTYPE_FP8_E4M3) return PKV_ERR_UNSUPPORTED;  // FP8 pools need their scales
  const size_t need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                                 split_tokens);
  if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH_TOO_SMALL;
  // Invalid shapes (need == 0) and empty batches are answered by the argument checks alone.
  if (need == 0 || num_seqs == 0)
    return decode_impl(out, out_dtype, query, key_pool, value_pool, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, scale, dtype, 1.f, 1.f, split_tokens,
                       nullptr, 0, err_flag, stream);
  void* ws = nullptr;
  const pkv_status st = scratch_address(&ws);
  if (st != PKV_OK) return st;
  return decode_impl(out, out_dtype, query, key_pool, value_pool, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, scale, dtype, 1.f, 1.f, split_tokens,
                     ws, PKV_NOALLOC_SCRATCH_BYTES, err_flag, stream);
}
