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
//     (every wave-wide load covers complete rows of the KV head) and staged in LDS;
//     S^T = K Q^T uses v_mfma_f32_16x16x32_bf16 with the 16 MFMA columns holding the G query
//     heads (zero-padded), and V is read back transposed with ds_read_b64_tr_b16 as the A operand
//     of O^T = V^T P^T.
//   * the online softmax runs in the log2 domain on the MFMA accumulator layout against a
//     reference max that is raised only when a weight would pass 2^20 (so the common step needs
//     no cross-lane max); the 4 waves' states merge in LDS, and a split's (o, m, l) goes to the workspace unless the sequence
//     fits one split, in which case the normalised row is written directly.
//   * fp32 pools take a plain VALU kernel with the same split/merge structure.
#include <cstdlib>
#include <cmath>

#include "common.hpp"

namespace pkv {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kMaxGroup = 16;
constexpr float kMaxWeight = 1048576.f;  // 2^20: largest softmax weight before the reference max moves

// E: bytes per pool element (2 for bf16, 1 for E4M3 codes); staging in LDS is bf16 either way.
template <int HD, int E = 2>
struct DecCfg {
  static constexpr int KK = HD / 32;          // k-steps of S^T = K Q^T over head_dim
  static constexpr int MT = HD / 16;          // 16-row tiles of O^T
  static constexpr int KPITCH = HD * 2 + 16;  // bytes per staged K row (conflict-free 16-byte reads)
  static constexpr int VPITCH = HD * 2 + 32;  // bytes per staged V row (conflict-free transposed reads)
  static constexpr int EPL = 16 / E;          // pool elements per 16-byte lane load
  static constexpr int LPR = HD / EPL;        // lanes per row in a 16-byte-per-lane load
  static constexpr int RPL = kWave / LPR;     // rows per wave-wide load
  static constexpr int VLD = kBlockSize / RPL;  // wave-wide loads per block and tensor
  static constexpr int STAGE = 2 * kBlockSize * (KPITCH + VPITCH);  // bytes per wave (two blocks of K and V)
  static constexpr int COMB = kMaxGroup * HD * 4;                   // bytes per wave for the merge
  static constexpr int BODY = (STAGE > COMB ? STAGE : COMB) * kDecWaves;
  static constexpr int LDS = BODY + kDecWaves * kMaxGroup * 2 * 4;
};

__device__ __forceinline__ void store_out(void* out, int64_t idx, float v, bool bf16) {
  if (bf16)
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
  else
    static_cast<float*>(out)[idx] = v;
}

// Merges the per-wave states held in LDS and writes either the final rows or the split partial.
template <int HD>
__device__ __forceinline__ void merge_waves(const float* comb_o, const float* comb_ml, int group, int s, int g,
                                            int split, int nsplit, int max_splits, int num_q_heads, float* ws_o,
                                            float* ws_ml, void* out, bool out_bf16, float v_scale) {
  for (int i = threadIdx.x; i < group * HD; i += kDecThreads) {
    const int hn = i / HD, d = i - hn * HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, comb_ml[(w * kMaxGroup + hn) * 2]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = comb_ml[(w * kMaxGroup + hn) * 2];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      O += f * comb_o[(w * kMaxGroup + hn) * HD + d];
      L += f * comb_ml[(w * kMaxGroup + hn) * 2 + 1];
    }
    const int h = g * group + hn;
    const int64_t row = static_cast<int64_t>(s) * num_q_heads + h;
    // v_scale: the FP8 pool's V scale (1 for bf16 pools, where the product is exact).
    O *= v_scale;
    if (nsplit == 1) {
      store_out(out, row * HD + d, L > 0.f ? O / L : 0.f, out_bf16);
    } else {
      const int64_t part = row * max_splits + split;
      ws_o[part * HD + d] = O;
      if (d == 0) {
        ws_ml[part * 2] = M;
        ws_ml[part * 2 + 1] = L;
      }
    }
  }
}

// Clamps a context length to the table; flags it in checked mode.
template <bool CHECK>
__device__ __forceinline__ int clamp_ctx(int ctx, int max_blocks, int32_t* err_flag, bool report) {
  if (ctx < 0 || ctx > max_blocks * kBlockSize) {
    if (CHECK && report) atomicOr(err_flag, PKV_FLAG_BAD_LENGTH);
    return ctx < 0 ? 0 : max_blocks * kBlockSize;
  }
  return ctx;
}

// Kernel arguments of the bf16 decode (one struct so that every launch form shares them).
struct DecArgs {
  const uint16_t* query;
  const void* key_pool;    // bf16 or E4M3 codes
  const void* value_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_o;
  float* ws_ml;
  void* out;
  int32_t* err_flag;
  int max_blocks, num_q_heads, num_kv_heads, group, num_blocks, split_tokens, max_splits, out_bf16;
  float scale_log2;  // scale * log2(e), times the K scale for FP8 pools
  float v_scale;     // V scale of an FP8 pool, 1 for bf16
};

template <int HD, int E>
struct DecBuf {
  uint4 k[2][DecCfg<HD, E>::VLD];
  uint4 v[2][DecCfg<HD, E>::VLD];
  int b0, b1;
};

// One work item: positions [split * split_tokens, min(+split_tokens, ctx)) of sequence s, KV head g,
// for all query heads of the group.  Called by all 256 threads of the workgroup.
// What a work item needs before its first gather: where it is, its block ids (one per lane) and the
// query fragment.  Loaded one item ahead so that these reads overlap the previous item's work.
template <int HD>
struct DecItem {
  int s, g, split, ctx, nsplit;
  int my_id[2];  // block ids of the split: lane j holds blocks j and 64 + j
  bf16x8 qf[DecCfg<HD>::KK];
};

template <int HD, bool CHECK>
__device__ __forceinline__ void decode_item_prologue(const DecArgs& A_, DecItem<HD>& it) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15, c = lane >> 4;
  const int tok0 = it.split * A_.split_tokens;
  const int tok_end = min(tok0 + A_.split_tokens, it.ctx);
  const int32_t* table = A_.block_tables + static_cast<int64_t>(it.s) * A_.max_blocks;
  // The split's block ids, two per lane (a split spans at most 128 blocks).
  const int nblk_split = it.ctx > 0 ? (tok_end - tok0 + kBlockSize - 1) / kBlockSize : 0;
  const int j0 = tok0 / kBlockSize;
  it.my_id[0] = lane < nblk_split ? load_block_id<CHECK>(table, j0 + lane, A_.num_blocks, A_.err_flag) : -1;
  it.my_id[1] = lane + kWave < nblk_split ? load_block_id<CHECK>(table, j0 + kWave + lane, A_.num_blocks, A_.err_flag)
                                          : -1;
  // Q^T as the B operand: lane (n, c) holds head n, head_dim elements 32kk + 8c .. +7.
  const bool live = n < A_.group && it.ctx > 0;
  const uint16_t* qrow =
      A_.query + (static_cast<int64_t>(it.s) * A_.num_q_heads + it.g * A_.group + (live ? n : 0)) * HD + 8 * c;
#pragma unroll
  for (int kk = 0; kk < DecCfg<HD>::KK; ++kk) it.qf[kk] = live ? as_bf16x8(ld16(qrow + 32 * kk)) : bf16x8{};
}

template <int HD, bool CHECK, bool NARROW, bool KV8>
__device__ __forceinline__ void decode_bf16_item(const DecArgs& A_, const DecItem<HD>& it, char* smem) {
  constexpr int E = KV8 ? 1 : 2;  // pool bytes per element
  using C = DecCfg<HD, E>;
  const int s = it.s, g = it.g, split = it.split, ctx = it.ctx, nsplit = it.nsplit;
  const int my_id0 = it.my_id[0], my_id1 = it.my_id[1];
  const bf16x8* qf = it.qf;
  const void* __restrict__ key_pool = A_.key_pool;
  const void* __restrict__ value_pool = A_.value_pool;
  const int num_q_heads = A_.num_q_heads, num_kv_heads = A_.num_kv_heads, group = A_.group;
  const int num_blocks = A_.num_blocks, split_tokens = A_.split_tokens;
  const float scale_log2 = A_.scale_log2;
  int32_t* err_flag = A_.err_flag;

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n = lane & 15, c = lane >> 4;
  const int tok0 = split * split_tokens;
  const int tok_end = min(tok0 + split_tokens, ctx);

  float m_ref = -INFINITY, l_run = 0.f;
  floatx4 acc[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  char* kstage = smem + wave * C::STAGE;                      // [32 rows][KPITCH]
  char* vstage = kstage + 2 * kBlockSize * C::KPITCH;         // [32 rows][VPITCH]
  const int units = (tok_end - tok0 + 31) / 32;
  const int row_base = lane / C::LPR, col = (lane % C::LPR) * C::EPL;  // col: first element of the lane

  // Step u covers positions tok0 + 32u .. +31 (two blocks).  K and V rows are read whole (each
  // wave-wide load covers RPL complete rows) and staged in LDS in their natural layout.
  const uint32_t blk_bytes = static_cast<uint32_t>(kBlockSize * num_kv_heads * HD * E);
  const uint32_t row_bytes = static_cast<uint32_t>(num_kv_heads * HD * E);
  const uint32_t c0 = static_cast<uint32_t>((row_base * num_kv_heads + g) * HD * E + col * E);
  auto load = [&](int u, DecBuf<HD, E>& B) {
    const int t0 = tok0 + 32 * u;
    // Blocks 2u and 2u + 1 of the split (u is the same across the wave).
    const int idreg = u < kWave / 2 ? my_id0 : my_id1;
    const int lane_b = (2 * u) & (kWave - 1);
    B.b0 = __builtin_amdgcn_readlane(idreg, lane_b);
    B.b1 = (t0 + kBlockSize < ctx) ? __builtin_amdgcn_readlane(idreg, lane_b + 1) : -1;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const int b = pg ? B.b1 : B.b0;
#pragma unroll
      for (int i = 0; i < C::VLD; ++i) {
        if (b >= 0) {
          const uint32_t cb = c0 + static_cast<uint32_t>(i * C::RPL) * row_bytes;
          B.k[pg][i] = ld16_nt(pool_at<NARROW>(key_pool, b, blk_bytes, cb));
          B.v[pg][i] = ld16_nt(pool_at<NARROW>(value_pool, b, blk_bytes, cb));
        } else {
          B.k[pg][i] = uint4{0, 0, 0, 0};
          B.v[pg][i] = uint4{0, 0, 0, 0};
        }
      }
    }
  };

  auto compute = [&](int u, const DecBuf<HD, E>& B) {
    const int t0 = tok0 + 32 * u;
    // Stage K and V as bf16 (V rows at or past ctx become zero so stale slots never reach the
    // MFMA).  E4M3 codes are converted exactly on the way.
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int i = 0; i < C::VLD; ++i) {
        const int row = pg * kBlockSize + i * C::RPL + row_base;
        const uint4 vv = (t0 + row < ctx) ? B.v[pg][i] : uint4{0, 0, 0, 0};
        if constexpr (KV8) {
          uint4 lo, hi;
          e4m3x16_to_bf16(B.k[pg][i], lo, hi);
          st16(kstage + row * C::KPITCH + col * 2, lo);
          st16(kstage + row * C::KPITCH + col * 2 + 16, hi);
          e4m3x16_to_bf16(vv, lo, hi);
          st16(vstage + row * C::VPITCH + col * 2, lo);
          st16(vstage + row * C::VPITCH + col * 2 + 16, hi);
        } else {
          st16(kstage + row * C::KPITCH + col * 2, B.k[pg][i]);
          st16(vstage + row * C::VPITCH + col * 2, vv);
        }
      }
    // The staged rows are read back by this wave only; keep the compiler from moving reads up.
    __asm__ volatile("" ::: "memory");
    // S^T = K Q^T for both blocks: lane (n, c) gets head n, tokens 4c .. 4c+3 of each block.
    floatx4 sacc[2];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const char* krow = kstage + (pg * kBlockSize + n) * C::KPITCH + 16 * c;
      sacc[pg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(krow), qf[0],
                                                         floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int kk = 1; kk < C::KK; ++kk)
        sacc[pg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(krow + 64 * kk), qf[kk],
                                                           sacc[pg], 0, 0, 0);
    }
    // Online softmax (log2 domain, scale folded into the exponent's FMA).  The reference max m_ref
    // trails the running max and is raised only when a weight would pass 2^20 (or before the first
    // key), so the common path needs no cross-lane max.
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const bool blk_ok = (pg ? B.b1 : B.b0) >= 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = t0 + pg * kBlockSize + 4 * c + j;
        sacc[pg][j] = (blk_ok && tok < ctx) ? sacc[pg][j] : -INFINITY;
      }
    }
    uint32_t pw[4];
    auto expo = [&]() {
      // A head that has seen no valid key yet keeps m_ref = -inf; its scores are used as they are.
      const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float p0 = fast_exp2(__builtin_fmaf(sacc[pg][2 * q], scale_log2, neg_m));
          const float p1 = fast_exp2(__builtin_fmaf(sacc[pg][2 * q + 1], scale_log2, neg_m));
          pw[2 * pg + q] = pack_bf16x2(p0, p1);
        }
      return add_bf16x2(pw[0], add_bf16x2(pw[1], add_bf16x2(pw[2], add_bf16x2(pw[3], 0.f))));
    };
    float ps = expo();
    if (__any(!(ps < kMaxWeight) || m_ref == -INFINITY)) {
      float mx = -INFINITY;
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sacc[pg][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = mx * scale_log2;
      const bool up = m_new > m_ref;
      const float alpha = up ? (m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - m_new)) : 1.f;
      m_ref = up ? m_new : m_ref;
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) acc[mt] *= alpha;
      ps = expo();
    }
    l_run += ps;
    const bf16x8 pb = __builtin_bit_cast(bf16x8, uint4{pw[0], pw[1], pw[2], pw[3]});

    // O^T += V^T P^T.  A operand: lane (n, c) needs V[token 4c+e][d = 16mt + n] of both blocks.
    const uint16_t* r0 = reinterpret_cast<const uint16_t*>(vstage + (4 * c + (n >> 2)) * C::VPITCH) + 4 * (n & 3);
    const uint16_t* r1 = r0 + kBlockSize * (C::VPITCH / 2);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      const bf16x8 a = concat(lds_read_tr16(r0 + 16 * mt), lds_read_tr16(r1 + 16 * mt));
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[mt], 0, 0, 0);
    }
    __asm__ volatile("" ::: "memory");
  };

  DecBuf<HD, E> A;
  for (int u = wave; u < units; u += kDecWaves) {
    load(u, A);
    compute(u, A);
  }

  // Normaliser of head n: sum the four lane groups.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  __syncthreads();  // every wave is done with its staging area
  float* comb_o = reinterpret_cast<float*>(smem);
  float* comb_ml = reinterpret_cast<float*>(smem + C::BODY);
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
    *reinterpret_cast<floatx4*>(comb_o + (wave * kMaxGroup + n) * HD + 16 * mt + 4 * c) = acc[mt];
  if (c == 0) {
    comb_ml[(wave * kMaxGroup + n) * 2] = m_ref;
    comb_ml[(wave * kMaxGroup + n) * 2 + 1] = l_run;
  }
  __syncthreads();
  merge_waves<HD>(comb_o, comb_ml, group, s, g, split, nsplit, A_.max_splits, num_q_heads, A_.ws_o, A_.ws_ml, A_.out,
                  A_.out_bf16, A_.v_scale);
}

// Work plan of the persistent decode.  A piece is one (sequence, split) pair; its length in
// 32-token steps is at most split_tokens / 32.  One workgroup sorts the pieces longest first (a
// counting sort on that length: full splits first, then the sequences' last splits by length; an
// empty sequence counts as one step) into `pieces` as {sequence << 16 | split, context length},
// stores their number in the plan header and sets the fetch counters.  Longest-first order with
// dynamic fetching keeps the workgroups' finishing times within about one short piece.
//
// Items: item i is piece i / Hkv for KV head i % Hkv.  Workgroup b of the persistent grid draws
// from queue q = b % queues the items q, q + queues, q + 2 queues, ...; its first two are items b
// and b + grid (no fetch), the rest come from queue q's counter, which the plan starts at
// 2 * grid / queues.  Each counter sits on its own 128-byte line.
constexpr int kPlanThreads = 1024;
constexpr int kMaxQueues = 64;
constexpr int kCounterStride = 32;  // ints: one 128-byte line per counter
constexpr int kPlanTotal = kMaxQueues * kCounterStride;
constexpr int kPlanInts = kPlanTotal + kCounterStride;
constexpr int kMaxClasses = 2048 / 32 + 1;

template <bool CHECK>
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(const int32_t* __restrict__ context_lens,
                                                                   int num_seqs, int max_blocks, int split_tokens,
                                                                   int2* __restrict__ pieces,
                                                                   int32_t* __restrict__ plan, int grid, int queues,
                                                                   int32_t* err_flag) {
  __shared__ int count[kMaxClasses];
  __shared__ int cursor[kMaxClasses];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int top = split_tokens / 32;  // class of a full split (<= 64)
  if (tid < kMaxClasses) count[tid] = 0;
  __syncthreads();
  for (int s = tid; s < num_seqs; s += kPlanThreads) {
    const int ctx = clamp_ctx<CHECK>(context_lens[s], max_blocks, err_flag, true);
    const int full = ctx / split_tokens, rem = ctx - full * split_tokens;
    if (full) atomicAdd(&count[top], full);
    if (rem || !ctx) atomicAdd(&count[rem ? (rem + 31) / 32 : 1], 1);
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
    const int ctx = clamp_ctx<false>(context_lens[s], max_blocks, nullptr, false);
    const int full = ctx / split_tokens, rem = ctx - full * split_tokens;
    const int tag = static_cast<int>(static_cast<uint32_t>(s) << 16);
    if (full) {
      const int at = atomicAdd(&cursor[top], full);
      for (int k = 0; k < full; ++k) pieces[at + k] = int2{tag | k, ctx};
    }
    if (rem || !ctx) pieces[atomicAdd(&cursor[rem ? (rem + 31) / 32 : 1], 1)] = int2{tag | full, ctx};
  }
}

// Persistent form: a fixed grid takes work items from the plan (see above).  With queues a
// multiple of 8 and workgroups dealt round-robin over the 8 XCDs, queue q runs on XCD q % 8 and
// holds only items with i % 8 == q % 8, so with Hkv = 8 each KV head stays on one XCD and blocks
// shared between sequences stay in that XCD's L2.  The item after next is fetched while the
// current item runs; the next item's block ids and query are loaded then too.
template <int HD, bool CHECK, bool NARROW, bool KV8>
__global__ __launch_bounds__(kDecThreads) void decode_bf16_kernel(DecArgs a, const int2* __restrict__ pieces,
                                                                  int32_t* __restrict__ plan, int queues) {
  __shared__ __attribute__((aligned(16))) char smem[DecCfg<HD>::LDS];
  __shared__ int fetched[2];
  const int tid = threadIdx.x;
  const int queue = blockIdx.x % queues;
  const int total = plan[kPlanTotal] * a.num_kv_heads;
  auto find = [&](int item, DecItem<HD>& it) {
    const int piece = item / a.num_kv_heads;
    const int2 code = pieces[piece];
    it.s = static_cast<int>(static_cast<uint32_t>(code.x) >> 16);
    it.split = code.x & 0xffff;
    it.g = item - piece * a.num_kv_heads;
    it.ctx = code.y;
    it.nsplit = (it.ctx + a.split_tokens - 1) / a.split_tokens;
  };
  int cur_i = blockIdx.x, nxt_i = blockIdx.x + gridDim.x;
  if (cur_i >= total) return;  // uniform over the workgroup
  DecItem<HD> cur, nxt;
  find(cur_i, cur);
  decode_item_prologue<HD, CHECK>(a, cur);
  // `fetched` alternates slots: slot p is written before the barrier that ends an item and read
  // right after it; the next write to slot p comes after one more barrier.
  for (int p = 0;; p ^= 1) {
    const bool have_next = nxt_i < total;
    int after = total;
    if (have_next) {
      if (tid == 0) after = atomicAdd(&plan[queue * kCounterStride], 1) * queues + queue;  // returns while this item runs
      find(nxt_i, nxt);
      decode_item_prologue<HD, CHECK>(a, nxt);  // in flight while this item runs
    }
    if (cur.ctx == 0) {
      for (int i = tid; i < a.group * HD; i += kDecThreads)
        store_out(a.out, (static_cast<int64_t>(cur.s) * a.num_q_heads + cur.g * a.group) * HD + i, 0.f, a.out_bf16);
    } else {
      decode_bf16_item<HD, CHECK, NARROW, KV8>(a, cur, smem);
    }
    if (tid == 0) fetched[p] = after;
    __syncthreads();  // the next item reuses the staging and merge areas; fetched[p] is published
    if (!have_next) break;
    cur = nxt;
    nxt_i = fetched[p];
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
  constexpr int COMB = kMaxGroup * HD * 4 * kDecWaves;
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
    for (int k = 0; k < DPL; ++k) comb_o[(wave * kMaxGroup + hn) * HD + lane + kWave * k] = o[hn][k];
    if (lane == 0) {
      comb_ml[(wave * kMaxGroup + hn) * 2] = m_run[hn];
      comb_ml[(wave * kMaxGroup + hn) * 2 + 1] = l_run[hn];
    }
  }
  __syncthreads();
  merge_waves<HD>(comb_o, comb_ml, group, s, g, split, nsplit, max_splits, num_q_heads, ws_o, ws_ml, out, out_bf16,
                  1.f);
}

// Log-sum-exp merge of split partials: grid (num_kv_heads, num_seqs); the 256 threads cover the
// group's query heads x head_dim.  Sequences that fit one split were finished by the main kernel.
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ ws_o,
                                                            const float* __restrict__ ws_ml,
                                                            const int32_t* __restrict__ context_lens, int max_blocks,
                                                            int num_q_heads, int group, int head_dim,
                                                            int split_tokens, int max_splits, void* __restrict__ out,
                                                            int out_bf16) {
  const int g = blockIdx.x, s = blockIdx.y;
  int ctx = context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > max_blocks * kBlockSize ? max_blocks * kBlockSize : ctx);
  const int nsplit = (ctx + split_tokens - 1) / split_tokens;
  if (nsplit <= 1) return;
  // Each thread owns four consecutive head_dim elements of one query head (16-byte loads).
  const int quads = head_dim / 4;
  for (int i = threadIdx.x; i < group * quads; i += blockDim.x) {
    const int hn = i / quads, d = 4 * (i - hn * quads);
    const int h = g * group + hn;
    const int64_t base = (static_cast<int64_t>(s) * num_q_heads + h) * max_splits;
    // One pass with a running max; the loads of a batch of splits are independent and issue together.
    float M = -INFINITY, L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < nsplit; p0 += 8) {
      float2 ml[8];
      float4 op[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool live = p0 + k < nsplit;
        const int64_t part = base + (live ? p0 + k : p0);
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

bool shapes_ok(int32_t num_seqs, int32_t hq, int32_t hkv, int32_t hd, int32_t max_blocks) {
  return num_seqs >= 0 && hq > 0 && hkv > 0 && hq % hkv == 0 && hq / hkv <= kMaxGroup &&
         (hd == 64 || hd == 128 || hd == 256) && max_blocks > 0;
}

int32_t resolve_split(int32_t requested, int32_t num_seqs, int32_t hq, int32_t hkv, int32_t hd, int32_t max_blocks) {
  if (requested > 0) return requested;
  return pkv_decode_split_tokens(num_seqs, hq, hkv, hd, max_blocks);
}

// Workspace: the plan (header ints, then 8 bytes per (sequence, split) piece), then, when a
// sequence can span several splits, the fp32 partial rows [num_seqs][hq][max_splits][hd] and
// their (max, normaliser) pairs.  Every part starts on a 256-byte boundary.
struct WsLayout {
  size_t pieces, o, ml, total;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

WsLayout ws_layout(int32_t num_seqs, int32_t hq, int32_t hd, int64_t max_splits) {
  WsLayout w;
  w.pieces = round256(kPlanInts * 4);
  w.o = w.pieces + round256(static_cast<size_t>(num_seqs) * max_splits * 8);
  const size_t rows = max_splits > 1 ? static_cast<size_t>(num_seqs) * hq * max_splits : 0;
  w.ml = w.o + round256(rows * hd * 4);
  w.total = w.ml + rows * 2 * 4;
  return w;
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
              scale_log2, kv8 ? v_scale : 1.f};
    // Two resident workgroups per CU at head_dim <= 128 (register bound), one at 256; never more
    // workgroups than the largest possible number of items.
    const int64_t max_items = static_cast<int64_t>(num_seqs) * num_kv_heads * max_splits;
    const int64_t resident = static_cast<int64_t>(pkv_host::cu_count()) * (head_dim <= 128 ? 2 : 1);
    const unsigned nwg = static_cast<unsigned>(max_items < resident ? max_items : resident);
    const int queues = nwg % kMaxQueues == 0 ? kMaxQueues : (nwg % 8 == 0 ? 8 : 1);
    const bool narrow = static_cast<uint64_t>(num_blocks) * kBlockSize * num_kv_heads * head_dim * (kv8 ? 1 : 2) <
                            (1ull << 32) &&
                        num_blocks < (1 << 24);
    if (err_flag)
      hipLaunchKernelGGL((decode_plan_kernel<true>), dim3(1), dim3(kPlanThreads), 0, st, context_lens, num_seqs,
                         max_blocks_per_seq, S, pieces, plan, static_cast<int>(nwg), queues, err_flag);
    else
      hipLaunchKernelGGL((decode_plan_kernel<false>), dim3(1), dim3(kPlanThreads), 0, st, context_lens, num_seqs,
                         max_blocks_per_seq, S, pieces, plan, static_cast<int>(nwg), queues, err_flag);
    if (pkv_host::launch_status() != PKV_OK) return PKV_ERR_HIP;
#define PKV_DEC_BF16(HD, CHECK, NARROW, KV8)                                                                    \
  hipLaunchKernelGGL((decode_bf16_kernel<HD, CHECK, NARROW, KV8>), dim3(nwg), dim3(kDecThreads), 0, st, a, pieces, \
                     plan, queues)
#define PKV_DEC_BF16_K(HD, CHECK, NARROW) \
  if (kv8) PKV_DEC_BF16(HD, CHECK, NARROW, true); else PKV_DEC_BF16(HD, CHECK, NARROW, false);
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
  } else {
    if (err_flag) { PKV_DEC_HD(decode_f32_kernel, float, true) } else { PKV_DEC_HD(decode_f32_kernel, float, false) }
  }
#undef PKV_DEC_HD
#undef PKV_DEC
  if (pkv_host::launch_status() != PKV_OK) return PKV_ERR_HIP;
  if (max_splits > 1) {
    hipLaunchKernelGGL(decode_reduce_kernel, dim3(num_kv_heads, num_seqs), dim3(256), 0, st, ws_o, ws_ml,
                       context_lens, max_blocks_per_seq, num_q_heads, group, head_dim, S, max_splits, out, ob);
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
