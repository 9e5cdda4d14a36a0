// Device side of the one-token paged decode (see decode.hip for what is computed and the design),
// shared by the decode kernels and the fused mixed-step kernel.
#pragma once

#include <cstdlib>
#include <cmath>
#include <type_traits>

#include "common.hpp"

namespace pkv {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kMaxGroup = 16;

// E: bytes per pool element (2 for bf16, 1 for E4M3 codes); staging in LDS is bf16 either way.
template <int HD, int E = 2>
struct DecCfg {
  static constexpr int KK = HD / 32;          // k-steps of S^T = K Q^T over head_dim
  static constexpr int MT = HD / 16;          // 16-row tiles of O^T
  static constexpr int KPITCH = HD * 2 + 32;  // bytes per staged K row (no LDS bank conflicts on the
                                              // staging writes or the 16-byte reads: counter-checked)
  static constexpr int VPITCH = HD * 2 + 32;  // bytes per staged V row (conflict-free transposed reads)
  static constexpr int EPL = 16 / E;          // pool elements per 16-byte lane load
  static constexpr int LPR = HD / EPL;        // lanes per row in a 16-byte-per-lane load
  static constexpr int RPL = kWave / LPR;     // rows per wave-wide load
  static constexpr int VLD = kBlockSize / RPL;  // wave-wide loads per block and tensor
  static constexpr int STAGE = 2 * kBlockSize * (KPITCH + VPITCH);  // bytes per wave (two blocks of K and V)
  static constexpr int CPITCH = HD + 4;  // floats per merge row: 4 more than HD, so the 16 rows a
                                        // wave stores at once fall in different LDS banks
  static constexpr int COMB = kMaxGroup * CPITCH * 4;               // bytes per wave for the merge
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
// comb_o holds wave w's row of query head hn at (w * kMaxGroup + hn) * DecCfg<HD>::CPITCH floats.
// slots: partial slots per (sequence, query head) row of the workspace; final: the item is the
// sequence's only part (one split and no shared-prefix partial), so it writes the normalised row.
template <int HD>
__device__ __forceinline__ void merge_waves(const float* comb_o, const float* comb_ml, int group, int s, int g,
                                            int split, bool final, int slots, int num_q_heads, float* ws_o,
                                            float* ws_ml, void* out, bool out_bf16, float v_scale) {
  for (int i = threadIdx.x & (kDecThreads - 1); i < group * HD; i += kDecThreads) {
    const int hn = i / HD, d = i - hn * HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, comb_ml[(w * kMaxGroup + hn) * 2]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = comb_ml[(w * kMaxGroup + hn) * 2];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      O += f * comb_o[(w * kMaxGroup + hn) * DecCfg<HD>::CPITCH + d];
      L += f * comb_ml[(w * kMaxGroup + hn) * 2 + 1];
    }
    const int h = g * group + hn;
    const int64_t row = static_cast<int64_t>(s) * num_q_heads + h;
    // v_scale: the FP8 pool's V scale (1 for bf16 pools, where the product is exact).
    O *= v_scale;
    if (final) {
      store_out(out, row * HD + d, L > 0.f ? O / L : 0.f, out_bf16);
    } else {
      const int64_t part = row * slots + split;
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
struct PreArgs;  // prefill_dev.hpp

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
  int num_seqs;
  // Shared-prefix decode (member != null): member[s] marks the sequences whose first
  // prefix_blocks blocks are the shared prefix; their items cover the positions after it (their
  // table rows and contexts are read past it) and always write partials, which the reduce merges
  // with the prefix partials.  slots: partial slots per (sequence, query head) row.
  const uint8_t* member;
  int prefix_blocks, slots;
};

template <int HD, int E>
struct DecBuf {
  uint4 k[2][DecCfg<HD, E>::VLD];
  uint4 v[2][DecCfg<HD, E>::VLD];
  int b0, b1;
};

// One work item: positions [split * split_tokens, min(+split_tokens, ctx)) of sequence s, KV head g,
// for all query heads of the group.  Called by all 256 threads of the workgroup.
// What a work item needs before its first gather: where it is and its block ids (one per lane).
// Loaded one item ahead so that these reads overlap the previous item's work.
template <int HD>
struct DecItem {
  int s, g, split, ctx, nsplit;
  int tbl0;  // first logical block of the item's table view (the prefix length for members, else 0)
  int my_id[2];   // block ids of the split: lane j holds blocks j and 64 + j
  int ref_id[2];  // the neighbouring sequence's ids at the same logical blocks (-2: none)
};

template <int HD, bool CHECK>
__device__ __forceinline__ void decode_item_prologue(const DecArgs& A_, DecItem<HD>& it) {
  const int lane = threadIdx.x & (kWave - 1);
  const int tok0 = it.split * A_.split_tokens;
  const int tok_end = min(tok0 + A_.split_tokens, it.ctx);
  const int32_t* table = A_.block_tables + static_cast<int64_t>(it.s) * A_.max_blocks + it.tbl0;
  // The split's block ids, two per lane (a split spans at most 128 blocks).
  const int nblk_split = it.ctx > 0 ? (tok_end - tok0 + kBlockSize - 1) / kBlockSize : 0;
  const int j0 = tok0 / kBlockSize;
  it.my_id[0] = lane < nblk_split ? load_block_id<CHECK>(table, j0 + lane, A_.num_blocks, A_.err_flag) : -1;
  it.my_id[1] = lane + kWave < nblk_split ? load_block_id<CHECK>(table, j0 + kWave + lane, A_.num_blocks, A_.err_flag)
                                          : -1;
  // The neighbouring sequence's ids (the previous one, or the second for the first): a block it
  // has at the same logical index is shared (a cached prefix), and is read with a temporal hint so
  // that it stays in L2 for the other sequences; a false match only changes the hint.
  const int ref = it.s > 0 ? it.s - 1 : 1;
  if (ref < A_.num_seqs) {
    const int32_t* rt = A_.block_tables + static_cast<int64_t>(ref) * A_.max_blocks + it.tbl0;
    it.ref_id[0] = lane < nblk_split ? rt[j0 + lane] : -2;
    it.ref_id[1] = lane + kWave < nblk_split ? rt[j0 + kWave + lane] : -2;
  } else {
    it.ref_id[0] = it.ref_id[1] = -2;
  }
}

// sync: barrier of the 256 threads running the item (the whole workgroup, or one half of a
// 512-thread workgroup in the fused mixed-step kernel).
// on_start: called by every thread once this wave's first gather is issued (the worker fetches
// its next item there, so those reads queue behind the gather rather than ahead of it).
template <int HD, bool CHECK, bool NARROW, bool KV8, class Sync, class OnStart>
__device__ __forceinline__ void decode_bf16_item(const DecArgs& A_, const DecItem<HD>& it, char* smem, Sync& sync,
                                                 OnStart&& on_start) {
  constexpr int E = KV8 ? 1 : 2;  // pool bytes per element
  using C = DecCfg<HD, E>;
  const int s = it.s, g = it.g, split = it.split, ctx = it.ctx, nsplit = it.nsplit;
  const int my_id0 = it.my_id[0], my_id1 = it.my_id[1];
  const int ref_id0 = it.ref_id[0], ref_id1 = it.ref_id[1];
  bf16x8 qf[DecCfg<HD>::KK];  // the query, loaded once the item's first gather is issued (below)
  const void* __restrict__ key_pool = A_.key_pool;
  const void* __restrict__ value_pool = A_.value_pool;
  const int num_q_heads = A_.num_q_heads, num_kv_heads = A_.num_kv_heads, group = A_.group;
  const int split_tokens = A_.split_tokens;
  const float scale_log2 = A_.scale_log2;

  const int lane = threadIdx.x & (kWave - 1), wave = (threadIdx.x / kWave) & (kDecWaves - 1);
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
  // The KV head's 16 rows of a block are one contiguous run (head-major blocks).
  const uint32_t row_bytes = static_cast<uint32_t>(HD * E);
  const uint32_t c0 = static_cast<uint32_t>((g * kBlockSize + row_base) * HD * E + col * E);
  auto load = [&](int u, DecBuf<HD, E>& B) {
    const int t0 = tok0 + 32 * u;
    // Blocks 2u and 2u + 1 of the split (u is the same across the wave).
    const int idreg = u < kWave / 2 ? my_id0 : my_id1;
    const int lane_b = (2 * u) & (kWave - 1);
    B.b0 = __builtin_amdgcn_readlane(idreg, lane_b);
    B.b1 = (t0 + kBlockSize < ctx) ? __builtin_amdgcn_readlane(idreg, lane_b + 1) : -1;
    // Private blocks are streamed (non-temporal); a step whose first block is shared is not.
    auto fill = [&](auto temporal) {
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) {
        const int b = pg ? B.b1 : B.b0;
#pragma unroll
        for (int i = 0; i < C::VLD; ++i) {
          if (b >= 0) {
            const uint32_t cb = c0 + static_cast<uint32_t>(i * C::RPL) * row_bytes;
            const char* kp = pool_at<NARROW>(key_pool, b, blk_bytes, cb);
            const char* vp = pool_at<NARROW>(value_pool, b, blk_bytes, cb);
            B.k[pg][i] = decltype(temporal)::value ? ld16(kp) : ld16_nt(kp);
            B.v[pg][i] = decltype(temporal)::value ? ld16(vp) : ld16_nt(vp);
          } else {
            B.k[pg][i] = uint4{0, 0, 0, 0};
            B.v[pg][i] = uint4{0, 0, 0, 0};
          }
        }
      }
    };
    const int refreg = u < kWave / 2 ? ref_id0 : ref_id1;
    if (B.b0 >= 0 && __builtin_amdgcn_readlane(refreg, lane_b) == B.b0)
      fill(std::true_type{});
    else
      fill(std::false_type{});
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
  if (wave < units) load(wave, A);
  {
    // Q^T as the B operand: lane (n, c) holds head n, head_dim elements 32kk + 8c .. +7.  Columns
    // n >= G repeat head G - 1 (their results are never written), so the loads need no select.
    // Issued behind the first gather, the query arrives before that gather does; not carrying it
    // over from the previous item keeps 16 (head_dim 128) to 32 registers free.
    const int hn = min(n, group - 1);
    const uint16_t* qrow = A_.query + (static_cast<int64_t>(s) * num_q_heads + g * group + hn) * HD + 8 * c;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) qf[kk] = as_bf16x8(ld16(qrow + 32 * kk));
  }
  on_start();
  if constexpr (KV8) {
    // E4M3 pools: a step's gathers are half the bytes of a bf16 step, so a wave keeps two steps in
    // flight (the next step's gathers are issued before this step is computed).  bf16 pools
    // already have enough bytes in flight, and a second buffer would push them into scratch.
    DecBuf<HD, E> B2;
    for (int u = wave; u < units; u += 2 * kDecWaves) {
      if (u + kDecWaves < units) load(u + kDecWaves, B2);
      compute(u, A);
      if (u + kDecWaves >= units) break;
      if (u + 2 * kDecWaves < units) load(u + 2 * kDecWaves, A);
      compute(u + kDecWaves, B2);
    }
  } else {
    for (int u = wave; u < units; u += kDecWaves) {
      if (u != wave) load(u, A);
      compute(u, A);
    }
  }

  // Normaliser of head n: sum the four lane groups.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  sync();  // every wave is done with its staging area
  float* comb_o = reinterpret_cast<float*>(smem);
  float* comb_ml = reinterpret_cast<float*>(smem + C::BODY);
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
    *reinterpret_cast<floatx4*>(comb_o + (wave * kMaxGroup + n) * C::CPITCH + 16 * mt + 4 * c) = acc[mt];
  if (c == 0) {
    comb_ml[(wave * kMaxGroup + n) * 2] = m_ref;
    comb_ml[(wave * kMaxGroup + n) * 2 + 1] = l_run;
  }
  sync();
  // A shared-prefix member always leaves a partial: the reduce merges it with the prefix's.
  const bool final = nsplit == 1 && it.tbl0 == 0;
  merge_waves<HD>(comb_o, comb_ml, group, s, g, split, final, A_.slots, num_q_heads, A_.ws_o, A_.ws_ml, A_.out,
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

// Persistent form: a fixed grid takes work items from the plan (see above).  With queues a
// multiple of 8 and workgroups dealt round-robin over the 8 XCDs, queue q runs on XCD q % 8 and
// holds only items with i % 8 == q % 8, so with Hkv = 8 each KV head stays on one XCD and blocks
// shared between sequences stay in that XCD's L2.  The item after next is fetched while the
// current item runs; the next item's block ids are loaded then too.
// worker / nworkers: this worker's index in the persistent grid and the grid's size (the workgroup
// index and count, or two workers per workgroup in the fused mixed-step kernel); smem holds
// DecCfg<HD>::LDS bytes and fetched two ints, both private to the worker.
// PLANNED false (no plan pass; at most 64 sequences, no shared-prefix members, and a worker for every
// possible item, so that each worker runs at most one item): the worker finds its item from the
// context lengths itself — sequence-major pieces, item i = piece i / Hkv, KV head i % Hkv — through a
// prefix sum of the pieces per sequence kept in `scan` (2 x 64 ints of LDS).
template <int HD, bool CHECK, bool NARROW, bool KV8, bool PLANNED = true, class Sync>
__device__ __forceinline__ void decode_worker(const DecArgs& a, const int2* __restrict__ pieces,
                                              int32_t* __restrict__ plan, int queues, int worker, int nworkers,
                                              char* smem, int* fetched, Sync& sync, int* scan = nullptr) {
  const int tid = threadIdx.x & (kDecThreads - 1);
  const int queue = worker % queues;
  int total;
  if constexpr (PLANNED) {
    total = plan[kPlanTotal] * a.num_kv_heads;
  } else {
    // Pieces per sequence: its splits, or one for an empty sequence (which writes zeros).
    if (tid < kWave) {
      const int ctx =
          tid < a.num_seqs ? clamp_ctx<CHECK>(a.context_lens[tid], a.max_blocks, a.err_flag, worker == 0) : 0;
      const int n = tid < a.num_seqs ? (ctx > 0 ? (ctx + a.split_tokens - 1) / a.split_tokens : 1) : 0;
      int incl = n;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (tid >= off) incl += v;
      }
      scan[tid] = incl;
      scan[kWave + tid] = ctx;
    }
    sync();
    total = scan[kWave - 1] * a.num_kv_heads;
  }
  auto find = [&](int item, DecItem<HD>& it) {
    const int piece = item / a.num_kv_heads;
    if constexpr (PLANNED) {
      const int2 code = pieces[piece];
      it.s = static_cast<int>(static_cast<uint32_t>(code.x) >> 16);
      it.split = code.x & 0xffff;
      it.ctx = code.y;
    } else {
      // First sequence whose inclusive piece count passes `piece` (binary search over 64 entries).
      int lo = 0;
#pragma unroll
      for (int step = kWave / 2; step > 0; step >>= 1)
        if (scan[lo + step - 1] <= piece) lo += step;
      it.s = lo;
      it.split = piece - (lo > 0 ? scan[lo - 1] : 0);
      it.ctx = scan[kWave + lo];
    }
    it.g = item - piece * a.num_kv_heads;
    it.nsplit = (it.ctx + a.split_tokens - 1) / a.split_tokens;
    it.tbl0 = (a.member != nullptr && a.member[it.s]) ? a.prefix_blocks : 0;
  };
  int cur_i = worker, nxt_i = worker + nworkers;
  if (cur_i >= total) return;  // uniform over the worker's threads
  DecItem<HD> cur, nxt;
  find(cur_i, cur);
  decode_item_prologue<HD, CHECK>(a, cur);
  // `fetched` alternates slots: slot p is written before the barrier that ends an item and read
  // right after it; the next write to slot p comes after one more barrier.
  for (int p = 0;; p ^= 1) {
    const bool have_next = nxt_i < total;
    // Lane 0's old counter value.  It is first read when the item ends, so the atomic's round trip
    // overlaps the item (this needs the library's build without the atomic optimizer, whose
    // wave-level aggregation reads the result right away).
    int ticket = 0;
    auto fetch_next = [&]() {
      if (have_next) {
        if (PLANNED && tid == 0) ticket = atomicAdd(&plan[queue * kCounterStride], 1);
        find(nxt_i, nxt);
        decode_item_prologue<HD, CHECK>(a, nxt);  // in flight while this item runs
      }
    };
    if (cur.ctx == 0) {
      fetch_next();
      for (int i = tid; i < a.group * HD; i += kDecThreads)
        store_out(a.out, (static_cast<int64_t>(cur.s) * a.num_q_heads + cur.g * a.group) * HD + i, 0.f, a.out_bf16);
    } else {
      decode_bf16_item<HD, CHECK, NARROW, KV8>(a, cur, smem, sync, fetch_next);
    }
    if (tid == 0) fetched[p] = have_next ? ticket * queues + queue : total;
    sync();  // the next item reuses the staging and merge areas; fetched[p] is published
    if (!have_next) break;
    cur = nxt;
    nxt_i = fetched[p];
  }
}

}  // namespace pkv

// Host helpers shared by the decode and mixed-step entry points.
namespace pkv_dec {

inline bool shapes_ok(int32_t num_seqs, int32_t hq, int32_t hkv, int32_t hd, int32_t max_blocks) {
  return num_seqs >= 0 && hq > 0 && hkv > 0 && hq % hkv == 0 && hq / hkv <= pkv::kMaxGroup &&
         (hd == 64 || hd == 128 || hd == 256) && max_blocks > 0;
}

// Workspace: the plan (header ints, then 8 bytes per (sequence, split) piece), then, when a
// sequence can span several splits, the fp32 partial rows [num_seqs][hq][max_splits][hd] and
// their (max, normaliser) pairs.  Every part starts on a 256-byte boundary.
struct WsLayout {
  size_t pieces, o, ml, total;
};

inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

inline WsLayout ws_layout(int32_t num_seqs, int32_t hq, int32_t hd, int64_t max_splits) {
  WsLayout w;
  w.pieces = round256(pkv::kPlanInts * 4);
  w.o = w.pieces + round256(static_cast<size_t>(num_seqs) * max_splits * 8);
  const size_t rows = max_splits > 1 ? static_cast<size_t>(num_seqs) * hq * max_splits : 0;
  w.ml = w.o + round256(rows * hd * 4);
  w.total = w.ml + rows * 2 * 4;
  return w;
}

// Launch the one-workgroup plan pass (decode.hip).
// members / num_members / prefix_blocks / member_out: the shared-prefix decode (null / 0 otherwise).
void launch_plan(bool check, const int32_t* context_lens, int num_seqs, int max_blocks, int split_tokens,
                 int2* pieces, int32_t* plan, int grid, int queues, int32_t* err_flag, hipStream_t st,
                 const int32_t* members = nullptr, int num_members = 0, int prefix_blocks = 0,
                 uint8_t* member_out = nullptr);
// Launch the shared-prefix decode (mixed.hip): the prefix items (prefill kernel in shared-prefix
// mode, pre_items workgroups) first, then dec_wgs workgroups of two decode workers each, in one
// launch; head_dim 64 or 128, bf16 or (kv8) E4M3 pools.
void launch_prefix_decode(const pkv::DecArgs& da, const int2* pieces, int32_t* plan, int queues, int dec_wgs,
                          const pkv::PreArgs& pa, int pre_items, int32_t head_dim, bool check, bool narrow, bool kv8,
                          hipStream_t st);
// Launch the split reduce (decode.hip).
// slots: partial slots per (sequence, query head); member / prefix_blocks / prefix_slot0 /
// prefix_parts: the shared-prefix decode, whose members also merge prefix_parts partials from slot
// prefix_slot0 on (null / 0 otherwise).
void launch_reduce(const float* ws_o, const float* ws_ml, const int32_t* context_lens, int max_blocks,
                   int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int split_tokens, int slots,
                   void* out, int out_bf16, hipStream_t st, const uint8_t* member = nullptr, int prefix_blocks = 0,
                   int prefix_slot0 = 0, int prefix_parts = 0);

}  // namespace pkv_dec
