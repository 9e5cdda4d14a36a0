// Device side of the chunked-prefill attention (see prefill.hip for what is computed and the
// design), shared by the prefill kernel and the fused mixed-step kernel.
#pragma once

#include <cmath>

#include "common.hpp"

namespace pkv {


constexpr int kPreWaves = 8;                    // eight row waves sharing every key tile
constexpr int kPreThreads = kPreWaves * kWave;
constexpr int kPreRows = 32;                    // query rows per wave
constexpr int kPreTile = kPreWaves * kPreRows;  // query rows per workgroup (256)
constexpr int kPreMaxSplit = 8;                 // largest number of key splits of one row tile
constexpr int kIdWindow = 2048;                 // block ids held in LDS (32,768 positions)

// E: bytes per pool element (2 for bf16, 1 for E4M3 codes); LDS tiles are bf16 either way.
template <int HD, int E = 2>
struct PreCfg {
  static constexpr int KT = HD == 256 ? 32 : 64;  // key positions per LDS tile
  static constexpr int MS = KT / 32;              // 32-key row tiles of S^T
  static constexpr int KA = KT / 16;              // 16-key k-steps of O^T
  static constexpr int KS = HD / 16;              // k-steps of S^T over head_dim
  static constexpr int MD = HD / 32;              // 32-row tiles of O^T
  static constexpr int KPITCH = HD * 2 + 16;      // LDS bytes per K row (conflict-free 16-byte reads)
  static constexpr int VPITCH = HD * 2 + 64;      // LDS bytes per V row (transposed reads without bank conflicts)
  static constexpr int EPC = 16 / E;              // pool elements per 16-byte chunk
  static constexpr int CPR = HD / EPC;            // 16-byte chunks per row
  static constexpr int TILE = KT * (KPITCH + VPITCH);
  static constexpr int LOADS = 2 * KT * CPR / kPreThreads;  // chunks per thread per tensor per tile pair
  static constexpr int LDS = 4 * TILE;                       // two buffers of a tile pair
  static_assert(LOADS * kPreThreads == 2 * KT * CPR, "pair loads must divide evenly");
};

// KV8: the pools hold E4M3 codes, converted exactly to bf16 on their way into LDS; scale_log2 then
// includes the K scale and v_scale multiplies the output (1 for bf16 pools).
// Arguments of the prefill chunk (one struct shared by the prefill and mixed-step kernels).
struct PreArgs {
  const uint16_t* query;
  const int32_t* cu_q_lens;
  const int32_t* chunk_offsets;
  const void* key_pool;  // bf16 or E4M3 codes
  const void* value_pool;
  const int32_t* block_tables;
  int max_blocks, q_tiles, num_q_heads, num_kv_heads, group, num_blocks, causal;
  float scale_log2;  // scale * log2(e), times the K scale for FP8 pools
  float v_scale;     // V scale of an FP8 pool, 1 for bf16
  void* out;
  int out_bf16;
  int32_t* err_flag;
  // Key split: the key range of a row tile is cut into ksplit runs of whole tile pairs, one per
  // workgroup; with ksplit > 1 each writes its (o, m, l) partial to ws_o / ws_ml and
  // prefill_merge_kernel writes the output.
  int ksplit;
  float* ws_o;   // [row items][ksplit][kPreTile][HD]
  float* ws_ml;  // [row items][ksplit][kPreTile][2]
  // Shared-prefix mode (prefix_members != null): the rows of KV head g are the pairs (member m,
  // query head g*G + i) of the decode queries, row m*G + i; the keys are the first prefix_blocks
  // blocks of member 0's table, all visible; the (o, m, l) partial of a row goes to slot
  // prefix_slot0 + key split of that query's row in the decode workspace (ws_o / ws_ml with
  // prefix_slots slots per (sequence, query head)).
  const int32_t* prefix_members;
  int num_members, prefix_blocks, prefix_slots, prefix_slot0, prefix_num_seqs;
  // Row layout of the items (prefill_body's PACK), read by the merge.
  int pack;
};

// One work item (one key split of 256 rows) on a 512-thread workgroup.  Rows: with PACK false, the
// chunk positions of one query head (row R = position R); with PACK true, the (position, query head)
// pairs of one KV head's group (row R = position R / G, query head g*G + R % G), so that one item's
// K/V tiles serve the whole group however short the chunk; shared-prefix rows are always (member,
// query head) pairs.
// id / items: the item's index among `items` consecutive workgroups (the remap below assumes
// workgroups are dealt round-robin over the 8 XCDs starting at an XCD boundary, and keeps the
// splits of a row tile next to each other, on one XCD).  smem holds PreCfg<HD>::LDS bytes and ids
// kIdWindow ints (the block ids of logical blocks [win0, win0 + kIdWindow)).
template <int HD, bool CHECK, bool NARROW, bool KV8, bool PACK>
__device__ __forceinline__ void prefill_body(const PreArgs& A_, int id, int items, char* smem, int* ids) {
  constexpr int E = KV8 ? 1 : 2;
  using C = PreCfg<HD, E>;
  const uint16_t* __restrict__ query = A_.query;
  const int32_t* __restrict__ cu_q_lens = A_.cu_q_lens;
  const int32_t* __restrict__ chunk_offsets = A_.chunk_offsets;
  const void* __restrict__ key_pool = A_.key_pool;
  const void* __restrict__ value_pool = A_.value_pool;
  const int32_t* __restrict__ block_tables = A_.block_tables;
  const int max_blocks = A_.max_blocks, q_tiles = A_.q_tiles, num_q_heads = A_.num_q_heads;
  const int num_kv_heads = A_.num_kv_heads, group = A_.group, num_blocks = A_.num_blocks, causal = A_.causal;
  const float scale_log2 = A_.scale_log2, v_scale = A_.v_scale;
  void* __restrict__ out = A_.out;
  const int out_bf16 = A_.out_bf16;
  int32_t* err_flag = A_.err_flag;

  // Work item: XCD-contiguous remap of the linear workgroup id.
  const int ksplit = A_.ksplit;
  const int wk = (items % 8 == 0) ? (id % 8) * (items / 8) + id / 8 : id;
  const int kh = wk % ksplit;  // key split
  const int w = wk / ksplit;   // row-tile item
  const bool prefix = A_.prefix_members != nullptr;
  const int t = w % q_tiles;
  int r = w / q_tiles;
  const int hi = (PACK || prefix) ? 0 : r % group;
  r = (PACK || prefix) ? r : r / group;
  const int g = r % num_kv_heads;
  const int s = prefix ? A_.prefix_members[0] : r / num_kv_heads;
  if (prefix && (s < 0 || s >= A_.prefix_num_seqs)) {
    if (CHECK && threadIdx.x == 0) atomicOr(err_flag, PKV_FLAG_BAD_LENGTH);
    return;
  }
  const int h = g * group + hi;

  const int qlo = prefix ? 0 : cu_q_lens[s];
  // PACK: the chunk's positions; rows L = positions x G.  Otherwise rows are positions (shared-prefix
  // rows: members x G).
  const int npos = prefix ? A_.num_members : cu_q_lens[s + 1] - qlo;
  const int L = PACK ? npos * group : (prefix ? A_.num_members * group : cu_q_lens[s + 1] - qlo);
  const int off = prefix ? 0 : chunk_offsets[s];
  const int row0 = t * kPreTile;
  if (row0 >= L) return;
  if (off < 0 || static_cast<int64_t>(off) + (PACK ? npos : L) > static_cast<int64_t>(max_blocks) * kBlockSize) {
    if (!prefix) {
      if (CHECK && threadIdx.x == 0 && t == 0 && hi == 0) atomicOr(err_flag, PKV_FLAG_BAD_LENGTH);
      return;
    }
  }
  const int kv_end = prefix   ? A_.prefix_blocks * kBlockSize
                     : causal ? off + (PACK ? (min(row0 + kPreTile, L) - 1) / group + 1 : min(row0 + kPreTile, L))
                              : off + (PACK ? npos : L);

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int qc = lane & 31, hh = lane >> 5;
  const int wrow0 = row0 + wave * kPreRows;
  const int myrow = wrow0 + qc;
  const int32_t* table = block_tables + static_cast<int64_t>(s) * max_blocks;
  // Shared-prefix mode: this row's decode query (member sequence, query head).
  int p_seq = prefix && myrow < L ? A_.prefix_members[myrow / group] : 0;
  if (prefix && (p_seq < 0 || p_seq >= A_.prefix_num_seqs)) {
    if (CHECK) atomicOr(err_flag, PKV_FLAG_BAD_LENGTH);
    p_seq = -1;
  }
  const bool row_ok = myrow < L && p_seq >= 0;
  // This row's chunk position and query head (p_head); with PACK, the first and last positions of
  // the wave's rows for the causal skip and the edge-tile test.
  const int mypos = PACK ? myrow / group : myrow;
  const int qpos = off + mypos;
  const int p_head = (PACK || prefix) ? g * group + myrow % group : h;
  const int wave_pos0 = PACK ? wrow0 / group : 0, wave_pos1 = PACK ? (min(wrow0 + kPreRows, L) - 1) / group : 0;

  // Q^T as the B operand: lane (qc, hh) holds query row qc, head_dim 16ks + 8hh .. +7.
  bf16x8 qf[C::KS];
  {
    const int64_t qr = prefix ? static_cast<int64_t>(row_ok ? p_seq : 0) * num_q_heads + p_head
                              : static_cast<int64_t>(qlo + (row_ok ? mypos : 0)) * num_q_heads + (PACK ? p_head : h);
    const uint16_t* qrow = query + qr * HD + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = row_ok ? as_bf16x8(ld16(qrow + 16 * ks)) : bf16x8{};
  }

  floatx16 acc[C::MD];
#pragma unroll
  for (int md = 0; md < C::MD; ++md)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[md][e] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;

  // Block ids live in an LDS window so that gathers never wait on a table read.  A checked run
  // turns a bad id into -1 (the positions of that block then read as zero and are flagged).
  const int nblk_kv = (kv_end + kBlockSize - 1) / kBlockSize;
  int win0 = 0;
  auto fill_ids = [&](int first) {
    for (int j = threadIdx.x; j < kIdWindow; j += kPreThreads)
      ids[j] = first + j < nblk_kv ? load_block_id<CHECK>(table, first + j, num_blocks, err_flag) : -1;
  };

  // Tile pair p holds key tiles 2p and 2p+1 (2*KT positions); all 512 threads gather it through
  // the block table.  Thread t's i-th 16-byte chunk is row t / CPR + i * RPI of the pair at column
  // (t % CPR) * 8; RPI is a multiple of 16, so the row's slot inside its block is the same for
  // every i and only the block id changes.
  constexpr int RPI = kPreThreads / C::CPR;  // pair rows per load round
  const int t_row = threadIdx.x / C::CPR;
  const uint32_t blk_bytes = static_cast<uint32_t>(kBlockSize * num_kv_heads * HD * E);
  const uint32_t c0 = static_cast<uint32_t>((g * kBlockSize + t_row % kBlockSize) * HD * E + (threadIdx.x % C::CPR) * 16);
  uint4 kreg[C::LOADS], vreg[C::LOADS];
  auto load_pair = [&](int p) {
    const int key0p = 2 * p * C::KT + t_row;
    const int idx0 = key0p / kBlockSize - win0;
    int idv[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) idv[i] = ids[idx0 + i * (RPI / kBlockSize)];
    // Whole pair inside the keys (and unchecked ids): plain loads, nothing to mask.
    if (!CHECK && (2 * p + 2) * C::KT <= kv_end) {
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        kreg[i] = ld16(pool_at<NARROW>(key_pool, idv[i], blk_bytes, c0));
        vreg[i] = ld16(pool_at<NARROW>(value_pool, idv[i], blk_bytes, c0));
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const bool ok = key0p + i * RPI < kv_end && idv[i] >= 0;
        const int b = ok ? idv[i] : 0;  // block 0 stands in for masked rows
        const uint4 kv = ld16(pool_at<NARROW>(key_pool, b, blk_bytes, c0));
        const uint4 vv = ld16(pool_at<NARROW>(value_pool, b, blk_bytes, c0));
        kreg[i] = ok ? kv : uint4{0, 0, 0, 0};
        vreg[i] = ok ? vv : uint4{0, 0, 0, 0};
      }
    }
  };
  auto store_pair = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int f = threadIdx.x + kPreThreads * i;
      const int tt = f / (C::KT * C::CPR);
      const int rem = f - tt * (C::KT * C::CPR);
      const int row = rem / C::CPR, col = (rem % C::CPR) * C::EPC;
      char* base = smem + (2 * buf + tt) * C::TILE;
      if constexpr (KV8) {
        uint4 lo, hi;
        e4m3x16_to_bf16(kreg[i], lo, hi);
        st16(base + row * C::KPITCH + col * 2, lo);
        st16(base + row * C::KPITCH + col * 2 + 16, hi);
        e4m3x16_to_bf16(vreg[i], lo, hi);
        st16(base + C::KT * C::KPITCH + row * C::VPITCH + col * 2, lo);
        st16(base + C::KT * C::KPITCH + row * C::VPITCH + col * 2 + 16, hi);
      } else {
        st16(base + row * C::KPITCH + col * 2, kreg[i]);
        st16(base + C::KT * C::KPITCH + row * C::VPITCH + col * 2, vreg[i]);
      }
    }
  };

  // This split's tile pairs: [p_lo, p_hi) of the row tile's pairs.
  const int ntiles = (kv_end + C::KT - 1) / C::KT;
  const int npairs_all = (ntiles + 1) / 2;
  const int per = (npairs_all + ksplit - 1) / ksplit;
  const int p_lo = min(kh * per, npairs_all), p_hi = min(p_lo + per, npairs_all);
  constexpr int kPairBlocks = 2 * C::KT / kBlockSize;
  win0 = p_lo * kPairBlocks;
  fill_ids(win0);
  __syncthreads();
  if (p_lo < p_hi) {
    load_pair(p_lo);
    store_pair(0);
  }
  __syncthreads();

  const int li = lane & 15, dg = (lane >> 4) & 1;
  constexpr int VP = C::VPITCH / 2;
  for (int pr = p_lo; pr < p_hi; ++pr) {
    const int cur = (pr - p_lo) & 1;
    // Slide the id window when pair pr + 1 (the one read ahead) would leave it.
    if ((pr + 2) * kPairBlocks - win0 > kIdWindow && (pr + 1) * kPairBlocks < nblk_kv) {
      win0 = (pr + 1) * kPairBlocks;
      fill_ids(win0);
      __syncthreads();
    }
    if (pr + 1 < p_hi) load_pair(pr + 1);
    // Every wave takes both tiles of the pair (one loop body: unrolling it doubles live registers).
#pragma unroll 1
    for (int tt = 0; tt < 2; ++tt) {
    const int kt = 2 * pr + tt;
    const int key0 = kt * C::KT;
    const bool active = kt < ntiles && wrow0 < L && (!causal || key0 <= off + (PACK ? wave_pos1 : wrow0 + kPreRows - 1));
    if (active) {
      const char* tile = smem + (2 * cur + tt) * C::TILE;
      floatx16 sacc[C::MS];
      // The MS accumulators are interleaved so that consecutive MFMAs are independent.
#pragma unroll
      for (int ms = 0; ms < C::MS; ++ms) {
        const char* krow = tile + (32 * ms + qc) * C::KPITCH + 16 * hh;
        sacc[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(krow), qf[0],
                                                           floatx16{}, 0, 0, 0);
      }
#pragma unroll
      for (int ks = 1; ks < C::KS; ++ks)
#pragma unroll
        for (int ms = 0; ms < C::MS; ++ms) {
          const char* krow = tile + (32 * ms + qc) * C::KPITCH + 16 * hh;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 32 * ks);
          sacc[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[ms], 0, 0, 0);
        }
      // Keep four K reads in flight ahead of the MFMAs that consume them.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < C::MS * C::KS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // Element e = 4i + j of sacc[ms] is key key0 + 32ms + 8i + 4hh + j for query row qc.  Only
      // tiles that cross the causal diagonal or the end of the keys need the mask.
      const bool edge = key0 + C::KT > kv_end || (causal && key0 + C::KT - 1 > off + (PACK ? wave_pos0 : wrow0));
      if (edge) {
#pragma unroll
        for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = key0 + 32 * ms + 8 * (e >> 2) + 4 * hh + (e & 3);
            const bool ok = key < kv_end && (!causal || key <= qpos);
            sacc[ms][e] = ok ? sacc[ms][e] : -INFINITY;
          }
      }
      // Softmax weights.  The reference max m_ref trails the running max: it is raised only when a
      // weight of this tile would exceed 2^20 (or no key was seen yet) or on edge tiles, so the
      // common path computes no row max.  m_ref only matters through rounding.
      auto raise_max = [&]() {
        float mx = -INFINITY;
#pragma unroll
        for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[ms][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = mx * scale_log2;
        const bool up = m_new > m_ref;
        const float alpha = up ? (m_ref == -INFINITY ? 0.f : fast_exp2(m_ref - m_new)) : 1.f;
        m_ref = up ? m_new : m_ref;
        l_run *= alpha;
#pragma unroll
        for (int md = 0; md < C::MD; ++md) acc[md] *= alpha;
      };
      uint32_t pw[C::MS * 8];
      auto expo = [&]() {
        const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float p0 = fast_exp2(__builtin_fmaf(sacc[ms][2 * q], scale_log2, neg_m));
            const float p1 = fast_exp2(__builtin_fmaf(sacc[ms][2 * q + 1], scale_log2, neg_m));
            const uint32_t w = pack_bf16x2(p0, p1);
            pw[ms * 8 + q] = w;
            if (q & 1) ps1 = add_bf16x2(w, ps1); else ps0 = add_bf16x2(w, ps0);
          }
        return ps0 + ps1;
      };
      if (edge) raise_max();
      float ps = expo();
      if (__any(!(ps < kMaxWeight) || m_ref == -INFINITY)) {
        raise_max();
        ps = expo();
      }
      l_run += ps;
      bf16x8 pb[C::KA];
#pragma unroll
      for (int a = 0; a < C::KA; ++a)
        pb[a] = __builtin_bit_cast(bf16x8, uint4{pw[4 * a], pw[4 * a + 1], pw[4 * a + 2], pw[4 * a + 3]});

      // O^T += V^T P^T.  k-step a covers keys 16a + 4hh + e and 16a + 8 + 4hh + e (e = 0..3),
      // matching pb[a]; the A operand lane (l % 32 = d, hh) reads those keys' V at d.
      const uint16_t* vbase = reinterpret_cast<const uint16_t*>(tile + C::KT * C::KPITCH);
      // The MD accumulators are interleaved so that consecutive MFMAs are independent.
#pragma unroll
      for (int a = 0; a < C::KA; ++a) {
        const int r0 = 16 * a + 4 * hh + (li >> 2);
#pragma unroll
        for (int md = 0; md < C::MD; ++md) {
          const int col = 32 * md + 16 * dg + 4 * (li & 3);
          const bf16x8 av = concat(lds_read_tr16(vbase + r0 * VP + col), lds_read_tr16(vbase + (r0 + 8) * VP + col));
          acc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[a], acc[md], 0, 0, 0);
        }
      }
      // Keep eight transposed V reads (four MFMA operands) in flight ahead of their MFMAs.
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < C::MD * C::KA - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    }
    if (pr + 1 < p_hi) store_pair(cur ^ 1);
    __syncthreads();
  }

  // Output.  One split: normalise and write the rows.  Several: see below.
  l_run += __shfl_xor(l_run, 32);
  if constexpr (HD <= 128) {
    if (prefix) {
      // The row's (o, m, l) partial goes to its decode query's prefix slot for this key split.
      if (!row_ok) return;
      const int64_t part = (static_cast<int64_t>(p_seq) * num_q_heads + p_head) * A_.prefix_slots + A_.prefix_slot0 + kh;
      float* my_o = A_.ws_o + part * HD;
#pragma unroll
      for (int md = 0; md < C::MD; ++md)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 32 * md + 8 * i + 4 * hh;
          *reinterpret_cast<float4*>(my_o + d) =
              float4{acc[md][4 * i] * v_scale, acc[md][4 * i + 1] * v_scale, acc[md][4 * i + 2] * v_scale,
                     acc[md][4 * i + 3] * v_scale};
        }
      if (hh == 0) *reinterpret_cast<float2*>(A_.ws_ml + part * 2) = float2{m_ref, l_run};
      return;
    }
  }
  const int64_t obase = (static_cast<int64_t>(qlo + mypos) * num_q_heads + (PACK ? p_head : h)) * HD;
  auto write_rows = [&](float ia) {
#pragma unroll
    for (int md = 0; md < C::MD; ++md)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * md + 8 * i + 4 * hh;
        const float v0 = acc[md][4 * i] * ia, v1 = acc[md][4 * i + 1] * ia, v2 = acc[md][4 * i + 2] * ia,
                    v3 = acc[md][4 * i + 3] * ia;
        if (out_bf16) {
          uint16_t* o = static_cast<uint16_t*>(out) + obase + d;
          const uint2 pk = uint2{static_cast<uint32_t>(f32_to_bf16(v0)) | (static_cast<uint32_t>(f32_to_bf16(v1)) << 16),
                                 static_cast<uint32_t>(f32_to_bf16(v2)) | (static_cast<uint32_t>(f32_to_bf16(v3)) << 16)};
          *reinterpret_cast<uint2*>(o) = pk;
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(out) + obase + d) = float4{v0, v1, v2, v3};
        }
      }
  };
  if (ksplit == 1) {
    if (!row_ok) return;
    const float inv = l_run > 0.f ? v_scale / l_run : 0.f;
    write_rows(inv);
    return;
  }
  // Several splits: write this split's (o, m, l) partial; prefill_merge_kernel combines them
  // after the launch (the kernel boundary orders the writes before the reads on every XCD).
  const int prow = wave * kPreRows + qc;  // row inside the tile
  const int64_t part = (static_cast<int64_t>(w) * ksplit + kh) * kPreTile + prow;
  float* my_o = A_.ws_o + part * HD;
#pragma unroll
  for (int md = 0; md < C::MD; ++md)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * md + 8 * i + 4 * hh;
      *reinterpret_cast<float4*>(my_o + d) = float4{acc[md][4 * i], acc[md][4 * i + 1], acc[md][4 * i + 2], acc[md][4 * i + 3]};
    }
  if (hh == 0) *reinterpret_cast<float2*>(A_.ws_ml + part * 2) = float2{m_ref, l_run};
}

}  // namespace pkv

// Host helpers shared by the prefill and mixed-step entry points.
namespace pkv_pre {

// Row tiles of one (sequence, head) with PACK false, or of one (sequence, KV head) with PACK true:
// max_q_len positions times the query heads sharing the rows, in tiles of kPreTile rows.
inline int64_t row_tiles(int32_t max_q_len, int32_t heads_per_row_set) {
  return (static_cast<int64_t>(max_q_len) * heads_per_row_set + pkv::kPreTile - 1) / pkv::kPreTile;
}

// Whether to pack the rows by KV head: only when that gives fewer row tiles (short chunks, or
// chunks well short of a multiple of kPreTile); otherwise the per-head layout is kept.
inline bool pack_rows(int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads) {
  const int32_t group = num_q_heads / num_kv_heads;
  return group > 1 &&
         num_kv_heads * row_tiles(max_q_len, group) < static_cast<int64_t>(num_q_heads) * row_tiles(max_q_len, 1);
}

// Key splits of a row tile: enough workgroups to give every CU one (each takes a whole CU's LDS),
// at most kPreMaxSplit, and no more than the tile pairs the longest possible context has.
inline int ksplit_for(int64_t row_items, int32_t max_blocks, int32_t head_dim, int cus) {
  if (row_items <= 0) return 1;
  int64_t k = (cus + row_items - 1) / row_items;
  const int kt = head_dim == 256 ? 32 : 64;
  const int64_t pairs = (static_cast<int64_t>(max_blocks) * pkv::kBlockSize + 2 * kt - 1) / (2 * kt);
  if (k > pkv::kPreMaxSplit) k = pkv::kPreMaxSplit;
  if (k > pairs) k = pairs;
  return k < 1 ? 1 : static_cast<int>(k);
}

// Workspace of the key splits: partial rows and their (max, normaliser) pairs, each part on a
// 256-byte boundary.  Nothing when there is one split.
struct Layout {
  size_t o, ml, total;
};

inline Layout layout(int64_t row_items, int ksplit, int32_t head_dim) {
  Layout l{0, 0, 0};
  if (ksplit <= 1) return l;
  auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = static_cast<size_t>(row_items) * ksplit * pkv::kPreTile;
  l.o = 0;
  l.ml = r256(rows * head_dim * 4);
  l.total = l.ml + r256(rows * 2 * 4);
  return l;
}

// Merge the key splits' partials into the output (prefill.hip); a no-op launch is never made.
void launch_merge(const pkv::PreArgs& a, int64_t row_items, int32_t head_dim, hipStream_t st);

}  // namespace pkv_pre
