/*
 * pagedkv.h — C ABI of libpagedkv.so: attention over a paged KV cache on AMD MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [vLLM-internals]  "Phase 17 · 04 — vLLM serving internals" (aiengineeringfromscratch.com),
 *                     PagedAttention section: fixed 16-token KV blocks, one block table per
 *                     sequence mapping logical token positions to physical block ids.
 *   [C13-L2]          "C13 推理 · 第2课 服务端:连续批处理与 PagedAttention" (geekvape-learning),
 *                     section 改进二:PagedAttention, figure 按块表取 K and its dimension table:
 *                     one pool per layer of blocks x block size x (KV heads x head dim); a
 *                     request's keys (and values) are the pool rows gathered through its table.
 *   [Chunked-Prefill] "Chunked Prefill" (Ultralytics glossary): prefill stores the prompt's K/V in
 *                     the cache and decode reads the whole cache each step (section on prefill and
 *                     decode); each chunk attends under a causal mask over absolute positions to the
 *                     cached K/V of all earlier chunks plus its own tokens (section on how chunked
 *                     prefill works, with its PyTorch example).
 *   [Engine-core]     "第2章:推理引擎核心技术" (aiinfra.vidrealm.tech), §1.2 (block-table example:
 *                     logical block j holds tokens 16j..16j+15), §1.4 (the paged kernel walks a
 *                     request's pages through the table and accumulates with an online softmax),
 *                     §1.5 (copy-on-write: sequences share pages and copy one only where they
 *                     diverge) and §3.2 (prefix cache: hash each page of a prompt's tokens, share
 *                     the physical page on a hit by raising its reference count).
 *   [C13-L2] also, same section: paging wastes at most b - 1 token slots per request and has no
 *                     external fragmentation; several sequences may point at the same blocks and a
 *                     shared block is copied only when one of them writes into it.
 *
 * Data layout shared by every call (all device memory, caller-owned):
 *   key_pool, value_pool  [num_blocks, num_kv_heads, 16, head_dim], row-major, same dtype: the
 *                         pages' pool of blocks x 16 x (num_kv_heads*head_dim) with each block's
 *                         16 rows grouped by KV head, so that one KV head's share of a block is a
 *                         contiguous run of 16*head_dim elements.  A "slot" block*16 + offset holds
 *                         one token: its row of KV head h is [block][h][offset][:].
 *   block_tables          int32 [num_seqs, max_blocks_per_seq], row-major.  Entry [s][j] is the
 *                         physical block of sequence s's tokens 16j..16j+15.  Entries past the
 *                         sequence's last live block are never read and may hold anything.
 *   query / out           [rows, num_q_heads, head_dim], contiguous.
 *   Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Conventions:
 *   - Device pointers are device memory; int arguments are host values.  `stream` is a
 *     hipStream_t (NULL = the null stream).  Every call only enqueues work on `stream` and returns;
 *     buffers must stay alive until the stream reaches the call.  No call synchronises, allocates
 *     or keeps state between calls (the only cached state is each device's compute-unit count and,
 *     for pkv_paged_attn_decode_noalloc, the device address of its static scratch); the block
 *     manager (pkv_bm_*) is host code whose state lives in a caller-owned host buffer.  Since a
 *     call only launches kernels on `stream`, calls can be captured in a HIP graph.
 *   - Calls return a pkv_status.  Argument errors are found on the host before any HIP call.
 *     PKV_ERR_HIP reports a failed launch (hipGetLastError).  No C++ exception crosses the ABI.
 *   - err_flag: if non-NULL (a device int32, zeroed by the caller), kernels check every block id
 *     and slot they read against the pool and OR a PKV_FLAG_* bit into *err_flag instead of
 *     touching memory out of range; the affected output is then unspecified.  With err_flag ==
 *     NULL the checks are skipped and out-of-range ids are undefined behaviour.
 *   - Empty work (num_tokens == 0, num_seqs == 0) is a successful no-op.
 *   - The attention calls read and write whole 16-byte vectors: query, out, the pools and the
 *     decode workspace must be 16-byte aligned, else PKV_ERR_INVALID_ARG.  (The cache write
 *     accepts any element-aligned pointer and picks its vector width from the alignment.)
 *   - Supported: head_dim in {64, 128, 256}; num_q_heads % num_kv_heads == 0 and
 *     num_q_heads / num_kv_heads <= 16; block_size == 16.  Cache write and decode take fp32 or
 *     bf16; the prefill chunk takes bf16 (bf16 MFMA with fp32 accumulation).  Outputs may be
 *     fp32 or bf16 (round to nearest even); accumulation is always fp32.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,         /* null pointer, negative size, inconsistent shapes */
  PKV_ERR_UNSUPPORTED = 2,         /* dtype, head_dim, head ratio or block size outside the list above */
  PKV_ERR_WORKSPACE_TOO_SMALL = 3, /* decode workspace below pkv_decode_workspace_bytes() */
  PKV_ERR_HIP = 4,                 /* a kernel launch failed */
  PKV_ERR_NO_SPACE = 5,            /* block manager: not enough free blocks (state left unchanged) */
  PKV_ERR_SCRATCH_TOO_SMALL = 6    /* pkv_paged_attn_decode_noalloc: the shapes need more than
                                      PKV_NOALLOC_SCRATCH_BYTES of workspace */
} pkv_status;

/* Element types.  FP8_E4M3 is the OCP 8-bit floating point E4M3 encoding (1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, largest finite 448); it is only
 * a pool storage type, used with a per-pool fp32 scale by the *_fp8 calls below. */
typedef enum { PKV_DTYPE_F32 = 0, PKV_DTYPE_BF16 = 1, PKV_DTYPE_FP8_E4M3 = 2 } pkv_dtype;

/* Bits OR-ed into *err_flag by checked kernels. */
#define PKV_FLAG_BAD_BLOCK 1   /* a block-table entry the call had to read is outside [0, num_blocks) */
#define PKV_FLAG_BAD_SLOT 2    /* a slot is >= num_blocks * 16 */
#define PKV_FLAG_BAD_LENGTH 4  /* a context / chunk end exceeds max_blocks_per_seq * 16, or is negative */
#define PKV_FLAG_SYNC_TIMEOUT 8 /* pkv_paged_attn_mixed / the shared-prefix decode: a wave of a decode
                                   worker gave up a bounded wait on its sibling waves (about 2^28
                                   cycles); that call's outputs are unspecified.  Never set by a
                                   correct run; with err_flag == NULL the event is not reported. */

/* Static description of a status code. */
const char* pkv_status_string(pkv_status status);

/*
 * Slot mapping ([Engine-core] §1.2; [vLLM-internals] PagedAttention section).
 * For every sequence s and i < cu_new_lens[s+1] - cu_new_lens[s], with absolute position
 * p = start_pos[s] + i:
 *     slot_mapping[cu_new_lens[s] + i] = block_tables[s][p / 16] * 16 + p % 16.
 *   slot_mapping  out, int32 [cu_new_lens[num_seqs]]
 *   cu_new_lens   int32 [num_seqs + 1], non-decreasing, cu_new_lens[0] == 0 (device)
 *   start_pos     int32 [num_seqs] (device)
 *   max_new_len   host upper bound of cu_new_lens[s+1] - cu_new_lens[s] (sizes the grid; tokens
 *                 beyond it are not mapped)
 * A position past the table (p / 16 >= max_blocks_per_seq) or a bad block id yields slot -1
 * and, with err_flag, PKV_FLAG_BAD_LENGTH / PKV_FLAG_BAD_BLOCK.
 */
pkv_status pkv_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* cu_new_lens, const int32_t* start_pos, int32_t num_seqs,
                            int32_t max_new_len, int32_t num_blocks, int32_t block_size, int32_t* err_flag,
                            void* stream);

/*
 * Cache write ([Chunked-Prefill], section on prefill and decode: the new tokens' K/V are stored in
 * the cache; [C13-L2]: each generated token fills one slot).
 * For t < num_tokens with slot = slot_mapping[t] >= 0: the key row key[t] (num_kv_heads*head_dim
 * elements, contiguous, token stride key_tok_stride elements) is copied bit for bit into
 * key_pool slot `slot`, and likewise value[t] into value_pool.  Negative slots are skipped.
 * Duplicate slots within one call are a caller error (which copy wins is unspecified).
 *   key, value        [num_tokens, num_kv_heads, head_dim] with the given token strides (in
 *                     elements, >= num_kv_heads*head_dim); same dtype as the pools; no conversion.
 *   num_blocks        pool size in blocks (used by the err_flag check).
 */
pkv_status pkv_cache_write(const void* key, const void* value, int64_t key_tok_stride, int64_t value_tok_stride,
                           void* key_pool, void* value_pool, const int32_t* slot_mapping, int32_t num_tokens,
                           int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           pkv_dtype dtype, int32_t* err_flag, void* stream);

/*
 * Paged gather ([C13-L2] figure 按块表取 K: a request's K is the pool rows named by its table, V alike).
 * Copies sequence s's first lengths[s] token rows of both pools, in logical order, into
 * key_out / value_out rows cu_out[s] .. cu_out[s] + lengths[s] - 1, bit for bit, using the same
 * address arithmetic as the attention kernels.  A diagnostic used to test block indexing.
 *   key_out, value_out  [cu_out[num_seqs], num_kv_heads, head_dim], pool dtype (F32, BF16 or
 *                       FP8_E4M3; a bit copy in every case)
 *   lengths, cu_out     int32 [num_seqs] and [num_seqs + 1] (device)
 *   max_len             host upper bound of lengths[s] (sizes the grid)
 */
pkv_status pkv_paged_gather(void* key_out, void* value_out, const void* key_pool, const void* value_pool,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* lengths,
                            const int32_t* cu_out, int32_t num_seqs, int32_t max_len, int32_t num_blocks,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_dtype dtype,
                            int32_t* err_flag, void* stream);

/*
 * Decode split size, in tokens, that pkv_paged_attn_decode uses for these shapes when called with
 * split_tokens == 0 (a multiple of 128).  Depends on the arguments only.
 */
int32_t pkv_decode_split_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_blocks_per_seq);

/*
 * Workspace bytes pkv_paged_attn_decode needs for these shapes and split size (0 = the default
 * above): the work plan (a 256-byte header and one 4-byte entry per (sequence, split) piece), and,
 * when a sequence can span several splits, per (sequence, query head, split) an fp32 partial
 * output row plus its running max and normaliser.  Never 0 for valid shapes; 0 for invalid ones.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t split_tokens);

/*
 * One-token paged decode ([Chunked-Prefill] section on prefill and decode: decode reads the whole
 * cache; [Engine-core] §1.4: walk the request's pages through the table, online softmax).
 * out[s][h] = sum_j softmax_j(scale * q[s][h] . K_s[j]) V_s[j] over positions j < context_lens[s]
 * of sequence s's cache, KV head h / (num_q_heads / num_kv_heads).  context_lens[s] counts the
 * current token, which must already be in the cache.  context_lens[s] == 0 gives a zero row.
 * Long contexts are cut into splits of split_tokens positions whose partial results are merged
 * with a log-sum-exp combine; results do not depend on the split size beyond fp32 rounding.
 *   out                 [num_seqs, num_q_heads, head_dim], dtype out_dtype
 *   query               [num_seqs, num_q_heads, head_dim], dtype `dtype` (the pool dtype)
 *   context_lens        int32 [num_seqs] (device), each <= max_blocks_per_seq * 16
 *   scale               > 0 (the usual 1/sqrt(head_dim)); other values are PKV_ERR_INVALID_ARG
 *   split_tokens        0 for the default, else a multiple of 128 in [128, 2048]
 *   workspace           device scratch of >= pkv_decode_workspace_bytes(...) bytes (never null);
 *                       contents on entry are ignored; must not be shared by calls running
 *                       concurrently.  bf16 pools: a one-workgroup pass first sorts the pieces
 *                       longest first into it, and the attention workgroups then take items from
 *                       that list through counters the pass clears.
 */
pkv_status pkv_paged_attn_decode(void* out, pkv_dtype out_dtype, const void* query, const void* key_pool,
                                 const void* value_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, float scale,
                                 pkv_dtype dtype, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                 int32_t* err_flag, void* stream);

/*
 * Decode that allocates nothing, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Computes exactly what
 * pkv_paged_attn_decode computes (the same kernels, the same split size for the same arguments),
 * with its workspace taken from a static device array of PKV_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each GPU it runs on, for the life of the process.
 *   Arguments as for pkv_paged_attn_decode, without workspace / workspace_bytes; BF16 or F32 pools.
 *   PKV_ERR_SCRATCH_TOO_SMALL (nothing launched) when pkv_decode_workspace_bytes() for these shapes
 *   and split size exceeds PKV_NOALLOC_SCRATCH_BYTES; PKV_ERR_HIP if the array's device address
 *   cannot be obtained.  The caller still owns query, out, pools and tables.
 *   All calls on one GPU share the array and it keeps the last call's contents (no call needs it
 *   cleared): calls that overlap on one GPU (several streams or host threads at once) race and
 *   give undefined results; serialise them, or use pkv_paged_attn_decode with a workspace each.
 *   The call performs no hipMalloc / hipFree and no other allocating HIP or library routine.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
pkv_status pkv_paged_attn_decode_noalloc(void* out, pkv_dtype out_dtype, const void* query, const void* key_pool,
                                         const void* value_pool, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                         int32_t num_blocks, float scale, pkv_dtype dtype, int32_t split_tokens,
                                         int32_t* err_flag, void* stream);

/*
 * Chunked-prefill attention ([Chunked-Prefill], section on how chunked prefill works and its
 * PyTorch example).  Sequence s owns query rows cu_q_lens[s] .. cu_q_lens[s+1]-1; row i of it sits
 * at absolute position chunk_offsets[s] + i, and the cache must already hold positions
 * 0 .. chunk_offsets[s] + L_s - 1 (earlier chunks plus this chunk, written by pkv_cache_write).
 * Causal: row i attends to positions 0 .. chunk_offsets[s] + i.  Non-causal: to all positions
 * 0 .. chunk_offsets[s] + L_s - 1.
 *   out, query          [cu_q_lens[num_seqs], num_q_heads, head_dim]; query bf16, out out_dtype
 *   cu_q_lens           int32 [num_seqs + 1] (device), non-decreasing from 0
 *   chunk_offsets       int32 [num_seqs] (device), >= 0
 *   max_q_len           host upper bound of L_s (sizes the grid; rows beyond it are not computed)
 *   scale               > 0 (the usual 1/sqrt(head_dim)); other values are PKV_ERR_INVALID_ARG
 *   workspace           device scratch of >= pkv_prefill_workspace_bytes(...) bytes (16-byte aligned;
 *                       may be NULL when that is 0); PKV_ERR_WORKSPACE_TOO_SMALL otherwise
 */
pkv_status pkv_paged_attn_prefill_chunk(void* out, pkv_dtype out_dtype, const void* query, const int32_t* cu_q_lens,
                                        const int32_t* chunk_offsets, const void* key_pool, const void* value_pool,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                                        int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t num_blocks, int32_t causal, float scale,
                                        pkv_dtype dtype, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                        void* stream);

/*
 * Workspace bytes the chunked-prefill calls need for these shapes: when there are fewer 256-row
 * tiles than compute units, each tile's key range is split over several workgroups whose fp32
 * partial rows, (max, normaliser) pairs and arrival counters live here.  0 when no split is made
 * (the workspace may then be NULL).  The calls clear the counters themselves; the contents on
 * entry are ignored.  A workspace must not be shared by calls that run concurrently.
 */
size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads, int32_t head_dim,
                                   int32_t max_blocks_per_seq);

/*
 * FP8 KV pool.  The pages run their model in FP8 ([vLLM-internals], opening benchmark and memory
 * section) without saying how a cache would be stored in it; these calls keep K and V pools of
 * E4M3 codes, one fp32 scale per pool (k_scale, v_scale > 0, finite), so that a code c stands for
 * value(c) * scale.  Pools are [num_blocks, num_kv_heads, 16, head_dim] bytes, laid out as for
 * the other dtypes; slot mapping, block tables, the gather and the block copy are unchanged.
 *
 * Cache write with quantisation: for t < num_tokens with slot = slot_mapping[t] >= 0, every
 * element x of key row t (bf16 or fp32 as in_dtype, widened exactly to fp32) is stored as the
 * E4M3 code of the fp32 product x * (1 / k_scale), the reciprocal rounded to nearest in fp32;
 * the product rounds to the nearest E4M3 value with ties to the even code, magnitudes >= 448 and
 * infinities saturate to +-448, NaN becomes the NaN code 0x7F, the sign of zero is kept.  Value
 * rows alike with v_scale.  Negative slots are skipped; duplicate slots are a caller error.
 *   key, value   [num_tokens, num_kv_heads, head_dim], token strides in elements
 *   key_pool, value_pool  FP8_E4M3 pools (16-byte aligned)
 */
pkv_status pkv_cache_write_fp8(const void* key, const void* value, int64_t key_tok_stride, int64_t value_tok_stride,
                               void* key_pool, void* value_pool, const int32_t* slot_mapping, int32_t num_tokens,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               pkv_dtype in_dtype, float k_scale, float v_scale, int32_t* err_flag, void* stream);

/*
 * Decode with a shared prefix ([Engine-core] §1.5 and §3.2: sequences that share a cached prefix
 * map its logical blocks to the same physical blocks).  Computes exactly what
 * pkv_paged_attn_decode computes (up to rounding order), attending the shared prefix once per KV
 * head for all member sequences together instead of once per sequence.
 *   prefix_members  device int32 [num_members]: distinct sequence indices whose block-table rows
 *                   all start with the same prefix_blocks physical ids (those of
 *                   prefix_members[0]) and whose context_lens are at least prefix_blocks * 16;
 *                   the caller guarantees this (a row that differs gives a wrong result for that
 *                   sequence; an index outside [0, num_seqs) sets PKV_FLAG_BAD_LENGTH in checked
 *                   mode and is skipped, and if it is prefix_members[0] the members' outputs are
 *                   undefined; a member shorter than the prefix sets the same flag)
 *   prefix_blocks   number of shared leading blocks (0 <= prefix_blocks <= max_blocks_per_seq)
 *   workspace       at least pkv_decode_prefix_workspace_bytes(...) bytes (16-byte aligned)
 * Other arguments as for pkv_paged_attn_decode; BF16 pools, head_dim 64 or 128.  With no members
 * or prefix_blocks == 0 this is pkv_paged_attn_decode with the same split size.
 * Work: the (member, query head) pairs of a KV head are the rows of an MFMA attention over the
 * prefix (one partial per key split), run in the same launch as the decode of every position past
 * the prefix; the split reduce merges the two.  It pays when the prefix is long against the
 * members' own positions; the plain decode reads a short shared prefix from L2 almost for free.
 */
pkv_status pkv_paged_attn_decode_prefix(void* out, pkv_dtype out_dtype, const void* query, const void* key_pool,
                                        const void* value_pool, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t num_blocks, float scale, pkv_dtype dtype,
                                        const int32_t* prefix_members, int32_t num_members, int32_t prefix_blocks,
                                        int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                        int32_t* err_flag, void* stream);

/*
 * Shared-prefix decode over FP8 pools ([Engine-core] §1.5 and §3.2, as pkv_paged_attn_decode_prefix;
 * the pools as for pkv_paged_attn_decode_fp8): computes what pkv_paged_attn_decode_fp8 computes
 * (attention over the dequantised values, bf16 queries) with the shared prefix attended once per
 * KV head.  k_scale, v_scale: the pools' scales (> 0, finite; PKV_ERR_INVALID_ARG otherwise).  Other
 * arguments, the workspace (pkv_decode_prefix_workspace_bytes) and the errors as for
 * pkv_paged_attn_decode_prefix; head_dim 64 or 128.
 */
pkv_status pkv_paged_attn_decode_prefix_fp8(void* out, pkv_dtype out_dtype, const void* query, const void* key_pool,
                                            const void* value_pool, const int32_t* block_tables,
                                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t num_blocks, float scale, float k_scale,
                                            float v_scale, const int32_t* prefix_members, int32_t num_members,
                                            int32_t prefix_blocks, int32_t split_tokens, void* workspace,
                                            size_t workspace_bytes, int32_t* err_flag, void* stream);

/* Workspace bytes of pkv_paged_attn_decode_prefix(_fp8) for these shapes (0 for unsupported shapes). */
size_t pkv_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_blocks_per_seq, int32_t split_tokens);

/*
 * Decode over FP8 pools ([Chunked-Prefill] section on prefill and decode; [Engine-core] §1.4):
 * pkv_paged_attn_decode with K_s[j] and V_s[j] replaced by their dequantised
 * values value(code) * k_scale and value(code) * v_scale.  query is bf16; out F32 or BF16.  The
 * workspace and split_tokens rules are those of pkv_paged_attn_decode (same sizes).
 */
pkv_status pkv_paged_attn_decode_fp8(void* out, pkv_dtype out_dtype, const void* query, const void* key_pool,
                                     const void* value_pool, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t num_blocks, float scale, float k_scale, float v_scale,
                                     int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                     int32_t* err_flag, void* stream);

/*
 * Chunked prefill over FP8 pools ([Chunked-Prefill], section on how chunked prefill works):
 * pkv_paged_attn_prefill_chunk with dequantised K and V as above; query bf16, out F32 or BF16.
 */
pkv_status pkv_paged_attn_prefill_chunk_fp8(void* out, pkv_dtype out_dtype, const void* query,
                                            const int32_t* cu_q_lens, const int32_t* chunk_offsets,
                                            const void* key_pool, const void* value_pool,
                                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                                            int32_t num_seqs, int32_t max_q_len, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                            int32_t causal, float scale, float k_scale, float v_scale,
                                            void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                            void* stream);

/*
 * Token-budget step composer (host code; [Chunked-Prefill], token-budget section: each step adds one
 * token per running decode first, then fills the rest of the budget with chunks of waiting prompts,
 * and a prompt that does not fit goes on in the next step; [vLLM-internals], scheduler loop).
 *   num_decode            running sequences that each want one decode token, in priority order; if
 *                         they exceed the budget only the first token_budget are scheduled (a reading:
 *                         the pages do not say)
 *   prefill_remaining     int32 [num_prefill], prompt tokens not yet prefilled, queue order, each > 0
 *   token_budget          tokens per step (> 0)
 *   max_chunk             cap on one prompt's chunk (<= 0: none); budget a capped prompt leaves goes on
 *                         to the next prompt
 *   chunk_len             out int32 [num_prefill]: tokens of each prompt scheduled this step (0 = none)
 *   num_decode_scheduled  out: decode tokens scheduled
 * Returns PKV_ERR_INVALID_ARG (writing nothing) on a bad argument.  Pointers are host memory.
 */
pkv_status pkv_compose_step(int32_t num_decode, const int32_t* prefill_remaining, int32_t num_prefill,
                            int32_t token_budget, int32_t max_chunk, int32_t* chunk_len,
                            int32_t* num_decode_scheduled);

/*
 * Iteration-level scheduler over synthetic requests (host code; [vLLM-internals], scheduler-loop
 * section and its four modes; [Engine-core] §2.3).  Each step it releases finished requests and
 * their blocks, admits waiting requests in queue order (only arrived ones, while a running slot is
 * free and the block manager can hold the request's whole final length), then assigns every running
 * request its work: a prompt (whole, or a chunk) or one decode token.  Modes:
 *   PKV_SCHED_NAIVE       one request at a time
 *   PKV_SCHED_STATIC      a batch is admitted only when the previous one has fully finished; a
 *                         finished request keeps its slot until its whole batch is done
 *   PKV_SCHED_CONTINUOUS  admission and release every step; a newly admitted prompt is prefilled
 *                         whole in its first step
 *   PKV_SCHED_CHUNKED     as CONTINUOUS, with the step composed under token_budget by the rule of
 *                         pkv_compose_step (decode tokens first, then prompt chunks, max_chunk cap)
 * The first output token of a request is produced by the step that finishes its prompt; each
 * later step gives one more token; a request is done after output_len tokens.  Block-table rows
 * live in the scheduler (pkv_sched_table, [max_running][max_blocks]); rows are filled through the
 * block manager whose state the caller passes (not shared with other users while in use).  All
 * pointers are host memory; the state is one caller-owned, 8-byte aligned buffer.
 */
typedef enum { PKV_SCHED_NAIVE = 0, PKV_SCHED_STATIC = 1, PKV_SCHED_CONTINUOUS = 2, PKV_SCHED_CHUNKED = 3 } pkv_sched_mode;

size_t pkv_sched_state_bytes(int32_t max_requests, int32_t max_running, int32_t max_blocks, int64_t max_itl_samples);
pkv_status pkv_sched_init(void* state, size_t state_bytes, int32_t mode, int32_t max_requests, int32_t max_running,
                          int32_t max_blocks, int64_t max_itl_samples, int32_t token_budget, int32_t max_chunk,
                          void* bm_state);
/* Requests arrive in id order (arrival times non-decreasing, any time unit); prompt_len, output_len > 0. */
pkv_status pkv_sched_add_request(void* state, int32_t prompt_len, int32_t output_len, double arrival, int32_t* id);
/* Plan the step starting at `now`.  Outputs (arrays of max_running entries): decode entries (table row,
 * context length counting the new token, whose K/V the step writes at position ctx - 1) and prompt
 * chunks (table row, first position, length; the step writes positions [offset, offset + len) and the
 * chunk attends causally to [0, offset + len)).  next_arrival: arrival of the next waiting request,
 * -1 if none (when nothing is planned the caller advances its clock to it). */
pkv_status pkv_sched_plan(void* state, double now, int32_t* num_decode, int32_t* dec_row, int32_t* dec_ctx,
                          int32_t* num_chunks, int32_t* chunk_row, int32_t* chunk_offset, int32_t* chunk_len,
                          double* next_arrival);
/* The planned step ended at `now`: record its tokens and release finished requests. */
pkv_status pkv_sched_complete(void* state, double now);
const int32_t* pkv_sched_table(const void* state);
int32_t pkv_sched_num_done(const void* state);
/* Arrival, first-token and finish times of request id (-1 where not reached yet). */
pkv_status pkv_sched_request_times(const void* state, int32_t id, double* arrival, double* first_token, double* finish);
/* Copies up to capacity inter-token gaps (time between consecutive tokens of one request, first
 * token excluded); returns how many were recorded (-1 on a bad argument). */
int64_t pkv_sched_itl(const void* state, double* out, int64_t capacity);

/*
 * Fused mixed-batch step ([vLLM-internals], scheduler-loop section: one step carries the decode
 * tokens and the prefill chunks through one forward call; [Chunked-Prefill], token-budget section).
 * One attention launch (plus the decode's plan pass and, for long contexts, its split reduce) that
 * computes exactly what pkv_paged_attn_decode computes for the decode arguments and what
 * pkv_paged_attn_prefill_chunk computes for the prefill arguments, over the same pools; outputs are
 * bit-identical to those two calls.  Either part may be empty (num_dec_seqs == 0, or
 * num_pre_seqs == 0 / max_q_len == 0).
 *   decode part   dec_out / dec_query [num_dec_seqs, num_q_heads, head_dim], dec_block_tables
 *                 [num_dec_seqs, dec_max_blocks], context_lens [num_dec_seqs]
 *   prefill part  pre_out / pre_query [cu_q_lens[num_pre_seqs], num_q_heads, head_dim], cu_q_lens,
 *                 chunk_offsets, pre_block_tables [num_pre_seqs, pre_max_blocks], max_q_len, causal
 *   dtype         BF16 pools, or FP8_E4M3 pools with k_scale / v_scale (ignored for BF16); queries bf16
 *   split_tokens, workspace  as for pkv_paged_attn_decode with the decode part's shapes
 *   pre_workspace       as the workspace of pkv_paged_attn_prefill_chunk for the prefill part
 * head_dim 64 or 128 (a decode workgroup runs two decode workers side by side); 256 is
 * PKV_ERR_UNSUPPORTED.
 */
pkv_status pkv_paged_attn_mixed(void* dec_out, const void* dec_query, const int32_t* dec_block_tables,
                                int32_t dec_max_blocks, const int32_t* context_lens, int32_t num_dec_seqs,
                                void* pre_out, const void* pre_query, const int32_t* cu_q_lens,
                                const int32_t* chunk_offsets, const int32_t* pre_block_tables,
                                int32_t pre_max_blocks, int32_t num_pre_seqs, int32_t max_q_len, int32_t causal,
                                const void* key_pool, const void* value_pool, int32_t num_blocks,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
                                pkv_dtype dtype, float k_scale, float v_scale, pkv_dtype out_dtype,
                                int32_t split_tokens, void* workspace, size_t workspace_bytes,
                                void* pre_workspace, size_t pre_workspace_bytes, int32_t* err_flag, void* stream);

/*
 * Block copy for copy-on-write ([Engine-core] §1.5; [C13-L2] 改进二, sharing paragraph): for each
 * pair i, the whole block src[i] (16 rows x num_kv_heads x head_dim, K and V) is copied bit for bit
 * to block dst[i].  src / dst: int32 [num_pairs] device arrays; src[i] == dst[i] is a no-op; a
 * block that is a destination must not be a source or destination of another pair in the same call
 * (undefined otherwise).  dtype F32, BF16 or FP8_E4M3 (a bit copy in every case).  With err_flag, ids outside
 * [0, num_blocks) set PKV_FLAG_BAD_BLOCK and that pair is skipped.
 */
pkv_status pkv_copy_blocks(void* key_pool, void* value_pool, const int32_t* src, const int32_t* dst,
                           int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, pkv_dtype dtype, int32_t* err_flag, void* stream);

/*
 * Block manager (host code; every pointer below is host memory).  It hands out physical blocks of
 * one pool to sequences and fills their block-table rows ([Engine-core] §1.2), shares blocks
 * between sequences with reference counts, finds a new prompt's cached prefix by a chained hash of
 * each full block's token ids ([Engine-core] §3.2), and copies a shared block before a sequence
 * writes into it ([Engine-core] §1.5).  Policies the pages leave open (stated readings):
 *   - free blocks sit in a FIFO queue: allocation takes the front, a freed block goes to the back,
 *     so the blocks freed longest ago are reused first;
 *   - the hash of full block j is FNV-1a (64-bit) over the 8 bytes of block j-1's hash (0 for j = 0)
 *     followed by the block's 16 token ids (4 bytes each, little-endian), with 0 mapped to 1;
 *   - a prompt's full blocks are registered under their hash when they are allocated (their K/V is
 *     written by that step's prefill); a freed block keeps its hash while it waits in the queue and
 *     can be found again until it is handed out for new content;
 *   - a lookup walks the prompt's full blocks from the start and stops at the first miss.
 * The state is one caller-owned buffer of pkv_bm_state_bytes(num_blocks) bytes (8-byte aligned);
 * calls on one state must not overlap (not thread-safe).  Every call validates its arguments and
 * leaves the state unchanged when it returns an error.
 */
size_t pkv_bm_state_bytes(int32_t num_blocks);

/* All blocks free.  free_order: NULL for 0, 1, ..., num_blocks-1, else a permutation of them giving
 * the initial queue order (e.g. a seeded shuffle).  block_size must be 16. */
pkv_status pkv_bm_init(void* state, size_t state_bytes, int32_t num_blocks, int32_t block_size,
                       const int32_t* free_order);

/* New sequence with prompt tokens[0..num_tokens): reuse the blocks of its longest cached prefix of
 * full blocks, allocate the rest, write table_row[0 .. ceil(num_tokens/16)).  *cached_tokens = the
 * number of leading tokens whose K/V the reused blocks already hold (a multiple of 16).
 * PKV_ERR_NO_SPACE if the free queue cannot cover the new blocks. */
pkv_status pkv_bm_add_sequence(void* state, const int32_t* tokens, int32_t num_tokens, int32_t* table_row,
                               int32_t max_blocks, int32_t* cached_tokens);

/* Append num_new tokens to a sequence holding ctx tokens: when its last block is partly filled and
 * shared, it is first replaced by a fresh copy (one pair in copy_src/copy_dst for
 * pkv_copy_blocks, *num_copies = 1, else 0); new blocks are allocated as positions cross block
 * boundaries.  slots[i] = slot of position ctx + i (the slot mapping for pkv_cache_write). */
pkv_status pkv_bm_append(void* state, int32_t* table_row, int32_t max_blocks, int32_t ctx, int32_t num_new,
                         int32_t* slots, int32_t* copy_src, int32_t* copy_dst, int32_t* num_copies);

/* child_row[0 .. ceil(ctx/16)) = parent_row's blocks, each shared (reference count + 1). */
pkv_status pkv_bm_fork(void* state, const int32_t* parent_row, int32_t ctx, int32_t* child_row,
                       int32_t max_blocks);

/* Drop a sequence of ctx tokens: each of its blocks loses one reference; blocks left with none go to
 * the back of the free queue. */
pkv_status pkv_bm_free_sequence(void* state, const int32_t* table_row, int32_t ctx);

/* Inspection (for tests and monitoring): free blocks, a block's reference count (-1 if out of
 * range), a block's registered hash (0 if none). */
int32_t pkv_bm_num_free(const void* state);
int32_t pkv_bm_refcount(const void* state, int32_t block);
uint64_t pkv_bm_block_hash(const void* state, int32_t block);

/*
 * Streaming-read reference (not part of the attention path): reads `bytes` bytes at `buf` (device,
 * 16-byte aligned, bytes % 16 == 0) once with 16-byte loads and XORs a fold of them into *sink
 * (a device uint32).  Its duration gives the bandwidth a plain read stream reaches on the device,
 * against which the decode's bandwidth is compared.
 */
pkv_status pkv_stream_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * Matrix-core reference (not part of the attention path): one 512-thread workgroup per compute
 * unit (two waves per SIMD), every wave issuing `iters` x 4 v_mfma_f32_32x32x16_bf16 (32,768 flop
 * each) in four independent chains on register operands and nothing else.  The operands are eight
 * A and eight B fragments of pseudo-random bf16 values per lane, cycled so that consecutive MFMAs
 * see different data (the switching activity, and so the power and clock, of a real kernel's
 * operands; constant operands would run faster than any real kernel can).  *sink (a device float)
 * is written only if the sums take a value they never take, so the work is kept but nothing is
 * stored.  Its duration gives the bf16 MFMA rate a kernel of pure matrix work reaches on the
 * device (its clock under that load included), against which the prefill's rate is compared.  The
 * flop count of one call is cu_count x 8 waves x iters x 4 x 32,768.  iters must be positive.
 */
pkv_status pkv_mfma_peak_probe(int32_t iters, float* sink, void* stream);
int32_t pkv_device_cu_count(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
