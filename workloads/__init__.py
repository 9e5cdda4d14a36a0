"""Seeded synthetic inputs for paged-KV attention.

This module only draws random numbers and lays out integer bookkeeping
(context lengths, a shuffled free list, block tables, which pool slots hold
live tokens).  It holds none of the attention arithmetic and none of the
slot-mapping formula: both the oracle and the HIP path receive the arrays it
returns and compute everything else on their own.

Storage conventions (shared by both sides because they are the *inputs*):

* The KV pool of one layer is ``[num_blocks, num_kv_heads, block_size,
  head_dim]``, K and V in separate pools: the pool drawn in "C13 推理 · 第2课
  服务端" (geekvape-learning), section "改进二:PagedAttention", figure "按块表取
  K" and its dimension table (pool = blocks x block size x D, D = KV heads x
  head dim), with each block's rows grouped by KV head.  Slot
  ``block * block_size + offset`` holds one token; its row of KV head g is
  ``pool[block, g, offset]``.
* bf16 values are carried as ``uint16`` bit patterns, produced from fp32
  draws with round-to-nearest-even.  fp32 values are plain ``float32``.
* Block tables are ``int32 [num_seqs, max_blocks_per_seq]``; entries past a
  sequence's last live block hold ``UNUSED_BLOCK_ID`` so that any read of
  them is out of range and shows up in a checked run.

The draw order for every config is fixed: contexts, block permutation,
queries, keys, values (each of K and V: pool first, then new tokens).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BLOCK_SIZE = 16
# A deliberately out-of-range id for block-table entries that no live token uses.
UNUSED_BLOCK_ID = 0x3FFFFFF0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even) and return the bit patterns.
    NaNs map to the canonical quiet NaN 0x7FC0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    xf, of = x.reshape(-1), out.reshape(-1)

    def conv(lo, hi):
        u = xf[lo:hi].view(np.uint32)
        # Finite values cannot overflow 32 bits here; NaNs are fixed up below.
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        of[lo:hi] = r.astype(np.uint16)
        nan = np.isnan(xf[lo:hi])
        if nan.any():
            of[lo:hi][nan] = 0x7FC0

    _parallel_chunks(xf.size, conv)
    return out


_CHUNK = 1 << 22
_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))


def _parallel_chunks(n: int, fn) -> None:
    edges = list(range(0, n, _CHUNK)) + [n]
    if len(edges) <= 2:
        fn(0, n)
        return
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(lambda i: fn(edges[i], edges[i + 1]), range(len(edges) - 1)))


def _normal_f32(seed: int, stream: int, shape) -> np.ndarray:
    """Standard normal fp32 array for draw number ``stream`` of config ``seed``.  The array is cut
    into fixed 2^22-element chunks, each filled by its own PCG64 child of
    ``SeedSequence([seed, stream])``, so the values do not depend on the thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, -(-n // _CHUNK))
    kids = np.random.SeedSequence([seed, stream]).spawn(nchunks)

    def fill(lo, hi):
        g = np.random.Generator(np.random.PCG64(kids[lo // _CHUNK]))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)

    _parallel_chunks(n, fill)
    return out.reshape(shape)


BF16_NAN_BITS = np.uint16(0x7FC0)


@dataclass
class PagedCase:
    """One synthetic workload: a pool, block tables, queries and the new tokens to write."""

    name: str
    kind: str  # "decode" or "prefill"
    dtype: str  # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    block_size: int
    scale: float
    context_lens: np.ndarray  # int32 [B]: tokens in cache each sequence attends over
    block_tables: np.ndarray  # int32 [B, W]
    key_pool: np.ndarray  # [num_blocks, block_size, Hkv, hd] (float32 or uint16 bits)
    value_pool: np.ndarray
    # New tokens, written before the attention call, packed by sequence.
    new_cu_lens: np.ndarray  # int32 [B+1]
    new_start_pos: np.ndarray  # int32 [B]: absolute position of each sequence's first new token
    key_new: np.ndarray  # [T, Hkv, hd]
    value_new: np.ndarray
    query: np.ndarray  # decode: [B, Hq, hd]; prefill: [sum L, Hq, hd]
    # Prefill only: the chunk rows of each sequence, packed.
    cu_q_lens: Optional[np.ndarray] = None  # int32 [B+1]
    chunk_offsets: Optional[np.ndarray] = None  # int32 [B]
    causal: bool = True
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def num_new_tokens(self) -> int:
        return int(self.new_cu_lens[-1])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


class _Draws:
    """Numbered value draws of one config: queries, then keys (pool, new), then values (pool, new)."""

    def __init__(self, seed: int):
        self.seed = seed
        self.k = 0

    def __call__(self, shape, dtype: str) -> np.ndarray:
        x = _normal_f32(self.seed, self.k, shape)
        self.k += 1
        return x if dtype == "f32" else f32_to_bf16_bits(x)


def _poison_value(dtype: str):
    return np.float32(np.nan) if dtype == "f32" else BF16_NAN_BITS


def allocate_from_free_list(free_list: np.ndarray, blocks_needed: List[int], width: int,
                            shared_prefix: Optional[np.ndarray] = None) -> np.ndarray:
    """Hand out blocks to sequences in index order from the front of ``free_list``.

    Each sequence takes exactly the number of blocks it needs, in logical order.
    With ``shared_prefix`` its first logical blocks map to those ids instead
    (up to the prefix length), and only the rest come from the free list.
    """
    tables = np.full((len(blocks_needed), width), UNUSED_BLOCK_ID, dtype=np.int32)
    cursor = 0
    for s, need in enumerate(blocks_needed):
        shared = 0
        if shared_prefix is not None:
            shared = min(need, len(shared_prefix))
            tables[s, :shared] = shared_prefix[:shared]
        own = need - shared
        tables[s, shared:need] = free_list[cursor:cursor + own]
        cursor += own
    return tables


def live_slot_mask(block_tables: np.ndarray, lens: np.ndarray, num_blocks: int,
                   block_size: int = BLOCK_SIZE) -> np.ndarray:
    """bool [num_blocks, block_size]: pool slots that hold one of the first ``lens[s]`` tokens of some sequence."""
    mask = np.zeros((num_blocks, block_size), dtype=bool)
    for s, n in enumerate(lens):
        n = int(n)
        full = n // block_size
        if full:
            mask[block_tables[s, :full]] = True
        rem = n - full * block_size
        if rem:
            mask[block_tables[s, full], :rem] = True
    return mask


def slot_rows(pool: np.ndarray) -> np.ndarray:
    """The pool's token rows in slot order, ``[num_blocks * block_size, Hkv, hd]`` (a copy)."""
    nblk, hkv, b, hd = pool.shape
    return np.ascontiguousarray(pool.transpose(0, 2, 1, 3)).reshape(nblk * b, hkv, hd)


def set_slots(pool: np.ndarray, mask: np.ndarray, value) -> None:
    """Store ``value`` in every element of the slots ``mask`` (bool [num_blocks, block_size])
    selects, for every KV head: pools are [num_blocks, Hkv, block_size, hd]."""
    pool.transpose(0, 2, 1, 3)[mask] = value


def _poison_dead_slots(case: PagedCase, live_lens: np.ndarray) -> None:
    live = live_slot_mask(case.block_tables, live_lens, case.num_blocks, case.block_size)
    dead = ~live
    p = _poison_value(case.dtype)
    set_slots(case.key_pool, dead, p)
    set_slots(case.value_pool, dead, p)


# ---------------------------------------------------------------------------------------------
# The five workloads.  Seeds are the config index.  ``with_data=False`` builds the integer
# bookkeeping only (contexts, tables, pool size) and leaves the value arrays empty.
# ---------------------------------------------------------------------------------------------


def _values(draw: "_Draws", shape, dtype: str, with_data: bool) -> np.ndarray:
    if with_data:
        return draw(shape, dtype)
    draw.k += 1
    return np.zeros((0,) + tuple(shape[1:]), np.float32 if dtype == "f32" else np.uint16)


def tiny_decode(poison: bool = True, with_data: bool = True) -> PagedCase:
    """Tiny paged decode: 4 sequences, contexts 17/50/100/128, 8 = 8 heads, head_dim 64, fp32,
    a 64-block pool handed out from a seeded shuffled free list.  All 295 tokens reach the pool
    through the cache write."""
    rng = np.random.default_rng(1)
    draw = _Draws(1)
    ctx = np.array([17, 50, 100, 128], dtype=np.int32)
    hq = hkv = 8
    hd = 64
    nblk = 64
    free = rng.permutation(nblk).astype(np.int32)
    need = [math.ceil(int(c) / BLOCK_SIZE) for c in ctx]
    bt = allocate_from_free_list(free, need, max(need))
    T = int(ctx.sum())
    q = _values(draw, (4, hq, hd), "f32", with_data)
    shape = (nblk, hkv, BLOCK_SIZE, hd)
    kpool = np.full(shape, np.nan if poison else 0.0, dtype=np.float32)
    knew = _values(draw, (T, hkv, hd), "f32", with_data)
    vpool = np.full(shape, np.nan if poison else 0.0, dtype=np.float32)
    vnew = _values(draw, (T, hkv, hd), "f32", with_data)
    cu = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    return PagedCase("tiny_decode", "decode", "f32", hq, hkv, hd, nblk, BLOCK_SIZE, 1.0 / math.sqrt(hd),
                     ctx, bt, kpool, vpool, cu, np.zeros(4, np.int32), knew, vnew, q)


def chunked_prefill_chunks(prompt_len: int = 1000, chunk: int = 256):
    """The chunk split of a prompt: (start, end) pairs of consecutive fixed-size chunks, last one ragged."""
    return [(s, min(s + chunk, prompt_len)) for s in range(0, prompt_len, chunk)]


def chunked_prefill(poison: bool = True, prompt_len: int = 1000, chunk: int = 256,
                    with_data: bool = True) -> PagedCase:
    """Chunked prefill equivalence: one sequence, a 1000-token prompt, 8 heads x 64 dims, bf16;
    70-block pool (63 blocks live + 10% free).  The returned case holds the whole prompt as new
    tokens and as queries; callers split it with ``chunked_prefill_chunks``."""
    rng = np.random.default_rng(2)
    draw = _Draws(2)
    hq = hkv = 8
    hd = 64
    need = math.ceil(prompt_len / BLOCK_SIZE)
    nblk = math.ceil(need * 1.1)
    free = rng.permutation(nblk).astype(np.int32)
    bt = allocate_from_free_list(free, [need], need)
    q = _values(draw, (prompt_len, hq, hd), "bf16", with_data)
    shape = (nblk, hkv, BLOCK_SIZE, hd)
    fill = BF16_NAN_BITS if poison else np.uint16(0)
    kpool = np.full(shape, fill, dtype=np.uint16)
    knew = _values(draw, (prompt_len, hkv, hd), "bf16", with_data)
    vpool = np.full(shape, fill, dtype=np.uint16)
    vnew = _values(draw, (prompt_len, hkv, hd), "bf16", with_data)
    ctx = np.array([prompt_len], np.int32)
    return PagedCase("chunked_prefill", "prefill", "bf16", hq, hkv, hd, nblk, BLOCK_SIZE, 1.0 / math.sqrt(hd),
                     ctx, bt, kpool, vpool, np.array([0, prompt_len], np.int32), np.zeros(1, np.int32),
                     knew, vnew, q, cu_q_lens=np.array([0, prompt_len], np.int32),
                     chunk_offsets=np.zeros(1, np.int32), causal=True,
                     notes={"chunks": chunked_prefill_chunks(prompt_len, chunk)})


# Lognormal context lengths with arithmetic mean 1500 and standard deviation 600.
LOGNORMAL_SIGMA = math.sqrt(math.log(1.0 + (600.0 / 1500.0) ** 2))
LOGNORMAL_MU = math.log(1500.0) - LOGNORMAL_SIGMA ** 2 / 2.0


def gqa_decode(poison: bool = False, num_seqs: int = 128, with_data: bool = True) -> PagedCase:
    """GQA decode, one 70B-style layer: 64 query heads over 8 KV heads x 128 dims, bf16, batch 128,
    contexts lognormal (mean 1500, sd 600) clipped to [16, 8192], pool = live blocks + 10% free,
    handed out from a shuffled free list.  The pool is already filled; nothing is written."""
    rng = np.random.default_rng(3)
    draw = _Draws(3)
    hq, hkv, hd = 64, 8, 128
    ctx = np.clip(np.rint(rng.lognormal(LOGNORMAL_MU, LOGNORMAL_SIGMA, size=num_seqs)), 16, 8192).astype(np.int32)
    need = [math.ceil(int(c) / BLOCK_SIZE) for c in ctx]
    nblk = math.ceil(1.1 * sum(need))
    free = rng.permutation(nblk).astype(np.int32)
    bt = allocate_from_free_list(free, need, 8192 // BLOCK_SIZE)
    q = _values(draw, (num_seqs, hq, hd), "bf16", with_data)
    shape = (nblk, hkv, BLOCK_SIZE, hd)
    kpool = _values(draw, shape, "bf16", with_data)
    vpool = _values(draw, shape, "bf16", with_data)
    case = PagedCase("gqa_decode", "decode", "bf16", hq, hkv, hd, nblk, BLOCK_SIZE, 1.0 / math.sqrt(hd),
                     ctx, bt, kpool, vpool, np.zeros(num_seqs + 1, np.int32), np.zeros(num_seqs, np.int32),
                     np.zeros((0, hkv, hd), np.uint16), np.zeros((0, hkv, hd), np.uint16), q)
    if poison and with_data:
        _poison_dead_slots(case, ctx)
    return case


def long_decode(poison: bool = False, num_seqs: int = 58, context: int = 4096, with_data: bool = True) -> PagedCase:
    """Long-context decode: 16 query heads over 4 KV heads x 256 dims, bf16, 58 sequences at
    context 4096 (256 blocks each, 14,848 blocks in all), randomly permuted physical ids.  Each
    sequence's last block (positions 4080..4095) is written by the cache write before the decode."""
    rng = np.random.default_rng(4)
    draw = _Draws(4)
    hq, hkv, hd = 16, 4, 256
    ctx = np.full(num_seqs, context, np.int32)
    per = context // BLOCK_SIZE
    nblk = num_seqs * per
    perm = rng.permutation(nblk).astype(np.int32)
    bt = perm.reshape(num_seqs, per).copy()
    new_per = BLOCK_SIZE
    q = _values(draw, (num_seqs, hq, hd), "bf16", with_data)
    shape = (nblk, hkv, BLOCK_SIZE, hd)
    kpool = _values(draw, shape, "bf16", with_data)
    knew = _values(draw, (num_seqs * new_per, hkv, hd), "bf16", with_data)
    vpool = _values(draw, shape, "bf16", with_data)
    vnew = _values(draw, (num_seqs * new_per, hkv, hd), "bf16", with_data)
    cu = (np.arange(num_seqs + 1) * new_per).astype(np.int32)
    start = np.full(num_seqs, context - new_per, np.int32)
    case = PagedCase("long_decode", "decode", "bf16", hq, hkv, hd, nblk, BLOCK_SIZE, 1.0 / math.sqrt(hd),
                     ctx, bt, kpool, vpool, cu, start, knew, vnew, q)
    if poison and with_data:
        # The slots the cache write fills start out poisoned, so a missed write shows.
        _poison_dead_slots(case, ctx - new_per)
    return case


SHARED_PREFIX_BLOCKS = 256


def shared_prefix_decode(poison: bool = False, num_seqs: int = 64, with_data: bool = True) -> PagedCase:
    """Decode batch behind one cached system prompt, 70B-style GQA (64/8 heads, head_dim 128,
    bf16): 64 sequences whose logical blocks 0..255 map to the same 256 physical blocks (a shared
    4,096-token prompt), each followed by a private part uniform in [1, 512] tokens; the pool is
    the live blocks + 10% free, handed out from a shuffled free list.  Every sequence is a member
    of the shared prefix (notes["members"], notes["prefix_blocks"])."""
    rng = np.random.default_rng(6)
    draw = _Draws(6)
    hq, hkv, hd = 64, 8, 128
    P = SHARED_PREFIX_BLOCKS
    ctx = (P * BLOCK_SIZE + rng.integers(1, 512, size=num_seqs, endpoint=True)).astype(np.int32)
    need = [math.ceil(int(c) / BLOCK_SIZE) for c in ctx]
    nblk = math.ceil(1.1 * (P + sum(n - P for n in need)))
    perm = rng.permutation(nblk).astype(np.int32)
    shared = perm[:P]
    bt = allocate_from_free_list(perm[P:], need, max(need), shared_prefix=shared)
    q = _values(draw, (num_seqs, hq, hd), "bf16", with_data)
    shape = (nblk, hkv, BLOCK_SIZE, hd)
    kpool = _values(draw, shape, "bf16", with_data)
    vpool = _values(draw, shape, "bf16", with_data)
    case = PagedCase("shared_prefix_decode", "decode", "bf16", hq, hkv, hd, nblk, BLOCK_SIZE, 1.0 / math.sqrt(hd),
                     ctx, bt, kpool, vpool, np.zeros(num_seqs + 1, np.int32), np.zeros(num_seqs, np.int32),
                     np.zeros((0, hkv, hd), np.uint16), np.zeros((0, hkv, hd), np.uint16), q,
                     notes={"shared_blocks": shared.copy(), "prefix_blocks": P,
                            "members": np.arange(num_seqs, dtype=np.int32)})
    if poison and with_data:
        _poison_dead_slots(case, ctx)
    return case


MIXED_PREFIX_BLOCKS = 63
MIXED_PROMPT = 32768
MIXED_CHUNK = 512
MIXED_OFFSET = 16384


def mixed_step(poison: bool = False, num_decode: int = 127, with_data: bool = True):
    """Mixed chunked-prefill + decode step, 70B-style GQA (64/8 heads, head_dim 128, bf16).

    Decode: 127 sequences with contexts uniform in [200, 8192]; logical blocks 0..62 of every
    sequence map to the same 63 physical blocks (a shared 1000-token prefix).  Prefill: one
    512-token chunk of a 32,768-token prompt at offset 16,384, attending to 16,384 cached tokens
    plus its own 512.  Both parts share one pool.  Returns (decode_case, prefill_case); the
    pool arrays are the same objects in both."""
    rng = np.random.default_rng(5)
    draw = _Draws(5)
    hq, hkv, hd = 64, 8, 128
    ctx = rng.integers(200, 8192, size=num_decode, endpoint=True).astype(np.int32)
    need = [math.ceil(int(c) / BLOCK_SIZE) for c in ctx]
    private = sum(max(0, n - MIXED_PREFIX_BLOCKS) for n in need)
    pre_blocks = (MIXED_OFFSET + MIXED_CHUNK) // BLOCK_SIZE
    nblk = math.ceil(1.1 * (MIXED_PREFIX_BLOCKS + private + pre_blocks))
    perm = rng.permutation(nblk).astype(np.int32)
    shared = perm[:MIXED_PREFIX_BLOCKS]
    rest = perm[MIXED_PREFIX_BLOCKS:]
    bt_dec = allocate_from_free_list(rest, need, 8192 // BLOCK_SIZE, shared_prefix=shared)
    pre_ids = rest[private:private + pre_blocks]
    bt_pre = np.full((1, MIXED_PROMPT // BLOCK_SIZE), UNUSED_BLOCK_ID, np.int32)
    bt_pre[0, :pre_blocks] = pre_ids
    q_dec = _values(draw, (num_decode, hq, hd), "bf16", with_data)
    q_pre = _values(draw, (MIXED_CHUNK, hq, hd), "bf16", with_data)
    shape = (nblk, hkv, BLOCK_SIZE, hd)
    kpool = _values(draw, shape, "bf16", with_data)
    knew = _values(draw, (MIXED_CHUNK, hkv, hd), "bf16", with_data)
    vpool = _values(draw, shape, "bf16", with_data)
    vnew = _values(draw, (MIXED_CHUNK, hkv, hd), "bf16", with_data)
    scale = 1.0 / math.sqrt(hd)
    dec = PagedCase("mixed_decode", "decode", "bf16", hq, hkv, hd, nblk, BLOCK_SIZE, scale,
                    ctx, bt_dec, kpool, vpool, np.zeros(num_decode + 1, np.int32), np.zeros(num_decode, np.int32),
                    np.zeros((0, hkv, hd), np.uint16), np.zeros((0, hkv, hd), np.uint16), q_dec,
                    notes={"shared_blocks": shared.copy()})
    pre = PagedCase("mixed_prefill", "prefill", "bf16", hq, hkv, hd, nblk, BLOCK_SIZE, scale,
                    np.array([MIXED_OFFSET + MIXED_CHUNK], np.int32), bt_pre, kpool, vpool,
                    np.array([0, MIXED_CHUNK], np.int32), np.array([MIXED_OFFSET], np.int32), knew, vnew, q_pre,
                    cu_q_lens=np.array([0, MIXED_CHUNK], np.int32),
                    chunk_offsets=np.array([MIXED_OFFSET], np.int32), causal=True)
    if poison and with_data:
        live = live_slot_mask(bt_dec, ctx, nblk) | live_slot_mask(bt_pre, np.array([MIXED_OFFSET]), nblk)
        dead = ~live
        set_slots(kpool, dead, BF16_NAN_BITS)
        set_slots(vpool, dead, BF16_NAN_BITS)
    return dec, pre


def random_case(seed: int, *, kind: str, dtype: str, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                head_dim: int, max_ctx: int, min_ctx: int = 0, q_len_max: int = 1, causal: bool = True,
                spare_blocks: int = 3, poison: bool = True, new_tokens: bool = True) -> PagedCase:
    """A small random case for parity sweeps: random contexts (and, for prefill, random chunk
    lengths and offsets), a shuffled pool, random queries.  For prefill the chunk's own tokens
    are the new tokens; for decode the last token of each sequence is."""
    rng = np.random.default_rng(seed)
    draw = _Draws(1000 + seed)
    if kind == "decode":
        ctx = rng.integers(min_ctx, max_ctx, size=num_seqs, endpoint=True).astype(np.int32)
        newl = (ctx > 0).astype(np.int32) if new_tokens else np.zeros(num_seqs, np.int32)
        qlen = None
        offs = None
    else:
        qlen = rng.integers(max(1, min_ctx), q_len_max, size=num_seqs, endpoint=True).astype(np.int32)
        offs = rng.integers(0, max(0, max_ctx - q_len_max), size=num_seqs, endpoint=True).astype(np.int32)
        ctx = (offs + qlen).astype(np.int32)
        newl = qlen.copy() if new_tokens else np.zeros(num_seqs, np.int32)
    need = [math.ceil(int(c) / BLOCK_SIZE) for c in ctx]
    nblk = sum(need) + spare_blocks
    free = rng.permutation(nblk).astype(np.int32)
    bt = allocate_from_free_list(free, need, max(1, max(need) + 1))
    nq = num_seqs if kind == "decode" else int(qlen.sum())
    q = draw((nq, num_q_heads, head_dim), dtype)
    shape = (nblk, num_kv_heads, BLOCK_SIZE, head_dim)
    T = int(newl.sum())
    kpool = draw(shape, dtype)
    knew = draw((T, num_kv_heads, head_dim), dtype)
    vpool = draw(shape, dtype)
    vnew = draw((T, num_kv_heads, head_dim), dtype)
    cu_new = np.concatenate([[0], np.cumsum(newl)]).astype(np.int32)
    start = (ctx - newl).astype(np.int32)
    case = PagedCase(f"random_{kind}_{seed}", kind, dtype, num_q_heads, num_kv_heads, head_dim, nblk, BLOCK_SIZE,
                     1.0 / math.sqrt(head_dim), ctx, bt, kpool, vpool, cu_new, start, knew, vnew, q)
    if kind == "prefill":
        case.cu_q_lens = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
        case.chunk_offsets = offs
        case.causal = causal
    if poison:
        _poison_dead_slots(case, ctx - newl)
    return case


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of K plus V one token occupies in one layer's pool."""
    return 2 * num_kv_heads * head_dim * elem_bytes


def kv_bytes_per_block(num_kv_heads: int, head_dim: int, elem_bytes: int, block_size: int = BLOCK_SIZE) -> int:
    """Bytes of K plus V one physical block occupies in one layer's pool."""
    return block_size * kv_bytes_per_token(num_kv_heads, head_dim, elem_bytes)
