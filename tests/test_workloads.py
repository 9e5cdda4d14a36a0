"""Invariants of the seeded input generators (CPU only).

Sizes are checked against the dimension table of "C13 推理 · 第2课 服务端"
(geekvape-learning), section "改进二:PagedAttention": one block of the anchor
model is 16 tokens x 65,536 B over 16 layers (1 MiB), with D = 4 KV heads x
256 dims and 256 blocks for a 4,096-token request; and against the paging
waste bound stated in the same lesson's evidence table: at most b - 1 tokens
wasted per request, no external fragmentation.
"""
import math

import numpy as np
import pytest

import workloads as wl


def test_block_size_arithmetic_anchor_model():
    # One layer, K plus V, bf16: 4 KV heads x 256 dims.
    per_token_layer = wl.kv_bytes_per_token(4, 256, 2)
    assert per_token_layer * 16 == 65536  # per token over 16 layers
    assert wl.kv_bytes_per_block(4, 256, 2) * 16 == 1 << 20  # one block over 16 layers = 1 MiB
    assert 4096 // wl.BLOCK_SIZE == 256


def test_long_decode_shapes():
    c = wl.long_decode(with_data=False)
    assert c.num_blocks == 14848 == 58 * 256
    assert c.block_tables.shape == (58, 256)
    assert sorted(c.block_tables.ravel().tolist()) == list(range(14848))
    assert c.num_new_tokens == 58 * 16
    assert (c.new_start_pos == 4080).all()


def _check_paging_bound(case, shared=()):
    shared = set(int(x) for x in shared)
    seen = {}
    for s in range(case.num_seqs):
        n = int(case.context_lens[s])
        nb = math.ceil(n / case.block_size)
        row = case.block_tables[s]
        assert (row[:nb] >= 0).all() and (row[:nb] < case.num_blocks).all()
        assert (row[nb:] == wl.UNUSED_BLOCK_ID).all()
        assert nb * case.block_size - n <= case.block_size - 1  # internal waste bound
        for j in range(nb):
            blk = int(row[j])
            if blk in shared:
                continue
            assert blk not in seen, "a private block handed to two sequences"
            seen[blk] = s


def test_tiny_decode_free_list_and_bound():
    c = wl.tiny_decode()
    assert c.context_lens.tolist() == [17, 50, 100, 128]
    assert c.num_blocks == 64
    assert [math.ceil(x / 16) for x in c.context_lens] == [2, 4, 7, 8]
    _check_paging_bound(c)
    assert c.num_new_tokens == 295


def test_gqa_decode_lognormal_contexts():
    c = wl.gqa_decode(with_data=False)
    assert c.num_seqs == 128 and c.num_q_heads == 64 and c.num_kv_heads == 8 and c.head_dim == 128
    assert c.context_lens.min() >= 16 and c.context_lens.max() <= 8192
    # The draw has mean 1500 and sd 600; a batch of 128 lands within a few standard errors.
    assert abs(c.context_lens.mean() - 1500) < 4 * 600 / math.sqrt(128)
    need = sum(math.ceil(x / 16) for x in c.context_lens)
    assert c.num_blocks == math.ceil(1.1 * need)
    _check_paging_bound(c)


def test_mixed_step_shared_prefix():
    dec, pre = wl.mixed_step(with_data=False)
    assert dec.num_seqs == 127
    assert dec.context_lens.min() >= 200 and dec.context_lens.max() <= 8192
    shared = dec.notes["shared_blocks"]
    assert len(shared) == 63
    for s in range(dec.num_seqs):
        nb = min(63, math.ceil(int(dec.context_lens[s]) / 16))
        assert (dec.block_tables[s, :nb] == shared[:nb]).all()
    _check_paging_bound(dec, shared=shared)
    assert pre.chunk_offsets.tolist() == [16384] and int(pre.cu_q_lens[-1]) == 512
    assert int(pre.context_lens[0]) == 16896
    pre_blocks = pre.block_tables[0, :1056]
    assert not set(pre_blocks.tolist()) & set(dec.block_tables[dec.block_tables != wl.UNUSED_BLOCK_ID].tolist())
    assert pre.key_pool is dec.key_pool


def test_chunked_prefill_split():
    c = wl.chunked_prefill()
    assert [e - s for s, e in c.notes["chunks"]] == [256, 256, 256, 232]
    assert c.num_blocks == 70
    _check_paging_bound(c)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 65504.0, np.inf], np.float32)
    bits = wl.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins; 1 + 3*2^-8 rounds up to 1 + 2^-6.
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 65536.0, np.inf]


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_random_case_poisons_only_dead_slots(kind):
    c = wl.random_case(7, kind=kind, dtype="bf16", num_seqs=3, num_q_heads=4, num_kv_heads=2, head_dim=16,
                       max_ctx=80, q_len_max=20, poison=True)
    live_before = wl.live_slot_mask(c.block_tables, c.context_lens - np.diff(c.new_cu_lens), c.num_blocks)
    nan = c.key_pool == wl.BF16_NAN_BITS
    assert not (nan.all(axis=(1, 3)) & live_before).any()  # all heads and dims of a slot
