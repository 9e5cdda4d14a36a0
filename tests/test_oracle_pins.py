"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Each test ties one part of the oracle to something other than itself: a
worked example printed on the pages (fixtures under tests/golden/), a closed
form, a 50-digit brute-force softmax, torch's scaled_dot_product_attention
in fp64, or an exact invariance.  The last tests plant mistakes in copies of
the oracle and check that these pins catch them.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import paged_attention as pa
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------------------------------
# Addressing pins
# ------------------------------------------------------------------------------------------


def test_block_table_example_engine_core_page():
    g = _golden("p4_block_table_example.json")
    b = g["block_size"]
    row = np.array(g["block_table"], np.int32)
    for pos, blk in g["physical_block_of_position"].items():
        assert pa.physical_block(row, int(pos), b) == blk
    positions = sorted(int(p) for p in g["slot_of_position"])
    # Every listed position as one sequence of new tokens each (start_pos = position, one token).
    bt = np.tile(row, (len(positions), 1))
    cu = np.arange(len(positions) + 1, dtype=np.int32)
    slots = oracle.slot_mapping(bt, cu, np.array(positions, np.int32), b)
    assert slots.tolist() == [g["slot_of_position"][str(p)] for p in positions]
    # The logical ranges of the example: tokens 16j .. 16j+15 all land in block table[j].
    for j, (lo, hi) in enumerate(g["logical_token_ranges"]):
        s = oracle.slot_mapping(row[None, :], np.array([0, hi - lo + 1], np.int32), np.array([lo], np.int32), b)
        assert (s // b == row[j]).all() and (s % b == np.arange(16)).all()


def test_gather_small_scale_instance():
    g = _golden("p2_gather_small.json")
    nblk, b, D = g["num_blocks"], g["block_size"], g["D"]
    pool = np.zeros((nblk, 1, b, D), np.float32)  # [blocks, KV heads, block size, D]
    for blk in range(nblk):
        for s in range(b):
            pool[blk, 0, s] = 100 * blk + 10 * s + np.arange(D)
    row = np.array(g["block_table"], np.int32)
    got6 = oracle.gather(pool, row, 6)[:, 0]
    got5 = oracle.gather(pool, row, 5)[:, 0]
    assert got6.tolist() == g["gathered_length_6"]
    assert got5.tolist() == g["gathered_length_5"]
    # Entries past ceil(length / b) are never read: poison them with an out-of-range id.
    longer = np.concatenate([row, [10 ** 6]]).astype(np.int32)
    assert oracle.gather(pool, longer, 6)[:, 0].tolist() == g["gathered_length_6"]


@pytest.mark.parametrize("block_size", [2, 16])
@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_write_then_gather_round_trip_is_bit_exact(block_size, storage):
    rng = np.random.default_rng(11)
    hkv, hd, n = 3, 8, 45
    nb = -(-n // block_size)
    nblk = nb + 5
    perm = rng.permutation(nblk).astype(np.int32)
    row = perm[:nb]
    if storage == "f32":
        seq_k = rng.integers(0, 2 ** 32, size=(n, hkv, hd), dtype=np.uint64).astype(np.uint32).view(np.float32)
        seq_v = rng.integers(0, 2 ** 32, size=(n, hkv, hd), dtype=np.uint64).astype(np.uint32).view(np.float32)
        pool = np.zeros((nblk, hkv, block_size, hd), np.float32)
    else:
        seq_k = rng.integers(0, 2 ** 16, size=(n, hkv, hd)).astype(np.uint16)
        seq_v = rng.integers(0, 2 ** 16, size=(n, hkv, hd)).astype(np.uint16)
        pool = np.zeros((nblk, hkv, block_size, hd), np.uint16)
    slots = oracle.slot_mapping(row[None, :], np.array([0, n], np.int32), np.array([0], np.int32), block_size)
    kp, vp = oracle.cache_write(pool, pool, seq_k, seq_v, slots)
    assert oracle.gather(kp, row, n).tobytes() == seq_k.tobytes()
    assert oracle.gather(vp, row, n).tobytes() == seq_v.tobytes()
    # Negative slots skip the token and leave the pool untouched.
    skip = slots.copy()
    skip[::2] = -1
    kp2, _ = oracle.cache_write(pool, pool, seq_k, seq_v, skip)
    flat = kp2.transpose(0, 2, 1, 3).reshape(nblk * block_size, -1)  # one token row per slot
    assert (flat[slots[::2]] == 0).all()
    assert flat[slots[1::2]].tobytes() == seq_k[1::2].reshape(len(slots[1::2]), -1).tobytes()


def test_bf16_widening_matches_torch_over_every_pattern():
    """oracle.as_f64 on bf16 storage against torch's own bf16 type: all 65,536 bit patterns give
    the same value (and sign of zero); NaN patterns give NaN."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
        got = oracle.as_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127  # exponent all ones with a non-zero mantissa, both signs
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_cache_write_rejects_bad_slots():
    pool = np.zeros((2, 1, 16, 4), np.float32)
    k = np.ones((2, 1, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.cache_write(pool, pool, k, k, np.array([3, 3], np.int32))
    with pytest.raises(ValueError):
        oracle.cache_write(pool, pool, k, k, np.array([3, 32], np.int32))


# ------------------------------------------------------------------------------------------
# Attention pins
# ------------------------------------------------------------------------------------------


def _contiguous_kv(case, s, n):
    """Sequence s's first n tokens taken from the case's contiguous new-token arrays (c1 layout:
    all tokens are new and packed by sequence)."""
    lo = int(case.new_cu_lens[s])
    return case.key_new[lo:lo + n], case.value_new[lo:lo + n]


def _sdpa(q, k, v, scale, mask=None, is_causal=False, gqa=False):
    return F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                          attn_mask=None if mask is None else torch.from_numpy(mask),
                                          is_causal=is_causal, scale=scale, enable_gqa=gqa).numpy()


def test_tiny_decode_matches_torch_sdpa_fp64():
    c = wl.tiny_decode()
    slots = oracle.slot_mapping(c.block_tables, c.new_cu_lens, c.new_start_pos, c.block_size)
    kp, vp = oracle.cache_write(c.key_pool, c.value_pool, c.key_new, c.value_new, slots)
    got = oracle.decode(c.query, kp, vp, c.block_tables, c.context_lens, c.scale, c.dtype)
    for s in range(c.num_seqs):
        n = int(c.context_lens[s])
        k, v = _contiguous_kv(c, s, n)
        q = c.query[s].astype(np.float64)[:, None, :]  # [H, 1, hd]
        ref = _sdpa(q, k.astype(np.float64).transpose(1, 0, 2), v.astype(np.float64).transpose(1, 0, 2), c.scale)
        np.testing.assert_allclose(got[s], ref[:, 0], rtol=0, atol=1e-12)


def test_gqa_decode_matches_torch_sdpa_enable_gqa():
    c = wl.random_case(21, kind="decode", dtype="f32", num_seqs=3, num_q_heads=8, num_kv_heads=2,
                       head_dim=16, max_ctx=70, min_ctx=1, new_tokens=False, poison=False)
    got = oracle.decode(c.query, c.key_pool, c.value_pool, c.block_tables, c.context_lens, c.scale, c.dtype)
    for s in range(c.num_seqs):
        n = int(c.context_lens[s])
        # Contiguous K/V assembled directly from pool rows named by the table, without oracle.gather.
        rows_k = np.stack([c.key_pool[c.block_tables[s, p // 16], :, p % 16] for p in range(n)]).astype(np.float64)
        rows_v = np.stack([c.value_pool[c.block_tables[s, p // 16], :, p % 16] for p in range(n)]).astype(np.float64)
        q = c.query[s].astype(np.float64)[:, None, :]
        ref = _sdpa(q, rows_k.transpose(1, 0, 2), rows_v.transpose(1, 0, 2), c.scale, gqa=True)
        np.testing.assert_allclose(got[s], ref[:, 0], rtol=0, atol=1e-12)


def _write_whole_prompt(c):
    slots = oracle.slot_mapping(c.block_tables, c.new_cu_lens, c.new_start_pos, c.block_size)
    return oracle.cache_write(c.key_pool, c.value_pool, c.key_new, c.value_new, slots)


def test_chunked_prefill_matches_torch_sdpa_and_one_pass():
    c = wl.chunked_prefill()
    g = _golden("p3_chunked_prefill_example.json")
    chunks = c.notes["chunks"]
    assert [e - s for s, e in chunks] == g["chunk_lengths"]
    assert len(chunks) == g["printed"]["num_chunks"]
    q64 = oracle.as_f64(c.query, "bf16")
    k64 = oracle.as_f64(c.key_new, "bf16")
    v64 = oracle.as_f64(c.value_new, "bf16")
    # One pass over the prompt (offset 0, L = 1000) after writing it whole.
    kp, vp = _write_whole_prompt(c)
    one = oracle.prefill_chunk(c.query, np.array([0, 1000], np.int32), np.array([0], np.int32), kp, vp,
                               c.block_tables, c.scale, "bf16", causal=True)
    ref = _sdpa(q64.transpose(1, 0, 2), k64.transpose(1, 0, 2), v64.transpose(1, 0, 2), c.scale, is_causal=True)
    np.testing.assert_allclose(one, ref.transpose(1, 0, 2), rtol=0, atol=1e-12)
    # Chunk by chunk: write the chunk's K/V into the paged pool, then attend.
    kp, vp = c.key_pool, c.value_pool
    outs = []
    for (s, e) in chunks:
        slots = oracle.slot_mapping(c.block_tables, np.array([0, e - s], np.int32), np.array([s], np.int32), 16)
        kp, vp = oracle.cache_write(kp, vp, c.key_new[s:e], c.value_new[s:e], slots)
        out = oracle.prefill_chunk(c.query[s:e], np.array([0, e - s], np.int32), np.array([s], np.int32), kp, vp,
                                   c.block_tables, c.scale, "bf16", causal=True)
        # Each chunk against SDPA with an explicit boolean mask over absolute positions.
        mask = np.arange(e)[None, :] <= np.arange(s, e)[:, None]
        r = _sdpa(q64[s:e].transpose(1, 0, 2), k64[:e].transpose(1, 0, 2), v64[:e].transpose(1, 0, 2), c.scale,
                  mask=mask)
        np.testing.assert_allclose(out, r.transpose(1, 0, 2), rtol=0, atol=1e-12)
        outs.append(out)
    chunked = np.concatenate(outs, axis=0)
    assert np.max(np.abs(chunked - one)) <= 1e-12


def test_chunked_fp32_equals_one_pass_at_the_page_tolerance():
    """The property the Chunked Prefill page's example prints (True): the prompt cut into the page's
    chunks, each chunk attending over the cache after its own K/V was stored, gives the one-pass
    causal result within the page's fp32 tolerance.  Chunk bounds, sizes, head shape and tolerance
    come from the fixture; the values are a seeded fp32 N(0,1) draw.  The chunks run through the
    oracle over a paged pool with shuffled block ids (dead slots NaN); the one-pass result is
    torch's fp32 attention with its built-in causal mask."""
    g = _golden("p3_chunked_prefill_example.json")
    setup = g["setup"]
    n, H, hd = setup["prompt_len"], setup["heads"], setup["head_dim"]
    bounds = np.cumsum([0] + g["chunk_lengths"])
    assert bounds[-1] == n and len(g["chunk_lengths"]) == g["printed"]["num_chunks"]
    rng = np.random.default_rng(setup["seed"])
    q, k, v = (rng.standard_normal((n, H, hd)).astype(np.float32) for _ in range(3))
    nb = -(-n // 16)
    nblk = nb + 5
    bt = rng.permutation(nblk)[:nb].astype(np.int32)[None, :]
    kp = np.full((nblk, H, 16, hd), np.nan, np.float32)
    vp = kp.copy()
    chunks = []
    for s, e in zip(bounds[:-1], bounds[1:]):
        cu, start = np.array([0, e - s], np.int32), np.array([s], np.int32)
        kp, vp = oracle.cache_write(kp, vp, k[s:e], v[s:e], oracle.slot_mapping(bt, cu, start, 16))
        chunks.append(oracle.prefill_chunk(q[s:e], cu, start, kp, vp, bt, 1.0 / math.sqrt(hd), "f32"))
    chunked = np.concatenate(chunks)
    heads_first = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))
    one = F.scaled_dot_product_attention(heads_first(q), heads_first(k), heads_first(v), is_causal=True)
    one = one.numpy().transpose(1, 0, 2).astype(np.float64)
    assert np.isfinite(chunked).all()
    assert np.allclose(chunked, one, rtol=0, atol=setup["atol"]) == g["printed"]["same_as_one_pass"]


def _decimal_attention(q, K, V, scale_sq_inv):
    """out = sum_j exp(s_j) v_j / sum_j exp(s_j) at 50 digits, no max subtraction.  The fp64 oracle
    may differ by rounding only: a few ulp of max|v| per term, so 1e-14 absolute on O(1) values."""
    getcontext().prec = 50
    sc = Decimal(1) / Decimal(scale_sq_inv).sqrt()
    qs = [Decimal(float(x)) for x in q]
    ws = []
    for krow in K:
        sdot = sum(qs[d] * Decimal(float(krow[d])) for d in range(len(qs)))
        ws.append((sc * sdot).exp())
    tot = sum(ws)
    return [float(sum(ws[j] * Decimal(float(V[j][d])) for j in range(len(ws))) / tot) for d in range(V.shape[1])]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decimal_bruteforce_decode_and_prefill(seed):
    rng = np.random.default_rng(100 + seed)
    hd, n = 4, 5
    hq, hkv = 2, 1
    k = (rng.standard_normal((n, hkv, hd)) * 2).astype(np.float32)
    v = rng.standard_normal((n, hkv, hd)).astype(np.float32)
    q = (rng.standard_normal((1, hq, hd)) * 2).astype(np.float32)
    bt = np.array([[1]], np.int32)
    pool = np.zeros((2, hkv, 16, hd), np.float32)
    kp, vp = oracle.cache_write(pool, pool, k, v, np.arange(16, 16 + n, dtype=np.int32))
    scale = 1.0 / math.sqrt(hd)
    got = oracle.decode(q, kp, vp, bt, np.array([n], np.int32), scale, "f32")
    for h in range(hq):
        ref = _decimal_attention(q[0, h], k[:, 0], v[:, 0], hd)
        np.testing.assert_allclose(got[0, h], ref, rtol=0, atol=1e-14)
    # Prefill: the chunk is the last 3 of 5 positions (offset 2); row i sees 2 + i + 1 keys.
    qc = (rng.standard_normal((3, hq, hd)) * 2).astype(np.float32)
    gotp = oracle.prefill_chunk(qc, np.array([0, 3], np.int32), np.array([2], np.int32), kp, vp, bt, scale, "f32")
    for i in range(3):
        for h in range(hq):
            ref = _decimal_attention(qc[i, h], k[:3 + i, 0], v[:3 + i, 0], hd)
            np.testing.assert_allclose(gotp[i, h], ref, rtol=0, atol=1e-14)
    # Non-causal: every row sees all 5 keys.
    gotn = oracle.prefill_chunk(qc, np.array([0, 3], np.int32), np.array([2], np.int32), kp, vp, bt, scale, "f32",
                                causal=False)
    for i in range(3):
        ref = _decimal_attention(qc[i, 0], k[:, 0], v[:, 0], hd)
        np.testing.assert_allclose(gotn[i, 0], ref, rtol=0, atol=1e-14)


def test_closed_forms():
    rng = np.random.default_rng(5)
    hd = 8
    pool = np.zeros((4, 1, 16, hd), np.float32)
    v = rng.standard_normal((40, 1, hd)).astype(np.float32)
    k = rng.standard_normal((40, 1, hd)).astype(np.float32)
    bt = np.array([[2, 0, 3]], np.int32)
    slots = oracle.slot_mapping(bt, np.array([0, 40], np.int32), np.array([0], np.int32), 16)
    q = rng.standard_normal((1, 1, hd)).astype(np.float32)
    # ctx = 1: the output is the first value row exactly.
    kp, vp = oracle.cache_write(pool, pool, k, v, slots)
    out = oracle.decode(q, kp, vp, bt, np.array([1], np.int32), 0.3, "f32")
    assert (out[0, 0] == v[0, 0].astype(np.float64)).all()
    # ctx = 0: zero row.
    out0 = oracle.decode(q, kp, vp, bt, np.array([0], np.int32), 0.3, "f32")
    assert (out0 == 0).all()
    # Identical keys: the output is the mean of the value rows.
    ksame = np.repeat(k[:1], 40, axis=0)
    kp2, vp2 = oracle.cache_write(pool, pool, ksame, v, slots)
    out2 = oracle.decode(q, kp2, vp2, bt, np.array([40], np.int32), 0.3, "f32")
    np.testing.assert_allclose(out2[0, 0], v[:, 0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-15)
    # One score 40 above all others: the output is that value row to within e^-40.
    q1 = np.zeros((1, 1, hd), np.float32)
    q1[0, 0, 0] = 1.0
    kd = np.zeros((40, 1, hd), np.float32)
    kd[17, 0, 0] = 40.0
    kp3, vp3 = oracle.cache_write(pool, pool, kd, v, slots)
    out3 = oracle.decode(q1, kp3, vp3, bt, np.array([40], np.int32), 1.0, "f32")
    bound = 39 * math.exp(-40.0) * np.abs(v[:, 0]).max() * 2
    assert np.max(np.abs(out3[0, 0] - v[17, 0])) <= bound


def test_block_permutation_leaves_output_bit_identical():
    c = wl.random_case(31, kind="decode", dtype="bf16", num_seqs=4, num_q_heads=4, num_kv_heads=2, head_dim=32,
                       max_ctx=90, min_ctx=1, new_tokens=False, poison=True)
    rng = np.random.default_rng(3)
    perm = rng.permutation(c.num_blocks).astype(np.int32)
    kp = np.empty_like(c.key_pool)
    vp = np.empty_like(c.value_pool)
    kp[perm] = c.key_pool
    vp[perm] = c.value_pool
    bt = c.block_tables.copy()
    used = bt != wl.UNUSED_BLOCK_ID
    bt[used] = perm[bt[used]]
    a = oracle.decode(c.query, c.key_pool, c.value_pool, c.block_tables, c.context_lens, c.scale, "bf16")
    b = oracle.decode(c.query, kp, vp, bt, c.context_lens, c.scale, "bf16")
    assert a.tobytes() == b.tobytes()


def test_decode_equals_last_prefill_row():
    c = wl.random_case(41, kind="decode", dtype="bf16", num_seqs=5, num_q_heads=4, num_kv_heads=4, head_dim=16,
                       max_ctx=70, min_ctx=1, new_tokens=False, poison=True)
    dec = oracle.decode(c.query, c.key_pool, c.value_pool, c.block_tables, c.context_lens, c.scale, "bf16")
    for s in range(c.num_seqs):
        n = int(c.context_lens[s])
        # A causal prefill over all n positions whose last row is this query.
        q = np.zeros((n, c.num_q_heads, c.head_dim), np.uint16)
        q[-1] = c.query[s]
        pre = oracle.prefill_chunk(q, np.array([0, n], np.int32), np.array([0], np.int32), c.key_pool, c.value_pool,
                                   c.block_tables[s:s + 1], c.scale, "bf16")
        assert np.max(np.abs(pre[-1] - dec[s])) <= 1e-13


def test_gqa_equals_repeated_mha():
    c = wl.random_case(51, kind="decode", dtype="f32", num_seqs=3, num_q_heads=8, num_kv_heads=2, head_dim=16,
                       max_ctx=60, min_ctx=1, new_tokens=False, poison=False)
    G = 4
    kp = np.repeat(c.key_pool, G, axis=1)  # the KV-head axis of [blocks, Hkv, 16, hd]
    vp = np.repeat(c.value_pool, G, axis=1)
    a = oracle.decode(c.query, c.key_pool, c.value_pool, c.block_tables, c.context_lens, c.scale, "f32")
    b = oracle.decode(c.query, kp, vp, c.block_tables, c.context_lens, c.scale, "f32")
    assert np.max(np.abs(a - b)) <= 1e-13


@pytest.mark.parametrize("split", [16, 48, 512])
def test_split_partials_combine_to_unsplit(split):
    c = wl.random_case(61, kind="decode", dtype="bf16", num_seqs=4, num_q_heads=4, num_kv_heads=2, head_dim=16,
                       max_ctx=300, min_ctx=1, new_tokens=False, poison=True)
    full = oracle.decode(c.query, c.key_pool, c.value_pool, c.block_tables, c.context_lens, c.scale, "bf16")
    parts = oracle.decode_split_partials(c.query, c.key_pool, c.value_pool, c.block_tables, c.context_lens,
                                         c.scale, "bf16", split)
    for (s, h), (o, m, l) in parts.items():
        assert len(m) == -(-int(c.context_lens[s]) // split)
        np.testing.assert_allclose(oracle.combine_splits(o, m, l), full[s, h], rtol=0, atol=1e-14)


# ------------------------------------------------------------------------------------------
# Planted mistakes: each mutated copy of the oracle must fail at least one pin above.
# ------------------------------------------------------------------------------------------


def _run_pins():
    failures = 0
    for fn in (test_block_table_example_engine_core_page, test_gather_small_scale_instance,
               test_bf16_widening_matches_torch_over_every_pattern,
               test_tiny_decode_matches_torch_sdpa_fp64, test_gqa_decode_matches_torch_sdpa_enable_gqa,
               test_closed_forms):
        try:
            fn()
        except Exception:
            failures += 1
    for seed in (0,):
        try:
            test_decimal_bruteforce_decode_and_prefill(seed)
        except Exception:
            failures += 1
    return failures


def test_pins_pass_on_the_oracle_as_written():
    assert _run_pins() == 0


@pytest.mark.parametrize("mutation", ["slot_offset", "kv_head_modulo", "causal_off_by_one", "gather_order",
                                      "scale_dropped", "bf16_no_widening"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    if mutation == "slot_offset":
        monkeypatch.setattr(pa, "physical_block", lambda row, p, b: int(row[p // b - 1 if p >= b else 0]))
    elif mutation == "kv_head_modulo":
        monkeypatch.setattr(pa, "kv_head_of", lambda h, hq, hkv: h % hkv)
    elif mutation == "causal_off_by_one":
        monkeypatch.setattr(pa, "visible_keys", lambda row, o, L, causal: o + row if causal else o + L)
    elif mutation == "gather_order":
        orig = pa.gather

        def reversed_blocks(pool, row, length):
            b = pool.shape[2]
            nb = -(-int(length) // b)
            return orig(pool, np.concatenate([row[:nb][::-1], row[nb:]]), length)
        monkeypatch.setattr(pa, "gather", reversed_blocks)
    elif mutation == "bf16_no_widening":
        orig_f64 = pa.as_f64

        def narrow_shift(x, dtype):
            if dtype != "bf16":
                return orig_f64(x, dtype)
            # The shift done in 16 bits: the pattern is lost before it reaches the fp32 exponent.
            bits = (np.asarray(x, dtype=np.uint16) << np.uint16(16)).astype(np.uint32)
            return bits.view(np.float32).astype(np.float64)
        monkeypatch.setattr(pa, "as_f64", narrow_shift)
        monkeypatch.setattr(oracle, "as_f64", narrow_shift)
    elif mutation == "scale_dropped":
        orig_sa = pa.softmax_attention
        monkeypatch.setattr(pa, "softmax_attention", lambda q, K, V, scale, vis: orig_sa(q, K, V, 1.0, vis))
    assert _run_pins() > 0
