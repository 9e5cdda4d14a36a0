"""GPU parity at the edges of the supported shapes (needs an MI355X): the largest GQA group at the
largest head_dim, contexts long enough for many decode splits, thousands of decode sequences, the
largest number of prefill key splits, and a prefill chunk spanning many row tiles.  Same bars as
test_gpu_parity (bf16 inputs: max-abs 1e-2, mean-abs 1e-3 against the fp64 oracle), both call
modes, NaN-poisoned dead slots.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_common import MODES, flag, new_err
from test_gpu_parity import Dev, assert_close, oracle_pools_after_write, to_dev, write_new_tokens

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_170_amd as m
    return m


@pytest.fixture()
def dev(pkv):
    return torch.device("cuda:0")


def _decode_case_check(pkv, dev, mode, c, splits=(0,)):
    d = Dev(c, dev)
    err = new_err(dev, mode)
    slots = write_new_tokens(pkv, d, err)
    rk, rv = oracle_pools_after_write(c, slots)
    ref = oracle.decode(c.query, rk, rv, c.block_tables, c.context_lens, c.scale, c.dtype)
    q = to_dev(c.query, dev, c.dtype)
    for split in splits:
        out = pkv.paged_attn_decode(q, d.kp, d.vp, d.bt, d.ctx, c.scale, err_flag=err, split_tokens=split)
        mx, mean = assert_close(out.cpu().numpy(), ref, c.dtype, f"decode split={split}")
        _say(f"  split {split}: max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert flag(err) == 0


@pytest.mark.parametrize("mode", MODES)
def test_decode_long_contexts_many_splits(pkv, dev, mode):
    c = wl.random_case(71, kind="decode", dtype="bf16", num_seqs=3, num_q_heads=16, num_kv_heads=2, head_dim=128,
                       max_ctx=32768, min_ctx=20000, poison=True)
    _say(f"case decode, long contexts {c.context_lens.tolist()} (up to 16 splits of 2048), 16/2 heads x 128")
    _decode_case_check(pkv, dev, mode, c, splits=(0, 512))


@pytest.mark.parametrize("mode", MODES)
def test_decode_thousands_of_sequences(pkv, dev, mode):
    c = wl.random_case(72, kind="decode", dtype="bf16", num_seqs=2000, num_q_heads=8, num_kv_heads=8, head_dim=64,
                       max_ctx=80, min_ctx=0, poison=True)
    _say(f"case decode, 2000 sequences, contexts 0..80 ({int((c.context_lens == 0).sum())} empty), 8/8 heads x 64")
    _decode_case_check(pkv, dev, mode, c)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", MODES)
def test_decode_group16_head_dim_256(pkv, dev, mode, dtype):
    c = wl.random_case(73, kind="decode", dtype=dtype, num_seqs=5, num_q_heads=16, num_kv_heads=1, head_dim=256,
                       max_ctx=3000, min_ctx=1, poison=True)
    _say(f"case decode, {dtype}, a group of 16 query heads over one KV head x 256, contexts {c.context_lens.tolist()}")
    _decode_case_check(pkv, dev, mode, c, splits=(0, 256))


def _prefill_case_check(pkv, dev, mode, c):
    d = Dev(c, dev)
    err = new_err(dev, mode)
    slots = write_new_tokens(pkv, d, err)
    rk, rv = oracle_pools_after_write(c, slots)
    maxl = int(np.diff(c.cu_q_lens).max())
    ws = pkv.prefill_workspace(to_dev(c.query, dev, c.dtype), len(c.chunk_offsets), maxl, c.block_tables.shape[1])
    out = pkv.paged_attn_prefill_chunk(to_dev(c.query, dev, c.dtype), to_dev(c.cu_q_lens, dev),
                                       to_dev(c.chunk_offsets, dev), d.kp, d.vp, d.bt, maxl, c.scale,
                                       causal=c.causal, err_flag=err, workspace=ws)
    ref = oracle.prefill_chunk(c.query, c.cu_q_lens, c.chunk_offsets, rk, rv, c.block_tables, c.scale, c.dtype,
                               causal=c.causal)
    mx, mean = assert_close(out.cpu().numpy(), ref, c.dtype, "prefill")
    _say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert flag(err) == 0
    return ws


@pytest.mark.parametrize("mode", MODES)
def test_prefill_largest_key_split(pkv, dev, mode):
    # One sequence and 8 query heads: 8 row tiles, so the key range is cut into the largest
    # number of splits (8) once the context holds at least 8 tile pairs.
    seed = next(s for s in range(100) if wl.random_case(s, kind="prefill", dtype="bf16", num_seqs=1, num_q_heads=8,
                                                        num_kv_heads=1, head_dim=128, max_ctx=6000, min_ctx=90,
                                                        q_len_max=100, poison=False).chunk_offsets[0] >= 2000)
    c = wl.random_case(seed, kind="prefill", dtype="bf16", num_seqs=1, num_q_heads=8, num_kv_heads=1, head_dim=128,
                       max_ctx=6000, min_ctx=90, q_len_max=100, poison=True)
    L, off = int(c.cu_q_lens[1]), int(c.chunk_offsets[0])
    _say(f"case prefill, one chunk of {L} rows at offset {off}, 8/1 heads x 128 (8 key splits)")
    ws = _prefill_case_check(pkv, dev, mode, c)
    # The workspace holds eight splits' partial rows: [8 row tiles][8 splits][256 rows] x (128 + 2) floats.
    assert ws is not None and ws.numel() >= 8 * 8 * 256 * (128 + 2) * 4


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("mode", MODES)
def test_prefill_group16_head_dim_256(pkv, dev, mode, causal):
    c = wl.random_case(74, kind="prefill", dtype="bf16", num_seqs=3, num_q_heads=16, num_kv_heads=1, head_dim=256,
                       max_ctx=1500, min_ctx=1, q_len_max=300, causal=causal, poison=True)
    _say(f"case prefill, a group of 16 over one KV head x 256, chunks {np.diff(c.cu_q_lens).tolist()} at offsets "
         f"{c.chunk_offsets.tolist()}, causal={causal}")
    _prefill_case_check(pkv, dev, mode, c)


@pytest.mark.parametrize("mode", MODES)
def test_prefill_chunk_of_many_row_tiles(pkv, dev, mode):
    c = wl.random_case(75, kind="prefill", dtype="bf16", num_seqs=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                       max_ctx=4500, min_ctx=2000, q_len_max=2100, poison=True)
    L, off = int(c.cu_q_lens[1]), int(c.chunk_offsets[0])
    _say(f"case prefill, one chunk of {L} rows ({-(-L // 256)} row tiles) at offset {off}, 4/1 heads x 64")
    _prefill_case_check(pkv, dev, mode, c)


@pytest.mark.parametrize("mode", MODES)
def test_prefill_block_id_window_slides(pkv, dev, mode):
    # The prefill stages the block ids of 2,048 blocks (32,768 positions) in LDS and moves that
    # window on when a key split reads past it.  A 1,024-row chunk over 64 query heads gives 256
    # row tiles, so one key split covers the whole context, here 35,538 positions (2,222 blocks).
    # The oracle checks 24 rows (at the start, middle and end of the chunk) of every head.
    c = wl.random_case(122, kind="prefill", dtype="bf16", num_seqs=1, num_q_heads=64, num_kv_heads=8, head_dim=64,
                       max_ctx=41000, min_ctx=1024, q_len_max=1024, poison=True)
    L, off = int(c.cu_q_lens[1]), int(c.chunk_offsets[0])
    assert L == 1024 and off + L > 32768 + 1024, "the case must read past the first id window"
    _say(f"case prefill, one chunk of {L} rows at offset {off} ({-(-(off + L) // 16)} blocks), 64/8 heads x 64")
    assert pkv.prefill_workspace_bytes(1, L, 64, 64, c.block_tables.shape[1]) == 0  # one key split
    d = Dev(c, dev)
    err = new_err(dev, mode)
    slots = write_new_tokens(pkv, d, err)
    rk, rv = oracle_pools_after_write(c, slots)
    out = pkv.paged_attn_prefill_chunk(to_dev(c.query, dev, c.dtype), to_dev(c.cu_q_lens, dev),
                                       to_dev(c.chunk_offsets, dev), d.kp, d.vp, d.bt, L, c.scale, causal=True,
                                       err_flag=err).cpu().numpy()
    assert flag(err) == 0
    for i0 in (0, 508, 1016):
        sub = slice(i0, i0 + 8)
        ref = oracle.prefill_chunk(c.query[sub], np.array([0, 8], np.int32), np.array([off + i0], np.int32), rk, rv,
                                   c.block_tables, c.scale, c.dtype)
        mx, mean = assert_close(out[sub], ref, c.dtype, f"prefill rows {i0}..{i0 + 7}")
        _say(f"  rows {i0}..{i0 + 7}: max-abs {mx:.2e} mean-abs {mean:.2e}")


def _ramp_keys(c, top=4.0):
    """Scale every live key row by 1 + (top - 1) * position / longest context (bf16, nearest-even),
    so that scores keep growing along each sequence."""
    kf = (c.key_pool.astype(np.uint32) << 16).view(np.float32)
    lens = c.context_lens if c.kind == "decode" else c.chunk_offsets + np.diff(c.cu_q_lens)
    longest = int(lens.max())
    for s in range(c.num_seqs):
        for j in range(int(lens[s])):
            b = int(c.block_tables[s, j // 16])
            kf[b, :, j % 16, :] *= np.float32(1.0 + (top - 1.0) * j / longest)
    c.key_pool[...] = wl.f32_to_bf16_bits(kf)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_softmax_reference_raised_mid_sequence(pkv, dev, mode, kind):
    # Scale 1.0 (scores of N(0,1) rows at head_dim 128 spread over about +-40 in log2 units) and
    # keys that grow 4x along the context: later tiles keep holding weights far above 2^20 times
    # the reference the earlier tiles set (up to exponentials that overflow), so the kernels take
    # their raise-and-recompute path again and again, not only on the first tile.
    if kind == "decode":
        c = wl.random_case(76, kind="decode", dtype="bf16", num_seqs=6, num_q_heads=16, num_kv_heads=2,
                           head_dim=128, max_ctx=3000, min_ctx=1500, poison=True, new_tokens=False)
    else:
        c = wl.random_case(77, kind="prefill", dtype="bf16", num_seqs=2, num_q_heads=16, num_kv_heads=2,
                           head_dim=128, max_ctx=3000, min_ctx=100, q_len_max=300, poison=True, new_tokens=False)
    _ramp_keys(c)
    scale = 1.0
    _say(f"case {kind}, keys ramped 1x..4x along the context, scale {scale}")
    d = Dev(c, dev)
    err = new_err(dev, mode)
    q = to_dev(c.query, dev, c.dtype)
    if kind == "decode":
        ref = oracle.decode(c.query, c.key_pool, c.value_pool, c.block_tables, c.context_lens, scale, c.dtype)
        outs = [pkv.paged_attn_decode(q, d.kp, d.vp, d.bt, d.ctx, scale, split_tokens=s, err_flag=err)
                for s in (0, 256)]
    else:
        ref = oracle.prefill_chunk(c.query, c.cu_q_lens, c.chunk_offsets, c.key_pool, c.value_pool, c.block_tables,
                                   scale, c.dtype)
        maxl = int(np.diff(c.cu_q_lens).max())
        outs = [pkv.paged_attn_prefill_chunk(q, to_dev(c.cu_q_lens, dev), to_dev(c.chunk_offsets, dev), d.kp, d.vp,
                                             d.bt, maxl, scale, causal=True, err_flag=err)]
    for i, o in enumerate(outs):
        mx, mean = assert_close(o.cpu().numpy(), ref, c.dtype, f"{kind} #{i}")
        _say(f"  #{i}: max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert flag(err) == 0
