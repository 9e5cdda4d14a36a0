"""GPU parity of the FP8 (E4M3) KV pool path against the oracle (needs an MI355X).

Bars: the quantising write is bit-exact (whole code pools compared byte for byte against
oracle/fp8.py); decode and prefill over FP8 pools are compared with exact attention over the
dequantised pools (value(code) * scale) at the bf16 tolerance (max-abs <= 1e-2, mean-abs <= 1e-3),
and a one-key decode returns the dequantised V rows exactly.  Every test runs in both call modes
(checked kernels with an err_flag, and the release kernels production callers run, err_flag NULL).
Pools are built by quantising the
bf16 pools of the ordinary generators (dead slots hold NaN there, so they become NaN codes here and
any stray read shows up); scales: K 0.0123 (not a power of two, some inputs saturate), V 2^-5.
"""
import sys

import numpy as np
import pytest

import oracle
from oracle import fp8 as ofp8
import workloads as wl
from gpu_common import MODES, flag, fp8_decode_reference, fp8_prefill_reference, mixed_step_case, new_err

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3
K_SCALE, V_SCALE = 0.0123, 2.0 ** -5


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


def to_dev(a, dev, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if bf16 else t).to(dev)


def f32_of(bits_bf16):
    return oracle.as_f64(bits_bf16, "bf16").astype(np.float32)


def codes_of(t):
    return t.cpu().view(torch.uint8).numpy()


def quantised_pools(pkv, c, dev, err):
    """FP8 pools of a bf16 case: every slot of its bf16 pools quantised by the GPU write, checked
    byte for byte against the oracle's quantisation."""
    nblk, hkv, b, hd = c.key_pool.shape
    rows_k = wl.slot_rows(c.key_pool)
    rows_v = wl.slot_rows(c.value_pool)
    kp = torch.zeros((nblk, hkv, b, hd), dtype=torch.float8_e4m3fn, device=dev)
    vp = torch.zeros_like(kp)
    slots = torch.arange(nblk * b, dtype=torch.int32, device=dev)
    pkv.cache_write_fp8(to_dev(rows_k, dev, True), to_dev(rows_v, dev, True), kp, vp, slots, K_SCALE, V_SCALE,
                        err_flag=err)
    rk = ofp8.quantize_bf16_bits(c.key_pool, K_SCALE)
    rv = ofp8.quantize_bf16_bits(c.value_pool, V_SCALE)
    assert codes_of(kp).tobytes() == rk.tobytes(), "K codes differ from the oracle"
    assert codes_of(vp).tobytes() == rv.tobytes(), "V codes differ from the oracle"
    return kp, vp, rk, rv


def write_new(pkv, c, dev, kp, vp, rk, rv, err):
    """Slot-map and quantise-write the case's new tokens; returns the oracle's pools after it."""
    T = c.num_new_tokens
    if T == 0:
        return rk, rv
    maxlen = int(np.diff(c.new_cu_lens).max())
    slots = pkv.slot_mapping(to_dev(c.block_tables, dev), to_dev(c.new_cu_lens, dev), to_dev(c.new_start_pos, dev),
                             maxlen, c.num_blocks, err_flag=err, total=T)
    pkv.cache_write_fp8(to_dev(c.key_new, dev, True), to_dev(c.value_new, dev, True), kp, vp, slots, K_SCALE,
                        V_SCALE, err_flag=err)
    ref_slots = oracle.slot_mapping(c.block_tables, c.new_cu_lens, c.new_start_pos, 16)
    rk, rv = ofp8.cache_write_fp8(rk, rv, f32_of(c.key_new), f32_of(c.value_new), ref_slots, K_SCALE, V_SCALE)
    assert codes_of(kp).tobytes() == rk.tobytes() and codes_of(vp).tobytes() == rv.tobytes()
    return rk, rv


def close(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, f"{what}: max-abs {d.max():.3e} mean-abs {d.mean():.3e}"
    return d.max(), d.mean()


@pytest.mark.parametrize("mode", MODES)
def test_quantising_write_bit_exact_special_values(pkv, dev, mode):
    """Ties, subnormals, saturation, signed zeros, infinities and NaN, from bf16 and fp32 rows,
    with strided input rows and skipped (negative) slots."""
    _say("case fp8 write: special values, bf16 and fp32 inputs")
    rng = np.random.default_rng(11)
    nblk, hkv, hd, T = 12, 2, 64, 150
    special = np.array([0.0, -0.0, 448.0, -448.0, 464.0, 500.0, 1e30, np.inf, -np.inf, np.nan, 2.0 ** -10,
                        3 * 2.0 ** -10, -2.0 ** -11, 1.0625, 1.1875, 2.0 ** -6, 2.0 ** -130], np.float32)
    for in_dt in ("f32", "bf16"):
        for scale in (1.0, K_SCALE):
            x = (rng.standard_normal((T, hkv, hd)) * rng.choice([0.01, 1, 4], (T, 1, 1))).astype(np.float32)
            x.reshape(-1)[: special.size * 4] = np.tile(special * np.float32(scale), 4)
            if in_dt == "bf16":
                bits = wl.f32_to_bf16_bits(x)
                xin = to_dev(np.stack([bits, bits], axis=1), dev, True)[:, 0]  # strided token rows
                xf = f32_of(bits)
            else:
                xin = to_dev(np.stack([x, x], axis=1), dev)[:, 0]
                xf = x
            assert xin.stride(0) == 2 * hkv * hd
            slots = rng.permutation(nblk * 16)[:T].astype(np.int32)
            slots[::7] = -1
            kp0 = rng.integers(0, 256, (nblk, hkv, 16, hd), dtype=np.uint8)
            vp0 = rng.integers(0, 256, (nblk, hkv, 16, hd), dtype=np.uint8)
            kp, vp = to_dev(kp0, dev).view(torch.float8_e4m3fn), to_dev(vp0, dev).view(torch.float8_e4m3fn)
            err = new_err(dev, mode)
            pkv.cache_write_fp8(xin, xin, kp, vp, to_dev(slots, dev), scale, V_SCALE, err_flag=err)
            rk, rv = ofp8.cache_write_fp8(kp0, vp0, xf, xf, slots, scale, V_SCALE)
            assert codes_of(kp).tobytes() == rk.tobytes(), f"K codes differ ({in_dt}, scale {scale})"
            assert codes_of(vp).tobytes() == rv.tobytes(), f"V codes differ ({in_dt}, scale {scale})"
            assert flag(err) == 0


@pytest.mark.parametrize("mode", MODES)
def test_one_key_decode_returns_dequantised_values(pkv, dev, mode):
    """With one cached position the softmax weight is exactly 1, so the output is the dequantised V
    row: every finite code times the power-of-two V scale, exactly."""
    _say("case fp8 decode: one-key sequences over every code")
    hq, hkv, hd = 8, 4, 128
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n_seq = 8
    row = np.resize(codes, (n_seq, hkv * hd))
    vp0 = np.zeros((n_seq, hkv, 16, hd), np.uint8)
    vp0[:, :, 0] = row.reshape(n_seq, hkv, hd)  # offset 0 of each block, every KV head
    rng = np.random.default_rng(2)
    kp0 = rng.integers(0, 0x70, (n_seq, hkv, 16, hd), dtype=np.uint8)  # finite K codes
    kp, vp = to_dev(kp0, dev).view(torch.float8_e4m3fn), to_dev(vp0, dev).view(torch.float8_e4m3fn)
    q = to_dev(wl.f32_to_bf16_bits(rng.standard_normal((n_seq, hq, hd)).astype(np.float32)), dev, True)
    bt = to_dev(np.arange(n_seq, dtype=np.int32)[:, None], dev)
    ctx = to_dev(np.ones(n_seq, np.int32), dev)
    out = pkv.paged_attn_decode_fp8(q, kp, vp, bt, ctx, hd ** -0.5, K_SCALE, V_SCALE,
                                    err_flag=new_err(dev, mode)).cpu().numpy()
    want = ofp8.dequantize(vp0[:, :, 0], V_SCALE)  # [n_seq, hkv, hd]
    for h in range(hq):
        assert np.array_equal(out[:, h].astype(np.float64), want[:, oracle.kv_head_of(h, hq, hkv)])


FP8_DECODE = [
    # (hq, hkv, hd, max_ctx, min_ctx)
    (64, 8, 128, 2000, 1),
    (16, 4, 256, 1100, 1),
    (8, 8, 64, 300, 0),
    (16, 1, 128, 1300, 1),
    (16, 1, 256, 1500, 1),
]


@pytest.mark.parametrize("hq,hkv,hd,max_ctx,min_ctx", FP8_DECODE)
@pytest.mark.parametrize("mode", MODES)
def test_fp8_decode_matches_oracle(pkv, dev, mode, hq, hkv, hd, max_ctx, min_ctx):
    _say(f"case fp8 decode: hq={hq} hkv={hkv} hd={hd} ctx<={max_ctx}")
    c = wl.random_case(5 * hq + hd + max_ctx, kind="decode", dtype="bf16", num_seqs=9, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=hd, max_ctx=max_ctx, min_ctx=min_ctx, poison=True)
    err = new_err(dev, mode)
    kp, vp, rk, rv = quantised_pools(pkv, c, dev, err)
    rk, rv = write_new(pkv, c, dev, kp, vp, rk, rv, err)
    ref = oracle.decode(c.query, ofp8.dequantize(rk, K_SCALE), ofp8.dequantize(rv, V_SCALE), c.block_tables,
                        c.context_lens, c.scale, "bf16", kv_dtype="f64")
    q, bt, ctx = to_dev(c.query, dev, True), to_dev(c.block_tables, dev), to_dev(c.context_lens, dev)
    for split in (0, 128):
        out = pkv.paged_attn_decode_fp8(q, kp, vp, bt, ctx, c.scale, K_SCALE, V_SCALE, split_tokens=split,
                                        err_flag=err)
        mx, mean = close(out.cpu().numpy(), ref, f"fp8 decode split={split}")
    _say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert flag(err) == 0


@pytest.mark.parametrize("mode", MODES)
def test_fp8_chunked_prefill_equals_one_pass(pkv, dev, mode):
    _say("case fp8 chunked prefill: 1000 tokens in chunks 256/256/256/232, 8 heads x 64")
    c = wl.chunked_prefill(poison=True)
    err = new_err(dev, mode)
    kp, vp, rk, rv = quantised_pools(pkv, c, dev, err)
    bt = to_dev(c.block_tables, dev)
    outs = []
    for (s, e) in c.notes["chunks"]:
        cu1 = np.array([0, e - s], np.int32)
        st1 = np.array([s], np.int32)
        slots = pkv.slot_mapping(bt, to_dev(cu1, dev), to_dev(st1, dev), e - s, c.num_blocks, err_flag=err,
                                 total=e - s)
        pkv.cache_write_fp8(to_dev(c.key_new[s:e], dev, True), to_dev(c.value_new[s:e], dev, True), kp, vp, slots,
                            K_SCALE, V_SCALE, err_flag=err)
        rs = oracle.slot_mapping(c.block_tables, cu1, st1, 16)
        rk, rv = ofp8.cache_write_fp8(rk, rv, f32_of(c.key_new[s:e]), f32_of(c.value_new[s:e]), rs, K_SCALE, V_SCALE)
        out = pkv.paged_attn_prefill_chunk_fp8(to_dev(c.query[s:e], dev, True), to_dev(cu1, dev), to_dev(st1, dev),
                                               kp, vp, bt, e - s, c.scale, K_SCALE, V_SCALE, err_flag=err)
        outs.append(out.cpu().numpy())
    assert codes_of(kp).tobytes() == rk.tobytes() and codes_of(vp).tobytes() == rv.tobytes()
    one = oracle.prefill_chunk(c.query, np.array([0, 1000], np.int32), np.array([0], np.int32),
                               ofp8.dequantize(rk, K_SCALE), ofp8.dequantize(rv, V_SCALE), c.block_tables, c.scale,
                               "bf16", kv_dtype="f64")
    mx, mean = close(np.concatenate(outs), one, "fp8 chunked vs one pass")
    _say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert flag(err) == 0


FP8_PREFILL = [
    # (hq, hkv, hd, max_ctx, q_len_max, causal)
    (16, 2, 128, 700, 300, True),
    (8, 1, 128, 300, 129, False),
    (4, 4, 256, 500, 200, True),
    (32, 2, 128, 1200, 513, True),
    (16, 1, 256, 900, 200, True),
    (8, 8, 64, 400, 150, True),
]


@pytest.mark.parametrize("hq,hkv,hd,max_ctx,q_len_max,causal", FP8_PREFILL)
@pytest.mark.parametrize("mode", MODES)
def test_fp8_prefill_matches_oracle(pkv, dev, mode, hq, hkv, hd, max_ctx, q_len_max, causal):
    _say(f"case fp8 prefill: hq={hq} hkv={hkv} hd={hd} ctx<={max_ctx} L<={q_len_max} causal={causal}")
    c = wl.random_case(7 * hq + hd + max_ctx + q_len_max, kind="prefill", dtype="bf16", num_seqs=4,
                       num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, max_ctx=max_ctx, q_len_max=q_len_max,
                       causal=causal, poison=True)
    err = new_err(dev, mode)
    kp, vp, rk, rv = quantised_pools(pkv, c, dev, err)
    rk, rv = write_new(pkv, c, dev, kp, vp, rk, rv, err)
    maxl = int(np.diff(c.cu_q_lens).max())
    out = pkv.paged_attn_prefill_chunk_fp8(to_dev(c.query, dev, True), to_dev(c.cu_q_lens, dev),
                                           to_dev(c.chunk_offsets, dev), kp, vp, to_dev(c.block_tables, dev), maxl,
                                           c.scale, K_SCALE, V_SCALE, causal=causal, err_flag=err)
    ref = oracle.prefill_chunk(c.query, c.cu_q_lens, c.chunk_offsets, ofp8.dequantize(rk, K_SCALE),
                               ofp8.dequantize(rv, V_SCALE), c.block_tables, c.scale, "bf16", causal=causal,
                               kv_dtype="f64")
    mx, mean = close(out.cpu().numpy(), ref, "fp8 prefill")
    _say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert flag(err) == 0


@pytest.mark.parametrize("mode", MODES)
def test_fp8_mixed_step_full_size(pkv, dev, mode):
    """The mixed-step workload at full size over E4M3 pools, in the configuration the benchmark
    runs (library-chosen split size, one workspace): the whole pools quantised by the library's
    write and compared byte for byte, then the decode of all 127 sequences and the 512-row chunk;
    every sequence and every row against the oracle over the dequantised pools."""
    _say("case fp8 mixed step: 127 decode sequences + 512-row chunk at 16,384, 64/8 x 128, E4M3 pools")
    dec, pre, _, _, _ = mixed_step_case()
    err = new_err(dev, mode)
    nblk, hkv, b, hd = pre.key_pool.shape
    kp = torch.empty((nblk, hkv, b, hd), dtype=torch.float8_e4m3fn, device=dev)
    vp = torch.empty_like(kp)
    pkv.cache_write_fp8(to_dev(wl.slot_rows(pre.key_pool), dev, True),
                        to_dev(wl.slot_rows(pre.value_pool), dev, True), kp, vp,
                        torch.arange(nblk * b, dtype=torch.int32, device=dev), K_SCALE, V_SCALE, err_flag=err)
    rk = ofp8.quantize_bf16_bits(pre.key_pool, K_SCALE)
    rv = ofp8.quantize_bf16_bits(pre.value_pool, V_SCALE)
    rk, rv = write_new(pkv, pre, dev, kp, vp, rk, rv, err)  # the chunk's tokens; whole pools compared
    d_out = pkv.paged_attn_decode_fp8(to_dev(dec.query, dev, True), kp, vp, to_dev(dec.block_tables, dev),
                                      to_dev(dec.context_lens, dev), dec.scale, K_SCALE, V_SCALE, err_flag=err)
    p_out = pkv.paged_attn_prefill_chunk_fp8(to_dev(pre.query, dev, True), to_dev(pre.cu_q_lens, dev),
                                             to_dev(pre.chunk_offsets, dev), kp, vp, to_dev(pre.block_tables, dev),
                                             int(np.diff(pre.cu_q_lens).max()), pre.scale, K_SCALE, V_SCALE,
                                             causal=True, err_flag=err)
    d_out, p_out = d_out.cpu().numpy(), p_out.cpu().numpy()
    assert flag(err) == 0
    ref = fp8_decode_reference(dec, rk, rv, K_SCALE, V_SCALE)
    mx, mean = close(d_out, ref, "fp8 mixed decode (all 127 sequences)")
    _say(f"  decode (all {dec.num_seqs} sequences) max-abs {mx:.2e} mean-abs {mean:.2e}")
    ref = fp8_prefill_reference(pre, rk, rv, K_SCALE, V_SCALE)
    mx, mean = close(p_out, ref, "fp8 mixed prefill (all 512 rows)")
    _say(f"  prefill (all {p_out.shape[0]} rows) max-abs {mx:.2e} mean-abs {mean:.2e}")
