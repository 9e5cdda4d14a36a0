"""GPU tests of the fused mixed-batch launch (needs an MI355X).

The fused call runs the decode and prefill device code of the separate calls in one launch, so the
bar is bit-identity with pkv_paged_attn_decode + pkv_paged_attn_prefill_chunk on the same inputs
(bf16 and FP8 pools), plus the usual oracle tolerance (max-abs <= 1e-2, mean-abs <= 1e-3) on the
fused outputs.  Cases: the 127-sequence mixed step with its 512-row chunk, small random batches
with both parts over one pool, and each part alone.  Every test runs in both call modes (checked
kernels with an err_flag, and the release kernels production callers run, err_flag NULL).
"""
import sys

import numpy as np
import pytest

import oracle
from oracle import fp8 as ofp8
import workloads as wl
from gpu_common import MODES, flag, mixed_step_case, mixed_step_reference, new_err

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3


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


def close(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, f"{what}: max-abs {d.max():.3e} mean-abs {d.mean():.3e}"
    return float(d.max()), float(d.mean())


def run_both(pkv, kp, vp, scale, dq, dbt, dctx, pq, cu, offs, pbt, maxl, causal=True, fp8=None, err=None):
    """(separate decode, separate prefill, fused decode, fused prefill) outputs on the host."""
    ks, vs = fp8 if fp8 else (1.0, 1.0)
    sep_d = sep_p = None
    if dq is not None:
        if fp8:
            sep_d = pkv.paged_attn_decode_fp8(dq, kp, vp, dbt, dctx, scale, ks, vs, err_flag=err)
        else:
            sep_d = pkv.paged_attn_decode(dq, kp, vp, dbt, dctx, scale, err_flag=err)
    if pq is not None:
        if fp8:
            sep_p = pkv.paged_attn_prefill_chunk_fp8(pq, cu, offs, kp, vp, pbt, maxl, scale, ks, vs, causal=causal,
                                                     err_flag=err)
        else:
            sep_p = pkv.paged_attn_prefill_chunk(pq, cu, offs, kp, vp, pbt, maxl, scale, causal=causal, err_flag=err)
    fd, fp = pkv.paged_attn_mixed(kp, vp, scale, dec_query=dq, dec_block_tables=dbt, context_lens=dctx,
                                  pre_query=pq, cu_q_lens=cu, chunk_offsets=offs, pre_block_tables=pbt, max_q_len=maxl,
                                  causal=causal, k_scale=ks, v_scale=vs, err_flag=err)
    host = lambda t: None if t is None else t.cpu().numpy()
    return host(sep_d), host(sep_p), host(fd), host(fp)


@pytest.mark.parametrize("mode", MODES)
def test_fused_mixed_step_bit_identical(pkv, dev, mode):
    """The mixed-step workload: 127 decode sequences (shared 63-block prefix) and a 512-row chunk at
    offset 16,384 of a 32,768-token prompt, after the chunk's cache write."""
    _say("case fused mixed step: 127 decode sequences + 512-row chunk, 64/8 x 128, bf16")
    dec, pre, ref_slots, _, _ = mixed_step_case()
    kp, vp = to_dev(dec.key_pool, dev, True), to_dev(dec.value_pool, dev, True)
    err = new_err(dev, mode)
    T = pre.num_new_tokens
    slots = pkv.slot_mapping(to_dev(pre.block_tables, dev), to_dev(pre.new_cu_lens, dev), to_dev(pre.new_start_pos, dev),
                             T, pre.num_blocks, err_flag=err, total=T)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    pkv.cache_write(to_dev(pre.key_new, dev, True), to_dev(pre.value_new, dev, True), kp, vp, slots, err_flag=err)
    args = (to_dev(dec.query, dev, True), to_dev(dec.block_tables, dev), to_dev(dec.context_lens, dev),
            to_dev(pre.query, dev, True), to_dev(pre.cu_q_lens, dev), to_dev(pre.chunk_offsets, dev),
            to_dev(pre.block_tables, dev), int(np.diff(pre.cu_q_lens).max()))
    sd, sp, fd, fp = run_both(pkv, kp, vp, dec.scale, *args, err=err)
    assert fd.tobytes() == sd.tobytes(), "fused decode differs from the decode call"
    assert fp.tobytes() == sp.tobytes(), "fused prefill differs from the prefill call"
    assert flag(err) == 0
    # The fused outputs against the oracle: every decode sequence and every chunk row.
    ref_d, ref_p = mixed_step_reference()
    mx, mean = close(fd, ref_d, "fused decode vs oracle (all 127 sequences)")
    _say(f"  decode max-abs {mx:.2e} mean-abs {mean:.2e}")
    mx, mean = close(fp, ref_p, "fused prefill vs oracle (all 512 rows)")
    _say(f"  prefill max-abs {mx:.2e} mean-abs {mean:.2e}")


MIXED_CASES = [
    # (hq, hkv, hd, max_ctx, q_len_max, fp8)
    (16, 2, 128, 900, 300, False),
    (8, 8, 64, 400, 150, False),
    (64, 8, 128, 1500, 200, True),
    (32, 4, 64, 700, 129, True),
]


@pytest.mark.parametrize("hq,hkv,hd,max_ctx,q_len_max,fp8", MIXED_CASES)
@pytest.mark.parametrize("mode", MODES)
def test_fused_random_batches(pkv, dev, mode, hq, hkv, hd, max_ctx, q_len_max, fp8):
    """Both parts over one pool: the prefill sequences' chunks, and one decode token per sequence
    at the end of each sequence's cached range; also each part alone."""
    _say(f"case fused random: hq={hq} hkv={hkv} hd={hd} ctx<={max_ctx} L<={q_len_max} fp8={fp8}")
    c = wl.random_case(hq + 11 * hd + max_ctx + q_len_max, kind="prefill", dtype="bf16", num_seqs=6, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=hd, max_ctx=max_ctx, q_len_max=q_len_max, causal=True, poison=True)
    err = new_err(dev, mode)
    kp, vp = to_dev(c.key_pool, dev, True), to_dev(c.value_pool, dev, True)
    maxl = int(np.diff(c.cu_q_lens).max())
    slots = pkv.slot_mapping(to_dev(c.block_tables, dev), to_dev(c.new_cu_lens, dev), to_dev(c.new_start_pos, dev),
                             maxl, c.num_blocks, err_flag=err, total=c.num_new_tokens)
    pkv.cache_write(to_dev(c.key_new, dev, True), to_dev(c.value_new, dev, True), kp, vp, slots, err_flag=err)
    rk, rv = oracle.cache_write(c.key_pool, c.value_pool, c.key_new, c.value_new,
                                oracle.slot_mapping(c.block_tables, c.new_cu_lens, c.new_start_pos, 16))
    scales = None
    kv_dtype = "bf16"
    if fp8:
        scales = (0.0123, 2.0 ** -5)
        n = c.num_blocks * 16
        kp8 = torch.empty(kp.shape, dtype=torch.float8_e4m3fn, device=dev)
        vp8 = torch.empty_like(kp8)
        # Every slot's token row (the pools are [blocks, Hkv, 16, hd]) through the quantising write.
        pkv.cache_write_fp8(kp.permute(0, 2, 1, 3).reshape(n, hkv, hd), vp.permute(0, 2, 1, 3).reshape(n, hkv, hd),
                            kp8, vp8,
                            torch.arange(n, dtype=torch.int32, device=dev), *scales, err_flag=err)
        kp, vp = kp8, vp8
        rk = ofp8.dequantize(ofp8.quantize_bf16_bits(rk, scales[0]), scales[0])
        rv = ofp8.dequantize(ofp8.quantize_bf16_bits(rv, scales[1]), scales[1])
        kv_dtype = "f64"
    ctx = (c.chunk_offsets + np.diff(c.cu_q_lens)).astype(np.int32)
    rng = np.random.default_rng(hq + hd)
    dq_host = wl.f32_to_bf16_bits(rng.standard_normal((6, hq, hd)).astype(np.float32))
    dq, dbt, dctx = to_dev(dq_host, dev, True), to_dev(c.block_tables, dev), to_dev(ctx, dev)
    pq, cu, offs, pbt = (to_dev(c.query, dev, True), to_dev(c.cu_q_lens, dev), to_dev(c.chunk_offsets, dev),
                         to_dev(c.block_tables, dev))
    for parts in ("both", "decode", "prefill"):
        d_args = (dq, dbt, dctx) if parts != "prefill" else (None, None, None)
        p_args = (pq, cu, offs, pbt, maxl) if parts != "decode" else (None, None, None, None, 0)
        sd, sp, fd, fp = run_both(pkv, kp, vp, c.scale, *d_args, *p_args, fp8=scales, err=err)
        if parts != "prefill":
            assert fd.tobytes() == sd.tobytes(), f"fused decode differs ({parts})"
        else:
            assert fd is None
        if parts != "decode":
            assert fp.tobytes() == sp.tobytes(), f"fused prefill differs ({parts})"
        else:
            assert fp is None
    ref_d = oracle.decode(dq_host, rk, rv, c.block_tables, ctx, c.scale, "bf16", kv_dtype=kv_dtype)
    ref_p = oracle.prefill_chunk(c.query, c.cu_q_lens, c.chunk_offsets, rk, rv, c.block_tables, c.scale, "bf16",
                                 kv_dtype=kv_dtype)
    _, _, fd, fp = run_both(pkv, kp, vp, c.scale, dq, dbt, dctx, pq, cu, offs, pbt, maxl, fp8=scales, err=err)
    close(fd, ref_d, "fused decode vs oracle")
    close(fp, ref_p, "fused prefill vs oracle")
    assert flag(err) == 0
