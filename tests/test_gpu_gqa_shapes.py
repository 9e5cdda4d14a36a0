"""GPU parity over model-shaped GQA layouts (needs an MI355X).

The other sweeps use power-of-two head groups.  Served models also put 3, 5, 6, 7 or 12 query
heads on each KV head, over odd KV head counts (40 query heads over 8 KV heads, 28 over 4, ...).
Each layout below runs through the decode (automatic and 128-position splits), the prefill chunk
(causal and not) and, at head_dim <= 128, the fused launch (bit-identical to the two separate
calls), over bf16 and E4M3 pools, against the oracle at the bf16-input tolerance (max-abs <= 1e-2,
mean-abs <= 1e-3).  Pool writes are compared byte for byte with the oracle's.  Inputs carry
NaN-poisoned dead slots.  Every test runs in both call modes (checked kernels with an err_flag,
and the release kernels production callers run).
"""
import sys

import numpy as np
import pytest

import oracle
from oracle import fp8 as ofp8
import workloads as wl
from gpu_common import MODES, close, flag, new_err, to_dev

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 0.0123, 2.0 ** -5

GQA_SHAPES = [
    # (query heads, KV heads, head_dim)
    (12, 4, 128),   # groups of 3
    (40, 8, 128),   # groups of 5
    (28, 4, 128),   # groups of 7
    (18, 3, 64),    # groups of 6 over three KV heads
    (60, 5, 64),    # groups of 12 over five KV heads
    (14, 2, 256),   # groups of 7
    (10, 5, 256),   # groups of 2 over five KV heads
    (48, 3, 128),   # groups of 16 (the largest) over three KV heads
]
POOLS = ("bf16", "fp8")


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


def _codes(t):
    return t.cpu().view(torch.uint8).numpy()


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


class Pools:
    """A case's pools on the device (bf16, or E4M3 codes of the bf16 pools written by the
    quantising write), with the oracle's copies: `rk` / `rv` hold bf16 bits or E4M3 codes, and
    `ref()` gives what the oracle attends over."""

    def __init__(self, pkv, c, dev, pool, err):
        self.pkv, self.c, self.dev, self.pool, self.err = pkv, c, dev, pool, err
        self.bt = to_dev(c.block_tables, dev)
        if pool == "bf16":
            self.kp, self.vp = to_dev(c.key_pool, dev, True), to_dev(c.value_pool, dev, True)
            self.rk, self.rv = c.key_pool, c.value_pool
            return
        nblk, hkv, b, hd = c.key_pool.shape
        self.kp = torch.zeros((nblk, hkv, b, hd), dtype=torch.float8_e4m3fn, device=dev)
        self.vp = torch.zeros_like(self.kp)
        slots = torch.arange(nblk * b, dtype=torch.int32, device=dev)
        pkv.cache_write_fp8(to_dev(wl.slot_rows(c.key_pool), dev, True), to_dev(wl.slot_rows(c.value_pool), dev, True),
                            self.kp, self.vp, slots, K_SCALE, V_SCALE, err_flag=err)
        self.rk = ofp8.quantize_bf16_bits(c.key_pool, K_SCALE)
        self.rv = ofp8.quantize_bf16_bits(c.value_pool, V_SCALE)
        self.check()

    def check(self):
        if self.pool == "bf16":
            assert _bits(self.kp).tobytes() == self.rk.tobytes(), "K pool differs from the oracle's"
            assert _bits(self.vp).tobytes() == self.rv.tobytes(), "V pool differs from the oracle's"
        else:
            assert _codes(self.kp).tobytes() == self.rk.tobytes(), "K codes differ from the oracle's"
            assert _codes(self.vp).tobytes() == self.rv.tobytes(), "V codes differ from the oracle's"

    def write_new(self):
        """Slot-map and write the case's new tokens on both sides; the pools must stay identical."""
        c, dev, err = self.c, self.dev, self.err
        T = c.num_new_tokens
        if T == 0:
            return
        maxlen = int(np.diff(c.new_cu_lens).max())
        slots = self.pkv.slot_mapping(self.bt, to_dev(c.new_cu_lens, dev), to_dev(c.new_start_pos, dev), maxlen,
                                      c.num_blocks, err_flag=err, total=T)
        ref_slots = oracle.slot_mapping(c.block_tables, c.new_cu_lens, c.new_start_pos, 16)
        assert np.array_equal(slots.cpu().numpy(), ref_slots), "slot mapping differs from the oracle"
        kn, vn = to_dev(c.key_new, dev, True), to_dev(c.value_new, dev, True)
        if self.pool == "bf16":
            self.pkv.cache_write(kn, vn, self.kp, self.vp, slots, err_flag=err)
            self.rk, self.rv = oracle.cache_write(self.rk, self.rv, c.key_new, c.value_new, ref_slots)
        else:
            self.pkv.cache_write_fp8(kn, vn, self.kp, self.vp, slots, K_SCALE, V_SCALE, err_flag=err)
            f32 = lambda b: oracle.as_f64(b, "bf16").astype(np.float32)
            self.rk, self.rv = ofp8.cache_write_fp8(self.rk, self.rv, f32(c.key_new), f32(c.value_new), ref_slots,
                                                    K_SCALE, V_SCALE)
        self.check()

    def ref(self):
        """(K pool, V pool, kv dtype) as the oracle reads them."""
        if self.pool == "bf16":
            return self.rk, self.rv, "bf16"
        return ofp8.dequantize(self.rk, K_SCALE), ofp8.dequantize(self.rv, V_SCALE), "f64"

    def decode(self, q, ctx, scale, **kw):
        if self.pool == "bf16":
            return self.pkv.paged_attn_decode(q, self.kp, self.vp, self.bt, ctx, scale, err_flag=self.err, **kw)
        return self.pkv.paged_attn_decode_fp8(q, self.kp, self.vp, self.bt, ctx, scale, K_SCALE, V_SCALE,
                                              err_flag=self.err, **kw)

    def prefill(self, q, cu, offs, maxl, scale, causal):
        if self.pool == "bf16":
            return self.pkv.paged_attn_prefill_chunk(q, cu, offs, self.kp, self.vp, self.bt, maxl, scale,
                                                     causal=causal, err_flag=self.err)
        return self.pkv.paged_attn_prefill_chunk_fp8(q, cu, offs, self.kp, self.vp, self.bt, maxl, scale, K_SCALE,
                                                     V_SCALE, causal=causal, err_flag=self.err)


def _seed(hq, hkv, hd, k):
    return hq * 7919 + hkv * 104729 + hd * 13 + k


@pytest.mark.parametrize("pool", POOLS)
@pytest.mark.parametrize("hq,hkv,hd", GQA_SHAPES)
@pytest.mark.parametrize("mode", MODES)
def test_decode_gqa_shapes(pkv, dev, mode, hq, hkv, hd, pool):
    _say(f"case gqa-shape decode: hq={hq} hkv={hkv} hd={hd} pool={pool} ({mode})")
    c = wl.random_case(_seed(hq, hkv, hd, 1), kind="decode", dtype="bf16", num_seqs=6, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=hd, max_ctx=700, min_ctx=0, poison=True)
    err = new_err(dev, mode)
    p = Pools(pkv, c, dev, pool, err)
    p.write_new()
    rk, rv, kvd = p.ref()
    ref = oracle.decode(c.query, rk, rv, c.block_tables, c.context_lens, c.scale, "bf16", kv_dtype=kvd)
    q, ctx = to_dev(c.query, dev, True), to_dev(c.context_lens, dev)
    for split in (0, 128):
        out = p.decode(q, ctx, c.scale, split_tokens=split).cpu().numpy()
        mx, mean = close(out, ref, f"decode split={split}")
        assert (out[c.context_lens == 0] == 0).all()
    _say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert flag(err) == 0


@pytest.mark.parametrize("pool", POOLS)
@pytest.mark.parametrize("hq,hkv,hd", GQA_SHAPES)
@pytest.mark.parametrize("mode", MODES)
def test_prefill_gqa_shapes(pkv, dev, mode, hq, hkv, hd, pool):
    _say(f"case gqa-shape prefill: hq={hq} hkv={hkv} hd={hd} pool={pool} ({mode})")
    c = wl.random_case(_seed(hq, hkv, hd, 2), kind="prefill", dtype="bf16", num_seqs=4, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=hd, max_ctx=600, q_len_max=170, poison=True)
    err = new_err(dev, mode)
    p = Pools(pkv, c, dev, pool, err)
    p.write_new()
    rk, rv, kvd = p.ref()
    maxl = int(np.diff(c.cu_q_lens).max())
    q, cu, offs = to_dev(c.query, dev, True), to_dev(c.cu_q_lens, dev), to_dev(c.chunk_offsets, dev)
    for causal in (True, False):
        out = p.prefill(q, cu, offs, maxl, c.scale, causal).cpu().numpy()
        ref = oracle.prefill_chunk(c.query, c.cu_q_lens, c.chunk_offsets, rk, rv, c.block_tables, c.scale, "bf16",
                                   causal=causal, kv_dtype=kvd)
        mx, mean = close(out, ref, f"prefill causal={causal}")
        _say(f"  causal={causal}: max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert flag(err) == 0


@pytest.mark.parametrize("pool", POOLS)
@pytest.mark.parametrize("hq,hkv,hd", [s for s in GQA_SHAPES if s[2] <= 128])
@pytest.mark.parametrize("mode", MODES)
def test_fused_gqa_shapes(pkv, dev, mode, hq, hkv, hd, pool):
    """The fused launch over one pool: the prefill sequences' chunks, and one decode token per
    sequence at the end of its cached range."""
    _say(f"case gqa-shape fused: hq={hq} hkv={hkv} hd={hd} pool={pool} ({mode})")
    c = wl.random_case(_seed(hq, hkv, hd, 3), kind="prefill", dtype="bf16", num_seqs=5, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=hd, max_ctx=800, q_len_max=150, poison=True)
    err = new_err(dev, mode)
    p = Pools(pkv, c, dev, pool, err)
    p.write_new()
    rk, rv, kvd = p.ref()
    maxl = int(np.diff(c.cu_q_lens).max())
    ctx_h = (c.chunk_offsets + np.diff(c.cu_q_lens)).astype(np.int32)
    rng = np.random.default_rng(_seed(hq, hkv, hd, 4))
    dq_h = wl.f32_to_bf16_bits(rng.standard_normal((c.chunk_offsets.shape[0], hq, hd)).astype(np.float32))
    dq, ctx = to_dev(dq_h, dev, True), to_dev(ctx_h, dev)
    pq, cu, offs = to_dev(c.query, dev, True), to_dev(c.cu_q_lens, dev), to_dev(c.chunk_offsets, dev)
    sd = p.decode(dq, ctx, c.scale).cpu().numpy()
    sp = p.prefill(pq, cu, offs, maxl, c.scale, True).cpu().numpy()
    scales = (K_SCALE, V_SCALE) if pool == "fp8" else (1.0, 1.0)
    fd, fp = pkv.paged_attn_mixed(p.kp, p.vp, c.scale, dec_query=dq, dec_block_tables=p.bt, context_lens=ctx,
                                  pre_query=pq, cu_q_lens=cu, chunk_offsets=offs, pre_block_tables=p.bt,
                                  max_q_len=maxl, causal=True, k_scale=scales[0], v_scale=scales[1], err_flag=err)
    fd, fp = fd.cpu().numpy(), fp.cpu().numpy()
    assert fd.tobytes() == sd.tobytes(), "fused decode differs from the decode call"
    assert fp.tobytes() == sp.tobytes(), "fused prefill differs from the prefill call"
    close(fd, oracle.decode(dq_h, rk, rv, c.block_tables, ctx_h, c.scale, "bf16", kv_dtype=kvd), "fused decode")
    close(fp, oracle.prefill_chunk(c.query, c.cu_q_lens, c.chunk_offsets, rk, rv, c.block_tables, c.scale, "bf16",
                                   kv_dtype=kvd), "fused prefill")
    assert flag(err) == 0
