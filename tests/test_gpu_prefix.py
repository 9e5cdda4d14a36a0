"""GPU tests of the shared-prefix decode (needs an MI355X).

pkv_paged_attn_decode_prefix attends the blocks its member sequences share ("第2章:推理引擎核心技术"
§1.5 and §3.2: sequences with a cached prefix map its logical blocks to the same physical blocks)
once per KV head and merges that partial with each member's own positions.  It computes what the
plain decode computes, so the bar is the oracle's tolerance (max-abs <= 1e-2, mean-abs <= 1e-3)
on every sequence, plus agreement with pkv_paged_attn_decode on the same inputs.  Cases: the mixed
step's 127 sequences (63 shared blocks; the members are the sequences that reach past them) and
the 64-sequence batch behind a 256-block shared prompt, both at full size; random batches in
which a subset shares a prefix, with a member that ends exactly at the prefix, members whose
rest spans several splits, non-members with empty contexts, and group sizes 1 to 16; and the
no-member call, which must equal the plain decode bit for bit.  Every test except the flag test
runs in both call modes (checked kernels with an err_flag, and the release kernels production
callers run, err_flag NULL).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_common import MODES, flag, new_err

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


def to_dev(a, dev, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if bf16 else t).to(dev)


def close(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, f"{what}: max-abs {d.max():.3e} mean-abs {d.mean():.3e}"
    return d.max(), d.mean()


@pytest.mark.parametrize("mode", MODES)
def test_mixed_step_decode_with_shared_prefix(pkv, mode):
    dev = torch.device("cuda:0")
    dec, _ = wl.mixed_step(poison=True)
    P = 63
    members = np.flatnonzero(dec.context_lens >= P * 16).astype(np.int32)
    _say(f"case prefix decode: mixed step, {len(members)} members of {dec.num_seqs} sharing {P} blocks")
    kp, vp = to_dev(dec.key_pool, dev, True), to_dev(dec.value_pool, dev, True)
    q, bt, ctx = to_dev(dec.query, dev, True), to_dev(dec.block_tables, dev), to_dev(dec.context_lens, dev)
    err = new_err(dev, mode)
    out = pkv.paged_attn_decode_prefix(q, kp, vp, bt, ctx, dec.scale, to_dev(members, dev), P, err_flag=err)
    plain = pkv.paged_attn_decode(q, kp, vp, bt, ctx, dec.scale, err_flag=err)
    torch.cuda.synchronize()
    assert flag(err) == 0
    ref = oracle.decode(dec.query, dec.key_pool, dec.value_pool, dec.block_tables, dec.context_lens, dec.scale, "bf16")
    mx, mean = close(out.cpu().numpy(), ref, "prefix decode vs oracle")
    _say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")
    d = (out - plain).abs()
    assert float(d.max()) <= 5e-3, f"prefix decode vs plain decode: max {float(d.max()):.3e}"


@pytest.mark.parametrize("mode", MODES)
def test_shared_prefix_workload_full_size(pkv, mode):
    """The 64-sequence, 256-shared-block decode batch timed by the benchmark, in its launch
    configuration, against the oracle on every sequence and against the plain decode."""
    dev = torch.device("cuda:0")
    dec = wl.shared_prefix_decode(poison=True)
    P = int(dec.notes["prefix_blocks"])
    _say(f"case prefix decode: shared-prefix workload, {dec.num_seqs} members, {P} blocks")
    kp, vp = to_dev(dec.key_pool, dev, True), to_dev(dec.value_pool, dev, True)
    q, bt, ctx = to_dev(dec.query, dev, True), to_dev(dec.block_tables, dev), to_dev(dec.context_lens, dev)
    err = new_err(dev, mode)
    ws = pkv.decode_prefix_workspace(q, dec.num_kv_heads, dec.max_blocks_per_seq)
    out = pkv.paged_attn_decode_prefix(q, kp, vp, bt, ctx, dec.scale, to_dev(dec.notes["members"], dev), P,
                                       workspace=ws, err_flag=err)
    plain = pkv.paged_attn_decode(q, kp, vp, bt, ctx, dec.scale, err_flag=err)
    torch.cuda.synchronize()
    assert flag(err) == 0
    ref = oracle.decode(dec.query, dec.key_pool, dec.value_pool, dec.block_tables, dec.context_lens, dec.scale, "bf16")
    mx, mean = close(out.cpu().numpy(), ref, "prefix decode vs oracle")
    _say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")
    d = (out - plain).abs()
    assert float(d.max()) <= 5e-3, f"prefix decode vs plain decode: max {float(d.max()):.3e}"


def shared_prefix_case(seed, hq, hkv, hd, P, num_seqs, member_ctx, other_ctx):
    """A random decode case whose members (the first len(member_ctx) sequences, in shuffled order)
    share P leading blocks; the others have private blocks only."""
    rng = np.random.default_rng(seed)
    ctx = np.array(list(member_ctx) + list(other_ctx), np.int32)
    assert len(ctx) == num_seqs
    order = rng.permutation(num_seqs)
    ctx = ctx[order]
    is_member = np.zeros(num_seqs, bool)
    is_member[np.argsort(order)[:len(member_ctx)]] = True
    members = np.flatnonzero(is_member).astype(np.int32)
    need = [-(-int(c) // 16) for c in ctx]
    private = [n - P if m else n for n, m in zip(need, is_member)]
    nblk = P + sum(private) + 4
    free = rng.permutation(nblk).astype(np.int32)
    shared = free[:P]
    width = max(need) + 1
    bt = np.full((num_seqs, width), wl.UNUSED_BLOCK_ID, np.int32)
    cursor = P
    for s in range(num_seqs):
        row = []
        if is_member[s]:
            row += list(shared)
        row += list(free[cursor:cursor + private[s]])
        cursor += private[s]
        bt[s, :len(row)] = row
    f32 = lambda shape: wl.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    kpool, vpool = f32((nblk, hkv, 16, hd)), f32((nblk, hkv, 16, hd))
    q = f32((num_seqs, hq, hd))
    # NaN in every slot no sequence may read: the tails of last blocks and the spare blocks.
    nan = np.uint16(0x7FC0)
    used = set()
    for s in range(num_seqs):
        nb = need[s]
        used.update(int(b) for b in bt[s, :nb])
        tail = int(ctx[s]) % 16
        if tail:
            b = bt[s, nb - 1]
            kpool[b, :, tail:] = nan
            vpool[b, :, tail:] = nan
    for b in range(nblk):
        if b not in used:
            kpool[b] = nan
            vpool[b] = nan
    return q, kpool, vpool, bt, ctx, members


PREFIX_CASES = [
    # (hq, hkv, hd, P, member contexts, other contexts, split_tokens)
    (64, 8, 128, 20, [320, 321, 900, 2100, 5000], [0, 17, 700], 0),
    (16, 2, 128, 9, [144, 160, 400, 1000], [1, 300], 128),
    (8, 8, 64, 5, [80, 81, 95, 640], [0, 50], 0),
    (16, 1, 128, 40, [640 + 3 * i for i in range(20)], [10, 2000], 256),
    (32, 2, 64, 3, [48, 48, 60, 800, 1500], [], 128),
]


@pytest.mark.parametrize("hq,hkv,hd,P,mctx,octx,split", PREFIX_CASES)
@pytest.mark.parametrize("mode", MODES)
def test_shared_prefix_random(pkv, mode, hq, hkv, hd, P, mctx, octx, split):
    dev = torch.device("cuda:0")
    _say(f"case prefix decode: hq={hq} hkv={hkv} hd={hd} P={P} members={len(mctx)} others={len(octx)} "
         f"split={split}")
    n = len(mctx) + len(octx)
    q, kpool, vpool, bt, ctx, members = shared_prefix_case(hq * 7 + hd + P, hq, hkv, hd, P, n, mctx, octx)
    kp, vp = to_dev(kpool, dev, True), to_dev(vpool, dev, True)
    qd, btd, ctxd = to_dev(q, dev, True), to_dev(bt, dev), to_dev(ctx, dev)
    err = new_err(dev, mode)
    scale = hd ** -0.5
    out = pkv.paged_attn_decode_prefix(qd, kp, vp, btd, ctxd, scale, to_dev(members, dev), P, split_tokens=split,
                                       err_flag=err)
    torch.cuda.synchronize()
    assert flag(err) == 0
    ref = oracle.decode(q, kpool, vpool, bt, ctx, scale, "bf16")
    mx, mean = close(out.cpu().numpy(), ref, "prefix decode vs oracle")
    _say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")
    # bf16 output as well.
    out16 = pkv.paged_attn_decode_prefix(qd, kp, vp, btd, ctxd, scale, to_dev(members, dev), P, split_tokens=split,
                                         out_dtype=torch.bfloat16, err_flag=err)
    d = (out16.float() - out).abs()
    assert float(d.max()) <= 2.0 ** -7 * max(1.0, float(out.abs().max()))
    assert flag(err) == 0


@pytest.mark.parametrize("mode", MODES)
def test_no_members_is_the_plain_decode(pkv, mode):
    dev = torch.device("cuda:0")
    _say("case prefix decode: no members")
    c = wl.random_case(77, kind="decode", dtype="bf16", num_seqs=7, num_q_heads=16, num_kv_heads=4, head_dim=128,
                       max_ctx=3000, min_ctx=0, new_tokens=False, poison=True)
    kp, vp = to_dev(c.key_pool, dev, True), to_dev(c.value_pool, dev, True)
    q, bt, ctx = to_dev(c.query, dev, True), to_dev(c.block_tables, dev), to_dev(c.context_lens, dev)
    none = torch.zeros(0, dtype=torch.int32, device=dev)
    err = new_err(dev, mode)
    a = pkv.paged_attn_decode_prefix(q, kp, vp, bt, ctx, c.scale, none, 5, err_flag=err)
    b = pkv.paged_attn_decode(q, kp, vp, bt, ctx, c.scale, err_flag=err)
    torch.cuda.synchronize()
    assert flag(err) == 0
    assert torch.equal(a, b)
    close(a.cpu().numpy(), oracle.decode(c.query, c.key_pool, c.value_pool, c.block_tables, c.context_lens, c.scale,
                                         "bf16"), "decode vs oracle")


def test_bad_member_index_is_flagged_and_skipped(pkv):
    """A member index outside [0, num_seqs) (not the first) sets the bad-length flag in checked
    mode and is skipped; every sequence's output is still the oracle's."""
    dev = torch.device("cuda:0")
    hq, hkv, hd, P = 16, 2, 128, 9
    _say("case prefix decode: an out-of-range member index")
    q, kpool, vpool, bt, ctx, members = shared_prefix_case(99, hq, hkv, hd, P, 6, [144, 400, 1000], [0, 300, 37])
    bad = np.concatenate([members, np.array([6 + 5], np.int32)])
    kp, vp = to_dev(kpool, dev, True), to_dev(vpool, dev, True)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    scale = hd ** -0.5
    out = pkv.paged_attn_decode_prefix(to_dev(q, dev, True), kp, vp, to_dev(bt, dev), to_dev(ctx, dev), scale,
                                       to_dev(bad, dev), P, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) & pkv.FLAG_BAD_LENGTH
    close(out.cpu().numpy(), oracle.decode(q, kpool, vpool, bt, ctx, scale, "bf16"), "prefix decode vs oracle")


@pytest.mark.parametrize("hq,hkv,hd,P,mctx,octx,split", [PREFIX_CASES[0], PREFIX_CASES[2], PREFIX_CASES[3]])
@pytest.mark.parametrize("mode", MODES)
def test_shared_prefix_fp8_pools(pkv, mode, hq, hkv, hd, P, mctx, octx, split):
    """E4M3 pools (quantised by the library's own write): the shared-prefix decode against the oracle
    over the dequantised pools and against the plain FP8 decode."""
    from oracle import fp8 as ofp8
    dev = torch.device("cuda:0")
    _say(f"case prefix decode fp8: hq={hq} hkv={hkv} hd={hd} P={P} members={len(mctx)} others={len(octx)}")
    n = len(mctx) + len(octx)
    q, kpool, vpool, bt, ctx, members = shared_prefix_case(hq * 5 + hd + P, hq, hkv, hd, P, n, mctx, octx)
    ks, vs = 2.0 ** -5, 0.0123
    nblk = kpool.shape[0]
    kp = torch.empty(kpool.shape, dtype=torch.float8_e4m3fn, device=dev)
    vp = torch.empty_like(kp)
    pkv.cache_write_fp8(to_dev(wl.slot_rows(kpool), dev, True), to_dev(wl.slot_rows(vpool), dev, True), kp, vp,
                        torch.arange(nblk * 16, dtype=torch.int32, device=dev), ks, vs)
    err = new_err(dev, mode)
    qd, btd, ctxd = to_dev(q, dev, True), to_dev(bt, dev), to_dev(ctx, dev)
    scale = hd ** -0.5
    out = pkv.paged_attn_decode_prefix_fp8(qd, kp, vp, btd, ctxd, scale, ks, vs, to_dev(members, dev), P,
                                           split_tokens=split, err_flag=err)
    plain = pkv.paged_attn_decode_fp8(qd, kp, vp, btd, ctxd, scale, ks, vs, split_tokens=split, err_flag=err)
    torch.cuda.synchronize()
    assert flag(err) == 0
    rk = ofp8.dequantize(ofp8.quantize_bf16_bits(kpool, ks), ks)
    rv = ofp8.dequantize(ofp8.quantize_bf16_bits(vpool, vs), vs)
    mx, mean = close(out.cpu().numpy(), oracle.decode(q, rk, rv, bt, ctx, scale, "bf16", kv_dtype="f64"),
                     "fp8 prefix decode vs oracle")
    _say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert float((out - plain).abs().max()) <= 5e-3
