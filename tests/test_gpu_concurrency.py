"""Calls from several host threads, each on its own stream, at the same time (needs an MI355X).

The library keeps no state between calls and every call only enqueues kernels on its stream, so
calls with their own workspaces may run concurrently: two persistent decode grids and a prefill
launch then share the device.  Three threads (a bf16 decode, an E4M3 decode and a prefill chunk)
each issue their call many times on a stream of their own; every output must be bit-identical to
the same call run alone, and (checked mode) no flag may be raised.  Streams keep the default
priority.
"""
import sys
import threading

import numpy as np
import pytest

import oracle
from oracle import fp8 as ofp8
import workloads as wl
from gpu_common import MODES, close, flag, new_err, to_dev

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 0.0123, 2.0 ** -5
REPS = 12


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


def _jobs(pkv, dev, err):
    """Three independent calls with their inputs on the device: (name, call(out), output shape,
    dtype, oracle result)."""
    jobs = []
    # bf16 decode, GQA 64/8 x 128, contexts long enough for several splits.
    c = wl.random_case(4101, kind="decode", dtype="bf16", num_seqs=24, num_q_heads=64, num_kv_heads=8,
                       head_dim=128, max_ctx=3000, min_ctx=1, poison=True, new_tokens=False)
    q, kp, vp = to_dev(c.query, dev, True), to_dev(c.key_pool, dev, True), to_dev(c.value_pool, dev, True)
    bt, ctx = to_dev(c.block_tables, dev), to_dev(c.context_lens, dev)
    ws = pkv.decode_workspace(q, c.num_kv_heads, c.max_blocks_per_seq)
    ref = oracle.decode(c.query, c.key_pool, c.value_pool, c.block_tables, c.context_lens, c.scale, "bf16")
    jobs.append(("bf16 decode", lambda out, c=c, q=q, kp=kp, vp=vp, bt=bt, ctx=ctx, ws=ws:
                 pkv.paged_attn_decode(q, kp, vp, bt, ctx, c.scale, out=out, workspace=ws, err_flag=err),
                 tuple(q.shape), ref))
    # E4M3 decode, 16/4 x 256.
    c8 = wl.random_case(4102, kind="decode", dtype="bf16", num_seqs=10, num_q_heads=16, num_kv_heads=4,
                        head_dim=256, max_ctx=2500, min_ctx=1, poison=True, new_tokens=False)
    n = c8.num_blocks * 16
    kp8 = torch.zeros(c8.key_pool.shape, dtype=torch.float8_e4m3fn, device=dev)
    vp8 = torch.zeros_like(kp8)
    pkv.cache_write_fp8(to_dev(wl.slot_rows(c8.key_pool), dev, True), to_dev(wl.slot_rows(c8.value_pool), dev, True),
                        kp8, vp8, torch.arange(n, dtype=torch.int32, device=dev), K_SCALE, V_SCALE, err_flag=err)
    rk = ofp8.dequantize(ofp8.quantize_bf16_bits(c8.key_pool, K_SCALE), K_SCALE)
    rv = ofp8.dequantize(ofp8.quantize_bf16_bits(c8.value_pool, V_SCALE), V_SCALE)
    q8, bt8, ctx8 = to_dev(c8.query, dev, True), to_dev(c8.block_tables, dev), to_dev(c8.context_lens, dev)
    ws8 = pkv.decode_workspace(q8, c8.num_kv_heads, c8.max_blocks_per_seq)
    ref8 = oracle.decode(c8.query, rk, rv, c8.block_tables, c8.context_lens, c8.scale, "bf16", kv_dtype="f64")
    jobs.append(("E4M3 decode", lambda out, c=c8, q=q8, bt=bt8, ctx=ctx8, ws=ws8:
                 pkv.paged_attn_decode_fp8(q, kp8, vp8, bt, ctx, c.scale, K_SCALE, V_SCALE, out=out, workspace=ws,
                                           err_flag=err),
                 tuple(q8.shape), ref8))
    # bf16 prefill chunks of four sequences, 32/4 x 128, with key splits.
    cp = wl.random_case(4103, kind="prefill", dtype="bf16", num_seqs=4, num_q_heads=32, num_kv_heads=4,
                        head_dim=128, max_ctx=2200, q_len_max=300, poison=True, new_tokens=False)
    pq, pkp, pvp = to_dev(cp.query, dev, True), to_dev(cp.key_pool, dev, True), to_dev(cp.value_pool, dev, True)
    cu, off, pbt = to_dev(cp.cu_q_lens, dev), to_dev(cp.chunk_offsets, dev), to_dev(cp.block_tables, dev)
    maxl = int(np.diff(cp.cu_q_lens).max())
    pws = pkv.prefill_workspace(pq, 4, maxl, cp.max_blocks_per_seq)
    refp = oracle.prefill_chunk(cp.query, cp.cu_q_lens, cp.chunk_offsets, cp.key_pool, cp.value_pool,
                                cp.block_tables, cp.scale, "bf16")
    jobs.append(("prefill chunk", lambda out, c=cp: pkv.paged_attn_prefill_chunk(
        pq, cu, off, pkp, pvp, pbt, maxl, c.scale, causal=True, out=out, workspace=pws, err_flag=err),
        tuple(pq.shape), refp))
    return jobs


@pytest.mark.parametrize("mode", MODES)
def test_calls_on_concurrent_streams_are_bit_identical(pkv, dev, mode):
    _say(f"case concurrency ({mode}): bf16 decode, E4M3 decode and prefill chunk from three threads, "
         f"{REPS} calls each")
    err = new_err(dev, mode)
    jobs = _jobs(pkv, dev, err)
    # Each call alone, on the default stream.
    alone = []
    for name, call, shape, ref in jobs:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
        call(out)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        close(o, ref, f"{name} alone")
        alone.append(o)
    # All three at once, each from its own thread on its own stream.
    outs = [[torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(REPS)] for _, _, shape, _ in jobs]
    streams = [torch.cuda.Stream(device=dev) for _ in jobs]
    torch.cuda.synchronize()
    failures = []

    def run(k):
        try:
            with torch.cuda.stream(streams[k]):
                for r in range(REPS):
                    jobs[k][1](outs[k][r])
            streams[k].synchronize()
        except Exception as e:  # reported on the main thread
            failures.append(f"{jobs[k][0]}: {e!r}")

    threads = [threading.Thread(target=run, args=(k,)) for k in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert not failures, failures
    for k, (name, _, _, _) in enumerate(jobs):
        for r in range(REPS):
            assert outs[k][r].cpu().numpy().tobytes() == alone[k].tobytes(), f"{name}: call {r} differs"
    assert flag(err) == 0
