"""The mixed step captured in a HIP graph (needs an MI355X).

Every launch of the library is a kernel on the caller's stream, with no allocation, host
synchronisation or memset inside the calls, so a serving loop can capture a whole step (slot
mapping, cache write, decode, prefill chunk) once and replay it; the decode that allocates
nothing (static scratch) is meant for exactly that.  The test captures the step twice (decode
with a caller workspace, and the no-alloc decode), then replays each graph three times with new
queries and new K/V copied into the captured buffers between replays (eager work and a
synchronisation in between), and requires every replay to equal, bit for bit, the same step run
eagerly on the same inputs; the first replay is also checked against the oracle.
"""
import sys

import numpy as np
import pytest

import workloads as wl
from gpu_common import close, mixed_step_case, mixed_step_reference

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


def _td(a, dev, bf=False):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if bf else t).to(dev)


@pytest.mark.parametrize("noalloc", [False, True])
def test_captured_mixed_step_replays_equal_eager(pkv, noalloc):
    dev = torch.device("cuda:0")
    dec, pre, _, _, _ = mixed_step_case()
    _say(f"case graph capture of the mixed step ({'no-alloc' if noalloc else 'workspace'} decode): "
         f"{dec.num_seqs} decode sequences, a {pre.num_new_tokens}-token chunk")
    kp, vp = _td(pre.key_pool, dev, True), _td(pre.value_pool, dev, True)
    kp0, vp0 = kp.clone(), vp.clone()  # pools before the step's write
    q, bt, ctx = _td(dec.query, dev, True), _td(dec.block_tables, dev), _td(dec.context_lens, dev)
    pq, pcu, poff, pbt = (_td(pre.query, dev, True), _td(pre.cu_q_lens, dev), _td(pre.chunk_offsets, dev),
                          _td(pre.block_tables, dev))
    w_cu, w_st = _td(pre.new_cu_lens, dev), _td(pre.new_start_pos, dev)
    kn, vn = _td(pre.key_new, dev, True), _td(pre.value_new, dev, True)
    T = pre.num_new_tokens
    L = int(pre.cu_q_lens[-1])
    slots = torch.empty(T, dtype=torch.int32, device=dev)
    dout = torch.empty((dec.num_seqs, dec.num_q_heads, dec.head_dim), dtype=torch.float32, device=dev)
    pout = torch.empty((L, pre.num_q_heads, pre.head_dim), dtype=torch.float32, device=dev)
    ws = None if noalloc else pkv.decode_workspace(q, dec.num_kv_heads, dec.max_blocks_per_seq)
    pws = pkv.prefill_workspace(pq, 1, L, pre.max_blocks_per_seq)

    def step():
        pkv.slot_mapping(pbt, w_cu, w_st, L, pre.num_blocks, out=slots, total=T)
        pkv.cache_write(kn, vn, kp, vp, slots)
        if noalloc:
            pkv.paged_attn_decode_noalloc(q, kp, vp, bt, ctx, dec.scale, out=dout)
        else:
            pkv.paged_attn_decode(q, kp, vp, bt, ctx, dec.scale, out=dout, workspace=ws)
        pkv.paged_attn_prefill_chunk(pq, pcu, poff, kp, vp, pbt, L, pre.scale, out=pout, workspace=pws)

    # Warm up on a side stream (the library's one-time queries happen outside the capture), then capture.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    dec_ref, pre_ref = mixed_step_reference()
    rng = np.random.default_rng(11)
    for r in range(3):
        if r > 0:  # new queries and new K/V for the chunk, written into the captured buffers
            q.copy_(_td(wl.f32_to_bf16_bits(rng.standard_normal(dec.query.shape).astype(np.float32)), dev, True))
            pq.copy_(_td(wl.f32_to_bf16_bits(rng.standard_normal(pre.query.shape).astype(np.float32)), dev, True))
            kn.copy_(_td(wl.f32_to_bf16_bits(rng.standard_normal(pre.key_new.shape).astype(np.float32)), dev, True))
            vn.copy_(_td(wl.f32_to_bf16_bits(rng.standard_normal(pre.value_new.shape).astype(np.float32)), dev, True))
        # Eager reference on the same inputs, from the pools as they were before the step.
        kp.copy_(kp0)
        vp.copy_(vp0)
        step()
        torch.cuda.synchronize()
        e_dec, e_pre, e_kp = dout.clone(), pout.clone(), kp.clone()
        kp.copy_(kp0)
        vp.copy_(vp0)
        dout.fill_(float("nan"))
        pout.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # Bitwise comparisons (the pools' dead slots hold NaN).
        assert torch.equal(kp.view(torch.int16), e_kp.view(torch.int16)), f"replay {r}: pools differ from the eager step"
        assert torch.equal(dout.view(torch.int32), e_dec.view(torch.int32)), f"replay {r}: decode output differs"
        assert torch.equal(pout.view(torch.int32), e_pre.view(torch.int32)), f"replay {r}: chunk output differs"
        if r == 0:
            close(dout.cpu().numpy(), dec_ref, "replayed decode vs oracle")
            close(pout.cpu().numpy(), pre_ref, "replayed chunk vs oracle")
        _say(f"  replay {r}: bit-identical to the eager step")
