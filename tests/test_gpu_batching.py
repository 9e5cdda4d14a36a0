"""GPU parity of the continuous-batching driver's steps (needs an MI355X).

The driver (batching.py) runs the scheduler's plan of each step on the GPU: slot mapping of the
step's new tokens through the scheduler's block-table rows, the cache write of their K/V, then one
fused launch attending the step's decode tokens and prompt chunks ("Phase 17 · 04 — vLLM serving
internals", scheduler-loop section and its modes; "Chunked Prefill", token-budget section).  This
test drives the same function over a small request set in CONTINUOUS and CONTINUOUS+CHUNKED modes,
with fresh random queries and K/V every step and NaN in every pool slot before it is written, and
mirrors each step on the host: the oracle's slot mapping over the same table rows, its cache write
into its own copy of the pools, then oracle.decode for the decode rows and oracle.prefill_chunk
for the chunk rows.  Bars: slots bit-exact, the pools byte for byte after every step, outputs
within max-abs 1e-2 / mean-abs 1e-3 of the oracle.  Both call modes run (checked kernels with an
err_flag, and the release kernels, err_flag NULL).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_common import MODES, close, flag, new_err, to_dev

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

HQ, HKV, HD = 16, 2, 128
BF16_NAN = 0x7FC0
# (prompt length, output length, arrival in virtual microseconds); each step advances the clock by
# STEP_US, so the later requests join while earlier ones are decoding or mid-prompt.
REQUESTS = [(37, 5, 0.0), (150, 3, 0.0), (300, 6, 0.0), (64, 4, 2500.0), (17, 8, 4500.0), (220, 3, 6500.0),
            (401, 2, 6500.0)]
STEP_US = 1000.0


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_170_amd as m
    return m


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("sched_mode", ["continuous", "chunked"])
@pytest.mark.parametrize("mode", MODES)
def test_scheduled_steps_match_the_oracle(pkv, mode, sched_mode):
    import batching

    dev = torch.device("cuda:0")
    code = batching.MODES[sched_mode]
    n = len(REQUESTS)
    max_blocks = max(-(-(p + o) // 16) for p, o, _ in REQUESTS)
    nblk = sum(-(-(p + o - 1) // 16) for p, o, _ in REQUESTS) + 9
    rng = np.random.default_rng(31 + code)
    bm = pkv.BlockManager(nblk, free_order=rng.permutation(nblk).astype(np.int32))
    max_running = 4
    sched = pkv.Scheduler(code, n, max_running, max_blocks, bm, token_budget=96, max_chunk=64,
                          max_itl_samples=1024)
    for p, o, a in REQUESTS:
        sched.add_request(p, o, a)
    _say(f"case batching ({mode}): {sched_mode}, {n} requests, {nblk} blocks of {HKV}x16x{HD} bf16, "
         f"{HQ}/{HKV} heads, at most {max_running} running")
    kp = torch.full((nblk, HKV, 16, HD), float("nan"), dtype=torch.bfloat16, device=dev)
    vp = torch.full_like(kp, float("nan"))
    rk = np.full((nblk, HKV, 16, HD), BF16_NAN, np.uint16)
    rv = rk.copy()
    d_table = torch.empty((max_running, max_blocks), dtype=torch.int32, device=dev)
    ws = pkv.decode_workspace(torch.empty((max_running, HQ, HD), dtype=torch.bfloat16, device=dev), HKV, max_blocks)
    scale = HD ** -0.5
    err = new_err(dev, mode)
    now, steps, mixed_steps, worst = 0.0, 0, 0, 0.0
    while sched.num_done() < n:
        assert steps < 200, "the schedule did not finish"
        plan = sched.plan(now)
        nd, nc = len(plan["dec_row"]), len(plan["chunk_row"])
        if nd + nc == 0:
            assert plan["next_arrival"] >= 0, "scheduler stalled with requests left"
            now = max(now, plan["next_arrival"])
            continue
        table = sched.table.copy()
        rows, lens, starts, cu = batching.step_layout(plan)
        T = int(cu[-1])
        q = wl.f32_to_bf16_bits(rng.standard_normal((T, HQ, HD)).astype(np.float32))
        kn = wl.f32_to_bf16_bits(rng.standard_normal((T, HKV, HD)).astype(np.float32))
        vn = wl.f32_to_bf16_bits(rng.standard_normal((T, HKV, HD)).astype(np.float32))
        d_table.copy_(torch.from_numpy(table))
        slots, dec_out, pre_out = batching.run_step(pkv, torch, kp, vp, d_table, plan, to_dev(q, dev, True),
                                                    to_dev(kn, dev, True), to_dev(vn, dev, True), ws, scale,
                                                    err_flag=err)
        torch.cuda.synchronize()
        assert flag(err) == 0, f"step {steps}: device checks flagged {flag(err):#x}"
        # The oracle's mirror of the step.
        bt = table[rows]
        ref_slots = oracle.slot_mapping(bt, cu, starts, 16)
        assert np.array_equal(slots.cpu().numpy(), ref_slots), f"step {steps}: slots differ"
        rk, rv = oracle.cache_write(rk, rv, kn, vn, ref_slots)
        assert bits(kp).tobytes() == rk.tobytes() and bits(vp).tobytes() == rv.tobytes(), \
            f"step {steps}: pools differ after the write"
        if nd:
            ref = oracle.decode(q[:nd], rk, rv, bt[:nd], plan["dec_ctx"], scale, "bf16")
            mx, _ = close(dec_out.cpu().numpy(), ref, f"step {steps} decode rows")
            worst = max(worst, mx)
        else:
            assert dec_out is None
        if nc:
            ccu = np.concatenate([[0], np.cumsum(plan["chunk_len"])]).astype(np.int32)
            ref = oracle.prefill_chunk(q[nd:], ccu, plan["chunk_offset"], rk, rv, bt[nd:], scale, "bf16")
            mx, _ = close(pre_out.cpu().numpy(), ref, f"step {steps} chunk rows")
            worst = max(worst, mx)
        else:
            assert pre_out is None
        mixed_steps += bool(nd and nc)
        now += STEP_US
        sched.complete(now)
        steps += 1
    assert bm.num_free() == nblk, "blocks leaked"
    assert mixed_steps >= 2, "no step carried decode tokens and prompt chunks together"
    _say(f"  {steps} steps ({mixed_steps} with both decode tokens and chunks), worst max-abs {worst:.2e}")
