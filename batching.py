"""Continuous-batching driver: the four scheduling modes of the serving pages run over one set of
synthetic requests, with every step's attention executed by the library's kernels on the GPU.

What is modelled ("Phase 17 · 04 — vLLM serving internals", scheduler-loop section and the toy
scheduler's four modes; "第2章:推理引擎核心技术" §2.3 iteration-level scheduling): requests arrive,
wait, are admitted when a running slot and KV blocks are free, have their prompt prefilled (whole,
or in budgeted chunks), then decode one token per step until their output length.  Each step is
executed for real on one attention layer of the 70B-style shape (64 query / 8 KV heads, head_dim
128, bf16, 16-token blocks): slot mapping and cache write of the step's new tokens (synthetic K/V),
then the fused decode + chunk attention launch.  There are no model weights: the virtual clock
advances by the measured GPU time of that attention work, so TTFT / ITL / throughput here are
attention-only figures, comparable between modes, not end-to-end serving numbers.

Synthetic requests (seeded): prompt lengths lognormal with mean 1500 and standard deviation 600,
clipped to [16, 8192] (the pages' exercise numbers), output lengths uniform in [32, 256] (the pages
give none), all arriving at time 0 unless --arrival-rate is given (Poisson, requests per second of
virtual time).

Usage: python batching.py [--requests 128] [--modes naive,static,continuous,chunked]
Prints one JSON line per mode on stdout.
"""
import argparse
import json
import math
import sys
import time

import numpy as np

MODES = {"naive": 0, "static": 1, "continuous": 2, "chunked": 3}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--requests", type=int, default=128)
    ap.add_argument("--max-running", type=int, default=128)
    ap.add_argument("--token-budget", type=int, default=2048, help="tokens per step in chunked mode")
    ap.add_argument("--max-chunk", type=int, default=512, help="largest prompt chunk in chunked mode")
    ap.add_argument("--arrival-rate", type=float, default=0.0, help="Poisson arrivals per virtual second (0: burst)")
    ap.add_argument("--modes", default="naive,static,continuous,chunked")
    ap.add_argument("--seed", type=int, default=17)
    return ap.parse_args()


def requests(n, seed, rate):
    rng = np.random.default_rng(seed)
    sigma = math.sqrt(math.log(1 + (600 / 1500) ** 2))
    mu = math.log(1500) - sigma ** 2 / 2
    prompt = np.clip(np.rint(rng.lognormal(mu, sigma, n)), 16, 8192).astype(np.int32)
    output = rng.integers(32, 257, n).astype(np.int32)
    arrival = np.zeros(n) if rate <= 0 else np.cumsum(rng.exponential(1e6 / rate, n))  # microseconds
    return prompt, output, arrival


def step_layout(plan):
    """Host-side layout of one planned step's new tokens: every decode entry writes one token (at
    position ctx - 1), then every prompt chunk writes its tokens; the step's queries are packed in
    the same order.  Returns (table rows, tokens per entry, first position per entry, cu offsets)."""
    nd = len(plan["dec_row"])
    rows = np.concatenate([plan["dec_row"], plan["chunk_row"]]).astype(np.int64)
    lens = np.concatenate([np.ones(nd, np.int32), plan["chunk_len"]]).astype(np.int32)
    starts = np.concatenate([plan["dec_ctx"] - 1, plan["chunk_offset"]]).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return rows, lens, starts, cu


def run_step(pkv, torch, kp, vp, table, plan, query, key_new, value_new, workspace, scale, err_flag=None,
             stream=None, events=None):
    """Execute one planned step on the GPU: slot mapping of the step's new tokens (step_layout's
    order) through the scheduler's table rows, the cache write of their K/V, then one fused
    attention launch of the step's decode tokens and prompt chunks (causal).

    table: the scheduler's block-table rows on the device (int32 [max_running, max_blocks]);
    query [T, Hq, hd], key_new / value_new [T, Hkv, hd] (bf16, T = the step's token count).
    events: optional (start, end) CUDA events recorded around the GPU work on `stream`.
    Returns (slots, decode output or None, chunk output or None); outputs are fp32."""
    dev = kp.device
    nd, nc = len(plan["dec_row"]), len(plan["chunk_row"])
    rows, lens, starts, cu = step_layout(plan)
    T = int(cu[-1])
    bt_all = table.index_select(0, torch.from_numpy(rows).to(dev))
    cu_d, st_d = torch.from_numpy(cu).to(dev), torch.from_numpy(starts).to(dev)
    dec_kw, pre_kw = {}, {}
    if nd:
        dec_kw = dict(dec_query=query[:nd], dec_block_tables=bt_all[:nd],
                      context_lens=torch.from_numpy(plan["dec_ctx"]).to(dev), workspace=workspace)
    if nc:
        ccu = np.concatenate([[0], np.cumsum(plan["chunk_len"])]).astype(np.int32)
        pre_kw = dict(pre_query=query[nd:nd + int(ccu[-1])], cu_q_lens=torch.from_numpy(ccu).to(dev),
                      chunk_offsets=torch.from_numpy(plan["chunk_offset"]).to(dev),
                      pre_block_tables=bt_all[nd:], max_q_len=int(plan["chunk_len"].max()))
    slots = torch.empty(T, dtype=torch.int32, device=dev)
    if events is not None:
        events[0].record(stream)
    pkv.slot_mapping(bt_all, cu_d, st_d, int(lens.max()), kp.shape[0], out=slots, err_flag=err_flag)
    pkv.cache_write(key_new[:T], value_new[:T], kp, vp, slots, err_flag=err_flag)
    dec_out, pre_out = pkv.paged_attn_mixed(kp, vp, scale, causal=True, err_flag=err_flag, **dec_kw, **pre_kw)
    if events is not None:
        events[1].record(stream)
    return slots, dec_out, pre_out


def run_mode(pkv, torch, mode, args, prompt, output, arrival):
    dev = torch.device("cuda:0")
    hq, hkv, hd = 64, 8, 128
    n = len(prompt)
    max_blocks = int(-(-(int(prompt.max()) + int(output.max())) // 16))
    need = int(sum(-(-(int(p) + int(o) - 1) // 16) for p, o in zip(prompt, output)))
    nblk = max(int(need * 1.1), 64)
    bm = pkv.BlockManager(nblk)
    sched = pkv.Scheduler(mode, n, args.max_running, max_blocks, bm, token_budget=args.token_budget,
                          max_chunk=args.max_chunk, max_itl_samples=int(output.sum()))
    for p, o, a in zip(prompt, output, arrival):
        sched.add_request(int(p), int(o), float(a))
    g = torch.Generator(device=dev).manual_seed(args.seed)
    kp = torch.zeros((nblk, hkv, 16, hd), dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    # Synthetic step inputs: slices of fixed random buffers (contents do not affect timing).
    max_tok = max(args.token_budget, int(prompt.max())) * (1 if mode == 3 else args.max_running) + args.max_running
    max_tok = min(max_tok, int(prompt.sum()) + n)
    kv_src = torch.randn((max_tok, hkv, hd), generator=g, device=dev).to(torch.bfloat16)
    q_src = torch.randn((max_tok, hq, hd), generator=g, device=dev).to(torch.bfloat16)
    d_table = torch.empty((args.max_running, max_blocks), dtype=torch.int32, device=dev)
    ws = pkv.decode_workspace(q_src[: args.max_running], hkv, max_blocks)
    scale = hd ** -0.5
    stream = torch.cuda.current_stream(dev)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    now, steps, gpu_ms, t_wall = 0.0, 0, 0.0, time.perf_counter()
    while sched.num_done() < n:
        plan = sched.plan(now)
        if len(plan["dec_row"]) + len(plan["chunk_row"]) == 0:
            if plan["next_arrival"] < 0:
                raise RuntimeError("scheduler stalled with requests left")
            now = max(now, plan["next_arrival"])
            continue
        d_table.copy_(torch.from_numpy(sched.table))
        run_step(pkv, torch, kp, vp, d_table, plan, q_src, kv_src, kv_src, ws, scale, stream=stream, events=ev)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1])
        gpu_ms += ms
        now += ms * 1e3  # microseconds of virtual time
        sched.complete(now)
        steps += 1
    wall = time.perf_counter() - t_wall
    times = np.array([sched.request_times(i) for i in range(n)])
    ttft = (times[:, 1] - times[:, 0]) / 1e3
    itl = sched.itl() / 1e3
    span = (times[:, 2].max() - times[:, 0].min()) / 1e6
    assert bm.num_free() == nblk, "blocks leaked"
    return {"mode": [k for k, v in MODES.items() if v == mode][0], "requests": n, "steps": steps,
            "generated_tokens": int(output.sum()), "virtual_s": span,
            "throughput_tok_per_s": float(output.sum()) / span, "ttft_ms_mean": float(ttft.mean()),
            "ttft_ms_p99": float(np.percentile(ttft, 99)), "itl_ms_p50": float(np.percentile(itl, 50)),
            "itl_ms_p99": float(np.percentile(itl, 99)), "attention_gpu_ms": gpu_ms, "wall_s": wall,
            "max_running": 1 if mode == 0 else args.max_running,
            "token_budget": args.token_budget if mode == 3 else None,
            "max_chunk": args.max_chunk if mode == 3 else None}


def main():
    args = parse()
    import torch

    import paged_kv_cache_170_amd as pkv

    if not torch.cuda.is_available():
        print("batching.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    prompt, output, arrival = requests(args.requests, args.seed, args.arrival_rate)
    print(f"[batching] {args.requests} requests: prompt mean {prompt.mean():.0f} (max {prompt.max()}), "
          f"output mean {output.mean():.0f}", file=sys.stderr, flush=True)
    for name in args.modes.split(","):
        res = run_mode(pkv, torch, MODES[name], args, prompt, output, arrival)
        print(f"[batching] {name}: {res['steps']} steps, {res['throughput_tok_per_s']:.0f} tok/s, TTFT mean "
              f"{res['ttft_ms_mean']:.2f} ms, ITL p99 {res['itl_ms_p99']:.3f} ms (wall {res['wall_s']:.1f} s)",
              file=sys.stderr, flush=True)
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
