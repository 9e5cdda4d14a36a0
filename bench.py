"""Benchmark of the paged-KV hot path on one MI355X.

A step is one pass of the whole path over the mixed chunked-prefill + decode workload
(70B-style GQA layer: 64 query heads / 8 KV heads x 128, bf16, 16-token blocks):
  1. slot mapping of the 512 new prompt tokens (chunk at offset 16,384 of a 32,768-token prompt),
  2. cache write of their K/V into the pool,
  3. decode of 127 sequences (contexts uniform in 200..8192, a shared 63-block prefix),
  4. prefill-chunk attention of the 512 rows over 16,384 cached + 512 causal positions,
all enqueued on one stream with inputs resident in HBM.

Timing: every timed step starts from cold caches.  Before each step (outside its events) a 1 GiB
buffer is read, which evicts the L2s and the 256 MB MALL without leaving dirty lines behind;
per-kernel times come from HIP events on the launch stream and are reported as median, p10 and
p90.  The same steps run back to back without the flush ("hot") are reported beside them.

Printed: one JSON line.  `value` is the decode KV-read bandwidth in GB/s over unique pool bytes
(the shared prefix counted once) at the median flushed decode call (plan, attention and reduce);
the prefill chunk's TFLOP/s, both fractions of peak, the hot figures, the two small configs
(tiny fp32 decode, 1000-token chunked prefill), a batch of short prefill chunks (32 prompts x
32 tokens at offset 2,048) and the decode of one 32,768-position sequence are in `secondary`; `roofline` describes the
kernel that takes the most time per step, at its average flushed duration.  `cpu_baseline` times
the fp64 oracle on this host on the same inputs (decode of every sequence, prefill of a sample of
rows), with the small configs' oracle times (all host threads and one thread) beside it.

Other workloads (--workload): gqa_decode and long_decode (decode only), and shared_prefix (64
sequences behind one 4,096-token cached prompt, decoded by the shared-prefix decode, with the
plain decode on the same inputs timed beside it; with --kv fp8 the FP8 variants of both).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6  # dense: 256 CUs x 2.4 GHz x 4096 flop/clk
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed_step",
                    choices=["mixed_step", "gqa_decode", "long_decode", "shared_prefix"])
    ap.add_argument("--kv", default="bf16", choices=["bf16", "fp8"],
                    help="KV pool storage: bf16, or E4M3 codes with per-pool scales (quantised from the bf16 "
                         "pools at setup; the step's new tokens go through the quantising write)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hot-steps", type=int, default=-1,
                    help="steps run back to back without the flush, reported beside the flushed ones "
                         "(default: as many as --steps; 0 skips them)")
    ap.add_argument("--no-flush", action="store_true",
                    help="time the steps without the cache flush (for profilers that count every launch)")
    ap.add_argument("--no-small-configs", action="store_true",
                    help="skip the tiny-decode, chunked-prefill, short-chunk and single-sequence runs in secondary")
    ap.add_argument("--cpu-sample-rows", type=int, default=64, help="prefill rows timed in the oracle baseline")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before timing, run a plain fp32 copy kernel over this many MiB (a known-size reference "
                         "for HBM byte counters)")
    return ap.parse_args()


def sources_hash(names):
    """Hash of a kernel's sources: the .hip file, its device header (if any) and common.hpp."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_170_amd", "csrc")
    for n in names:
        for f_name in (n, n.replace(".hip", "_dev.hpp")):
            path = os.path.join(csrc, f_name)
            if f_name != n and not os.path.exists(path):
                continue
            with open(path, "rb") as f:
                h.update(f.read())
    with open(os.path.join(ROOT, "paged_kv_cache_170_amd", "csrc", "common.hpp"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def counter_record(kernel_key: str, src):
    """A committed counter summary (profiles/counters_<kernel>_<workload>.json), if it was taken
    on these sources (src: one .hip file or a list of them); else None."""
    path = os.path.join(PROFILES, f"counters_{kernel_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_hash") != sources_hash([src] if isinstance(src, str) else list(src)):
        return None
    return rec


def counter_traffic(kernel_key: str, src):
    """HBM bytes per launch from a committed counter summary taken on these sources."""
    rec = counter_record(kernel_key, src)
    return None if rec is None else rec.get("traffic_bytes_per_launch")


def unique_kv_bytes(case) -> int:
    """K+V elements of the distinct pool rows the decode reads (shared blocks counted once)."""
    rows = set()
    for s in range(case.num_seqs):
        n = int(case.context_lens[s])
        nb = -(-n // 16)
        for j in range(nb):
            b = int(case.block_tables[s, j])
            cnt = 16 if j < nb - 1 else n - 16 * (nb - 1)
            rows.update(b * 16 + o for o in range(cnt))
    return len(rows) * 2 * case.num_kv_heads * case.head_dim


def decode_algorithmic_bytes(case, out_bytes=4, kv_elem=None):
    kv_elem = case.elem_bytes if kv_elem is None else kv_elem
    kv = unique_kv_bytes(case) * kv_elem
    logical = int(case.context_lens.astype(np.int64).sum()) * 2 * case.num_kv_heads * case.head_dim * kv_elem
    q = case.num_seqs * case.num_q_heads * case.head_dim * case.elem_bytes
    o = case.num_seqs * case.num_q_heads * case.head_dim * out_bytes
    table = 4 * int(sum(-(-int(n) // 16) for n in case.context_lens))
    return kv + q + o + table + 4 * case.num_seqs, kv, logical


def prefill_flops(case) -> int:
    total = 0
    for s in range(len(case.chunk_offsets)):
        L = int(case.cu_q_lens[s + 1] - case.cu_q_lens[s])
        o = int(case.chunk_offsets[s])
        vis = L * o + L * (L + 1) // 2 if case.causal else L * (o + L)
        total += vis
    return 4 * case.head_dim * case.num_q_heads * total


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # pragma: no cover
        return 1


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the kernels run on a "
              f"single device; sharding is described in the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_170_amd as pkv
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    if args.workload == "mixed_step":
        dec, pre = wl.mixed_step(poison=False)
    elif args.workload == "gqa_decode":
        dec, pre = wl.gqa_decode(poison=False), None
    elif args.workload == "shared_prefix":
        dec, pre = wl.shared_prefix_decode(poison=False), None
    else:
        dec, pre = wl.long_decode(poison=False), None
    gen_s = time.perf_counter() - t_gen
    print(f"[bench] workload {args.workload} generated in {gen_s:.1f}s", file=sys.stderr, flush=True)

    def to_dev(a, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf16 else t).to(dev)

    bf = dec.dtype == "bf16"
    kp, vp = to_dev(dec.key_pool, bf), to_dev(dec.value_pool, bf)
    # The new tokens of this step (the prefill chunk for the mixed step, the last block per
    # sequence for long decode).
    wcase = pre if pre is not None else dec
    has_write = wcase.num_new_tokens > 0
    if has_write:
        w_bt = to_dev(wcase.block_tables)
        w_cu = to_dev(wcase.new_cu_lens)
        w_start = to_dev(wcase.new_start_pos)
        w_k, w_v = to_dev(wcase.key_new, bf), to_dev(wcase.value_new, bf)
        w_max = int(np.diff(wcase.new_cu_lens).max())
        slots = torch.empty(wcase.num_new_tokens, dtype=torch.int32, device=dev)
    fp8 = args.kv == "fp8"
    if fp8 and not bf:
        raise SystemExit("--kv fp8 needs a bf16 workload")
    # FP8 pools: every slot of the bf16 pools quantised by the library's own write (setup, untimed).
    # Scale 2^-5 for both pools: N(0,1) values stay far inside E4M3's +-448 range.
    k_scale = v_scale = 2.0 ** -5
    if fp8:
        kp8 = torch.empty(kp.shape, dtype=torch.float8_e4m3fn, device=dev)
        vp8 = torch.empty_like(kp8)
        nrow = kp.shape[0] * kp.shape[2]
        all_slots = torch.arange(nrow, dtype=torch.int32, device=dev)
        # Token rows in slot order (pools are [blocks, Hkv, 16, hd]) through the quantising write.
        rows = lambda p: p.permute(0, 2, 1, 3).reshape(nrow, p.shape[1], p.shape[3])
        pkv.cache_write_fp8(rows(kp), rows(vp), kp8, vp8,
                            all_slots, k_scale, v_scale)
        torch.cuda.synchronize()
        del all_slots
    d_q = to_dev(dec.query, bf)
    d_bt, d_ctx = to_dev(dec.block_tables), to_dev(dec.context_lens)
    d_out = torch.empty((dec.num_seqs, dec.num_q_heads, dec.head_dim), dtype=torch.float32, device=dev)
    ws = pkv.decode_workspace(d_q, dec.num_kv_heads, dec.max_blocks_per_seq)
    # Shared-prefix workload: the decode attends the shared blocks once for all members.
    pfx = args.workload == "shared_prefix"
    if pfx:
        d_members = to_dev(dec.notes["members"])
        pfx_blocks = int(dec.notes["prefix_blocks"])
        ws = pkv.decode_prefix_workspace(d_q, dec.num_kv_heads, dec.max_blocks_per_seq)
    if pre is not None:
        p_q = to_dev(pre.query, bf)
        p_cu, p_off, p_bt = to_dev(pre.cu_q_lens), to_dev(pre.chunk_offsets), to_dev(pre.block_tables)
        p_out = torch.empty((pre.query.shape[0], pre.num_q_heads, pre.head_dim), dtype=torch.float32, device=dev)
        p_maxl = int(np.diff(pre.cu_q_lens).max())
        p_ws = pkv.prefill_workspace(p_q, len(pre.chunk_offsets), p_maxl, pre.max_blocks_per_seq)
    torch.cuda.synchronize()

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] copy reference: 3 x ({args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written)",
              file=sys.stderr, flush=True)

    names = ["slot_mapping", "cache_write", "decode", "prefill"]
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        if has_write:
            pkv.slot_mapping(w_bt, w_cu, w_start, w_max, dec.num_blocks, out=slots)
        mark(1)
        if has_write:
            if fp8:
                pkv.cache_write_fp8(w_k, w_v, kp8, vp8, slots, k_scale, v_scale)
            else:
                pkv.cache_write(w_k, w_v, kp, vp, slots)
        mark(2)
        if fp8 and pfx:
            pkv.paged_attn_decode_prefix_fp8(d_q, kp8, vp8, d_bt, d_ctx, dec.scale, k_scale, v_scale, d_members,
                                             pfx_blocks, out=d_out, workspace=ws)
        elif fp8:
            pkv.paged_attn_decode_fp8(d_q, kp8, vp8, d_bt, d_ctx, dec.scale, k_scale, v_scale, out=d_out, workspace=ws)
        elif pfx:
            pkv.paged_attn_decode_prefix(d_q, kp, vp, d_bt, d_ctx, dec.scale, d_members, pfx_blocks, out=d_out,
                                         workspace=ws)
        else:
            pkv.paged_attn_decode(d_q, kp, vp, d_bt, d_ctx, dec.scale, out=d_out, workspace=ws)
        mark(3)
        if pre is not None:
            if fp8:
                pkv.paged_attn_prefill_chunk_fp8(p_q, p_cu, p_off, kp8, vp8, p_bt, p_maxl, pre.scale, k_scale, v_scale,
                                                 causal=True, out=p_out, workspace=p_ws)
            else:
                pkv.paged_attn_prefill_chunk(p_q, p_cu, p_off, kp, vp, p_bt, p_maxl, pre.scale, causal=True,
                                             out=p_out, workspace=p_ws)
        mark(4)

    # The flush: a 1 GiB read evicts the L2s and the 256 MB MALL and leaves only clean lines, so no
    # write-back of the flush itself lands inside the next step.
    flush_buf = None if args.no_flush else torch.ones(1 << 28, dtype=torch.int32, device=dev)

    def flush():
        if flush_buf is not None:
            torch.amax(flush_buf)

    def collect(evs):
        out = {n: [] for n in names + ["step"]}
        for ev in evs:
            for i, n in enumerate(names):
                out[n].append(ev[i].elapsed_time(ev[i + 1]))
            out["step"].append(ev[0].elapsed_time(ev[len(names)]))
        return out

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        flush()
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = collect(events)
    avg_ms = {n: float(np.mean(v)) for n, v in per.items()}
    med_ms = {n: float(np.median(v)) for n, v in per.items()}
    ms_per_step = wall * 1e3 / args.steps
    print(f"[bench] {args.steps} {'flushed ' if flush_buf is not None else ''}steps in {wall:.3f}s; per-kernel "
          "median ms " + ", ".join(f"{n}={med_ms[n]:.4f}" for n in names), file=sys.stderr, flush=True)

    def spread(v):
        return {"p10": float(np.percentile(v, 10)), "p50": float(np.median(v)), "p90": float(np.percentile(v, 90))}

    # The same steps back to back, caches warm from the previous step.
    hot_steps = args.steps if args.hot_steps < 0 else args.hot_steps
    hot = None
    if hot_steps > 0:
        hev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(hot_steps)]
        for k in range(hot_steps):
            step(hev[k])
        torch.cuda.synchronize()
        hot = collect(hev)
        print(f"[bench] {hot_steps} hot steps; per-kernel median ms "
              + ", ".join(f"{n}={float(np.median(hot[n])):.4f}" for n in names), file=sys.stderr, flush=True)
    del flush_buf

    # Bandwidth a plain read stream reaches on this device: read the whole key pool (>= 1 GB).
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        pkv.stream_read_probe(kp, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        pkv.stream_read_probe(kp, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    stream_gbs = 5 * kp.numel() * kp.element_size() / (e0.elapsed_time(e1) * 1e-3) / 1e9

    # Rate a kernel of pure bf16 MFMA work reaches on this device (every SIMD issuing 32x32x16
    # MFMAs on operands that change from one MFMA to the next, and nothing else), run for about as
    # long as the prefill chunk takes.
    mfma_loop = None
    if pre is not None:
        msink = torch.zeros(1, dtype=torch.float32, device=dev)
        pkv.mfma_peak_probe(2000, msink)
        e0.record(stream)
        mflop = sum(pkv.mfma_peak_probe(2000, msink) for _ in range(5))
        e1.record(stream)
        torch.cuda.synchronize()
        mt = e0.elapsed_time(e1) / 5
        mfma_loop = {"ms_per_call": mt, "tflops": mflop / 5 / (mt * 1e-3) / 1e12}
        mfma_loop["frac_of_peak"] = mfma_loop["tflops"] / BF16_MFMA_PEAK_TFLOPS

    # Fused mixed-batch launch against the two separate attention calls (same inputs, same pools).
    fused_info = None
    if pre is not None:
        fkp, fvp = (kp8, vp8) if fp8 else (kp, vp)
        sc = (k_scale, v_scale) if fp8 else (1.0, 1.0)

        def fused():
            pkv.paged_attn_mixed(fkp, fvp, dec.scale, dec_query=d_q, dec_block_tables=d_bt, context_lens=d_ctx,
                                 pre_query=p_q, cu_q_lens=p_cu, chunk_offsets=p_off, pre_block_tables=p_bt,
                                 max_q_len=p_maxl, causal=True, k_scale=sc[0], v_scale=sc[1], dec_out=d_out,
                                 pre_out=p_out, workspace=ws, pre_workspace=p_ws)

        def separate():
            if fp8:
                pkv.paged_attn_decode_fp8(d_q, kp8, vp8, d_bt, d_ctx, dec.scale, k_scale, v_scale, out=d_out,
                                          workspace=ws)
                pkv.paged_attn_prefill_chunk_fp8(p_q, p_cu, p_off, kp8, vp8, p_bt, p_maxl, pre.scale, k_scale,
                                                 v_scale, causal=True, out=p_out, workspace=p_ws)
            else:
                pkv.paged_attn_decode(d_q, kp, vp, d_bt, d_ctx, dec.scale, out=d_out, workspace=ws)
                pkv.paged_attn_prefill_chunk(p_q, p_cu, p_off, kp, vp, p_bt, p_maxl, pre.scale, causal=True,
                                             out=p_out, workspace=p_ws)

        times = {}
        for name, fn in (("separate", separate), ("fused", fused), ("separate", separate), ("fused", fused)):
            fn()
            e0.record(stream)
            for _ in range(10):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times[name] = min(times.get(name, 1e9), e0.elapsed_time(e1) / 10)
        fused_info = {"fused_ms": times["fused"], "separate_ms": times["separate"],
                      "speedup": times["separate"] / times["fused"]}

    # Shared-prefix workload: the plain decode on the same inputs (every shared block read once per
    # member, mostly from L2), for comparison.
    plain_info = None
    if pfx:
        p_out = torch.empty_like(d_out)
        pws = pkv.decode_workspace(d_q, dec.num_kv_heads, dec.max_blocks_per_seq)
        pt = 1e9

        def plain():
            if fp8:
                pkv.paged_attn_decode_fp8(d_q, kp8, vp8, d_bt, d_ctx, dec.scale, k_scale, v_scale, out=p_out,
                                          workspace=pws)
            else:
                pkv.paged_attn_decode(d_q, kp, vp, d_bt, d_ctx, dec.scale, out=p_out, workspace=pws)
        for _ in range(3):
            plain()
            e0.record(stream)
            for _ in range(10):
                plain()
            e1.record(stream)
            torch.cuda.synchronize()
            pt = min(pt, e0.elapsed_time(e1) / 10)
        step()
        torch.cuda.synchronize()
        # Both back to back (warm caches): the plain decode's best of three, the prefix decode's hot median.
        pfx_ms = float(np.median(hot["decode"])) if hot is not None else avg_ms["decode"]
        plain_info = {"plain_decode_ms": pt, "prefix_decode_ms": pfx_ms,
                      "speedup": pt / pfx_ms, "max_abs_diff": float((p_out - d_out).abs().max()),
                      "members": int(len(dec.notes["members"])), "prefix_blocks": pfx_blocks}
        del p_out, pws

    # Copy-on-write block copies on this pool: 512 disjoint pairs (K and V, read + written).
    nblk = dec.num_blocks
    cp = torch.randperm(nblk, device="cpu")[:1024].to(torch.int32)
    c_src, c_dst = cp[:512].to(dev), cp[512:].to(dev)
    for _ in range(2):
        pkv.copy_blocks(kp, vp, c_src, c_dst)
    e0.record(stream)
    for _ in range(10):
        pkv.copy_blocks(kp, vp, c_src, c_dst)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / 10
    block_bytes = kp[0].numel() * kp.element_size()
    copy_info = {"pairs": 512, "ms": copy_ms, "gbs": 4 * 512 * block_bytes / (copy_ms * 1e-3) / 1e9}

    # Host-side block manager on the decode batch's shape: every sequence is added (a shared
    # prefix of full blocks: the workload's own, else 63 as in the mixed step), extended by one
    # decode token, and freed.
    bm = pkv.BlockManager(nblk)
    rows = np.full((dec.num_seqs, dec.max_blocks_per_seq), -1, np.int32)
    prefix = np.arange(int((dec.notes or {}).get("prefix_blocks", 63)) * 16, dtype=np.int32)
    prompts = [np.concatenate([prefix, np.full(max(int(c) - 1 - prefix.size, 0), 100000 + s, np.int32)])[: int(c) - 1]
               for s, c in enumerate(dec.context_lens)]
    t_bm = time.perf_counter()
    hits = 0
    for s in range(dec.num_seqs):
        hits += bm.add_sequence(prompts[s], rows[s]) > 0
    for s in range(dec.num_seqs):
        bm.append(rows[s], prompts[s].size, 1)
    for s in range(dec.num_seqs):
        bm.free_sequence(rows[s], prompts[s].size + 1)
    bm_us = (time.perf_counter() - t_bm) * 1e6 / (3 * dec.num_seqs)
    bm_info = {"sequences": dec.num_seqs, "prefix_hits": hits, "us_per_operation": bm_us}

    dec_bytes, dec_kv_unique, dec_kv_logical = decode_algorithmic_bytes(dec, kv_elem=1 if fp8 else None)
    # Headline: the median flushed decode call (plan, attention, reduce).
    dec_s = med_ms["decode"] * 1e-3
    dec_gbs = dec_bytes / dec_s / 1e9
    secondary = {
        "timing": ("flushed: a 1 GiB read before each step evicts L2 and MALL; medians over the timed steps"
                   if not args.no_flush else "no flush: steps back to back"),
        "decode_ms": med_ms["decode"],
        "decode_ms_avg": avg_ms["decode"],
        "decode_gbs_unique": dec_gbs,
        "decode_frac_hbm_peak": dec_gbs / HBM_PEAK_GBS,
        "decode_gbs_logical": (dec_bytes - dec_kv_unique + dec_kv_logical) / dec_s / 1e9,
        "decode_kv_bytes_unique": dec_kv_unique,
        "decode_kv_bytes_logical": dec_kv_logical,
        "stream_read_gbs": stream_gbs,
        "decode_frac_of_stream_read": dec_gbs / stream_gbs,
        "fused_mixed_step": fused_info,
        "shared_prefix_vs_plain": plain_info,
        "copy_blocks": copy_info,
        "block_manager_host": bm_info,
    }
    ran = [n for n in names if (has_write or n not in ("slot_mapping", "cache_write")) and (pre is not None or n != "prefill")]
    secondary["kernel_ms"] = {n: spread(per[n]) for n in ran + ["step"]}
    hot_info = None
    if hot is not None:
        hot_info = {"kernel_ms": {n: spread(hot[n]) for n in ran + ["step"]}}
        hdec = float(np.median(hot["decode"]))
        hot_info.update({"decode_ms": hdec, "decode_gbs_unique": dec_bytes / (hdec * 1e-3) / 1e9,
                         "decode_frac_hbm_peak": dec_bytes / (hdec * 1e-3) / 1e9 / HBM_PEAK_GBS})
    secondary["hot"] = hot_info
    # The shared-prefix decode also runs the fused launch (mixed.hip) and the prefill body.
    dec_src = ["decode.hip", "mixed.hip", "prefill.hip"] if pfx else "decode.hip"
    # Roofline of each kernel at its average flushed duration over the timed steps.
    dec_gbs_avg = dec_bytes / (avg_ms["decode"] * 1e-3) / 1e9
    kernels = {"decode": (avg_ms["decode"], "hbm", dec_bytes, dec_gbs_avg, HBM_PEAK_GBS, "GB/s", dec_src)}
    tag = args.workload + ("_fp8" if fp8 else "")
    if pre is not None:
        fl = prefill_flops(pre)
        pre_tf = fl / (med_ms["prefill"] * 1e-3) / 1e12
        secondary.update({"prefill_ms": med_ms["prefill"], "prefill_ms_avg": avg_ms["prefill"], "prefill_flop": fl,
                          "prefill_tflops": pre_tf, "prefill_frac_mfma_peak": pre_tf / BF16_MFMA_PEAK_TFLOPS,
                          "mfma_loop": mfma_loop,
                          "prefill_frac_of_mfma_loop": pre_tf / mfma_loop["tflops"] if mfma_loop else None})
        if hot is not None:
            hpre = float(np.median(hot["prefill"]))
            hot_info.update({"prefill_ms": hpre, "prefill_tflops": fl / (hpre * 1e-3) / 1e12,
                             "prefill_frac_mfma_peak": fl / (hpre * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS})
        pre_tf_avg = fl / (avg_ms["prefill"] * 1e-3) / 1e12
        kernels["prefill"] = (avg_ms["prefill"], "mfma", fl, pre_tf_avg, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s", "prefill.hip")
        # Matrix-core counters of the prefill kernel (committed summary of a rocprofv3 pass on these sources).
        rec = counter_record(f"prefill_{tag}", "prefill.hip")
        secondary["prefill_mfma_counters"] = None if rec is None else rec.get("mfma")
    if has_write:
        # read the new rows (bf16 or fp32) and write them into the pools (E4M3: one byte each)
        wb = (2 * wcase.num_new_tokens * wcase.num_kv_heads * wcase.head_dim * (wcase.elem_bytes + (1 if fp8 else wcase.elem_bytes))
              + 4 * wcase.num_new_tokens)
        secondary.update({"cache_write_ms": med_ms["cache_write"], "slot_mapping_ms": med_ms["slot_mapping"],
                          "cache_write_gbs": wb / (med_ms["cache_write"] * 1e-3) / 1e9})
    dominant = max(kernels, key=lambda k: kernels[k][0])
    ms, bound, work, achieved, peak, unit, src = kernels[dominant]
    roofline = {"kernel": dominant, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": counter_traffic(f"{dominant}_{tag}", src),
                "work_per_launch": work, "avg_launch_ms": ms}
    for k, (ms_k, bound_k, work_k, ach_k, peak_k, unit_k, src_k) in kernels.items():
        secondary[f"roofline_{k}"] = {"bound": bound_k, "achieved": ach_k, "peak": peak_k, "unit": unit_k,
                                      "frac": ach_k / peak_k, "avg_launch_ms": ms_k,
                                      "traffic": counter_traffic(f"{k}_{tag}", src_k)}
    small = None
    if not args.no_small_configs and not fp8 and args.workload == "mixed_step":
        small = small_configs(pkv, torch, dev, flush_bytes=0 if args.no_flush else 1 << 30)
        secondary["small_configs"] = small["gpu"]
        secondary["short_chunk_batch"] = short_chunk_batch(pkv, torch, dev, flush_bytes=0 if args.no_flush else 1 << 30)
        secondary["single_sequence_decode"] = single_sequence_decode(pkv, torch, dev,
                                                                     flush_bytes=0 if args.no_flush else 1 << 30)

    cpu = None
    if fp8:
        print("[bench] cpu baseline is reported for the bf16 pools only", file=sys.stderr, flush=True)
    elif not args.no_cpu_baseline:
        cpu = cpu_baseline(dec, pre, kp, vp, has_write, args, torch)
        if small is not None:
            cpu["small_configs"] = small_configs_oracle(small)

    config = {"workload": args.workload, "num_seqs_decode": dec.num_seqs, "q_heads": dec.num_q_heads,
              "kv_heads": dec.num_kv_heads, "head_dim": dec.head_dim, "block_size": 16,
              "context_lens": {"mixed_step": "uniform 200..8192, shared 63-block prefix",
                               "gqa_decode": "lognormal mean 1500, sd 600, clipped 16..8192",
                               "long_decode": "4096 each",
                               "shared_prefix": "shared 256-block (4,096-token) prefix + uniform 1..512 private"
                               }[args.workload],
              "seed": {"mixed_step": 5, "gqa_decode": 3, "long_decode": 4, "shared_prefix": 6}[args.workload],
              "kv_storage": "fp8_e4m3 (k_scale = v_scale = 2^-5)" if fp8 else ("bf16" if bf else "f32")}
    if pre is not None:
        config.update({"prefill_chunk": int(pre.cu_q_lens[-1]), "prefill_offset": int(pre.chunk_offsets[0])})
    line = {"metric": "paged decode KV-read GB/s (% HBM peak); chunked-prefill TFLOP/s (% MFMA)",
            "value": dec_gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16" if bf else "f32", "data": "synthetic", "config": config,
            "roofline": roofline, "cpu_baseline": cpu, "secondary": secondary,
            "kernel_ms_median": med_ms}
    print(json.dumps(line), flush=True)


def small_configs(pkv, torch, dev, flush_bytes, runs=20):
    """The two small configs on the GPU: the tiny fp32 decode (4 sequences, contexts 17/50/100/128,
    8 heads x 64) and the 1000-token chunked prefill (8 heads x 64, bf16, chunks 256/256/256/232).
    A run writes the new tokens (slot mapping + cache write) and attends (the decode; the four
    chunks, each written before its attention).  Median over `runs` runs, each after the flush,
    of the attention time and of the whole run (HIP events).  Both are launch-bound: a handful of
    microseconds per call."""
    import workloads as wl

    stream = torch.cuda.current_stream(dev)
    flush_buf = torch.ones(flush_bytes // 4, dtype=torch.int32, device=dev) if flush_bytes else None

    def td(a, bf=False):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf else t).to(dev)

    def timed(fn, marks):
        res = []
        for r in range(runs + 2):
            if flush_buf is not None:
                torch.amax(flush_buf)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(marks)]
            fn(ev)
            torch.cuda.synchronize()
            if r >= 2:
                res.append(ev)
        return res

    # Tiny decode (fp32).
    c1 = wl.tiny_decode(poison=False)
    kp, vp = td(c1.key_pool), td(c1.value_pool)
    bt, ctx = td(c1.block_tables), td(c1.context_lens)
    cu, st = td(c1.new_cu_lens), td(c1.new_start_pos)
    kn, vn, q = td(c1.key_new), td(c1.value_new), td(c1.query)
    slots = torch.empty(c1.num_new_tokens, dtype=torch.int32, device=dev)
    out = torch.empty((c1.num_seqs, c1.num_q_heads, c1.head_dim), dtype=torch.float32, device=dev)
    ws = pkv.decode_workspace(q, c1.num_kv_heads, c1.max_blocks_per_seq)
    max_new = int(np.diff(c1.new_cu_lens).max())

    def run_c1(ev):
        ev[0].record(stream)
        pkv.slot_mapping(bt, cu, st, max_new, c1.num_blocks, out=slots)
        pkv.cache_write(kn, vn, kp, vp, slots)
        ev[1].record(stream)
        pkv.paged_attn_decode(q, kp, vp, bt, ctx, c1.scale, out=out, workspace=ws)
        ev[2].record(stream)

    evs = timed(run_c1, 3)
    att = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    whole = float(np.median([e[0].elapsed_time(e[2]) for e in evs]))
    c1_bytes, _, _ = decode_algorithmic_bytes(c1)
    gpu = {"tiny_decode": {"decode_ms": att, "run_ms": whole, "decode_bytes": c1_bytes,
                           "decode_gbs": c1_bytes / (att * 1e-3) / 1e9,
                           "decode_frac_hbm_peak": c1_bytes / (att * 1e-3) / 1e9 / HBM_PEAK_GBS}}

    # Chunked prefill equivalence (bf16).
    c2 = wl.chunked_prefill(poison=False)
    chunks = c2.notes["chunks"]
    kp2, vp2 = td(c2.key_pool, True), td(c2.value_pool, True)
    bt2 = td(c2.block_tables)
    kn2, vn2, q2 = td(c2.key_new, True), td(c2.value_new, True), td(c2.query, True)
    cus = [td(np.array([0, e - s], np.int32)) for s, e in chunks]
    offs = [td(np.array([s], np.int32)) for s, _ in chunks]
    slots2 = [torch.empty(e - s, dtype=torch.int32, device=dev) for s, e in chunks]
    out2 = torch.empty((c2.query.shape[0], c2.num_q_heads, c2.head_dim), dtype=torch.float32, device=dev)
    ws2 = pkv.prefill_workspace(q2, 1, max(e - s for s, e in chunks), c2.max_blocks_per_seq)

    def run_c2(ev):
        for i, (s, e) in enumerate(chunks):
            ev[2 * i].record(stream)
            pkv.slot_mapping(bt2, cus[i], offs[i], e - s, c2.num_blocks, out=slots2[i])
            pkv.cache_write(kn2[s:e], vn2[s:e], kp2, vp2, slots2[i])
            ev[2 * i + 1].record(stream)
            pkv.paged_attn_prefill_chunk(q2[s:e], cus[i], offs[i], kp2, vp2, bt2, e - s, c2.scale, causal=True,
                                         out=out2[s:e], workspace=ws2)
        ev[2 * len(chunks)].record(stream)

    evs = timed(run_c2, 2 * len(chunks) + 1)
    n = len(chunks)
    att = float(np.median([sum(e[2 * i + 1].elapsed_time(e[2 * i + 2]) for i in range(n)) for e in evs]))
    whole = float(np.median([e[0].elapsed_time(e[2 * n]) for e in evs]))
    fl = 0
    for s, e in chunks:
        L = e - s
        fl += 4 * c2.head_dim * c2.num_q_heads * (L * s + L * (L + 1) // 2)
    gpu["chunked_prefill"] = {"chunks": [e - s for s, e in chunks], "prefill_ms": att, "run_ms": whole,
                              "prefill_flop": fl, "prefill_tflops": fl / (att * 1e-3) / 1e12,
                              "prefill_frac_mfma_peak": fl / (att * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
    del flush_buf
    return {"gpu": gpu, "c1": c1, "c2": c2, "c1_bytes": c1_bytes, "c2_flop": fl}


def short_chunk_batch(pkv, torch, dev, flush_bytes, runs=20, num_seqs=32, chunk=32, offset=2048):
    """A batch of short prefill chunks, as a continuous-batching step with chunked prefill carries
    them: 32 prompts, each a 32-token chunk at offset 2,048 (so 2,080 cached positions each), the
    mixed step's 64/8 x 128 bf16 heads.  Median over `runs` calls, each after the flush, of the
    chunk call (HIP events); TFLOP/s over the causal algorithmic flops, GB/s over the K/V bytes the
    chunks attend to.  Synthetic N(0,1) pools with a shuffled block table."""
    hq, hkv, hd = 64, 8, 128
    ctx = offset + chunk
    nb = -(-ctx // 16)
    nblk = nb * num_seqs + 8
    g = torch.Generator(device="cpu").manual_seed(7)
    kp = torch.randn((nblk, hkv, 16, hd), generator=g).to(torch.bfloat16).to(dev)
    vp = torch.randn((nblk, hkv, 16, hd), generator=g).to(torch.bfloat16).to(dev)
    bt = torch.randperm(nblk, generator=g)[: nb * num_seqs].to(torch.int32).reshape(num_seqs, nb).contiguous().to(dev)
    q = torch.randn((num_seqs * chunk, hq, hd), generator=g).to(torch.bfloat16).to(dev)
    cu = torch.arange(0, num_seqs * chunk + 1, chunk, dtype=torch.int32).to(dev)
    offs = torch.full((num_seqs,), offset, dtype=torch.int32).to(dev)
    ws = pkv.prefill_workspace(q, num_seqs, chunk, nb)
    scale = 1.0 / math.sqrt(hd)
    out = pkv.paged_attn_prefill_chunk(q, cu, offs, kp, vp, bt, chunk, scale, causal=True, workspace=ws)
    flush_buf = torch.ones(flush_bytes // 4, dtype=torch.int32, device=dev) if flush_bytes else None
    stream = torch.cuda.current_stream(dev)
    times = []
    for r in range(runs + 2):
        if flush_buf is not None:
            torch.amax(flush_buf)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pkv.paged_attn_prefill_chunk(q, cu, offs, kp, vp, bt, chunk, scale, causal=True, out=out, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        if r >= 2:
            times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    flop = 4 * hd * hq * num_seqs * (chunk * offset + chunk * (chunk + 1) // 2)
    kv_bytes = num_seqs * ctx * 2 * hkv * hd * 2
    del flush_buf
    return {"config": f"{num_seqs} chunks of {chunk} tokens at offset {offset}, {hq}/{hkv} heads x {hd}, bf16",
            "ms": ms, "tflops": flop / (ms * 1e-3) / 1e12, "kv_gbs": kv_bytes / (ms * 1e-3) / 1e9,
            "kv_frac_hbm_peak": kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def single_sequence_decode(pkv, torch, dev, flush_bytes, runs=20, ctx=32768):
    """Decode latency of one long request: one sequence at 32,768 cached positions, the mixed
    step's 64/8 x 128 bf16 heads (134 MB of K/V).  Median over `runs` calls, each after the flush
    (HIP events); GB/s over the K/V bytes.  Synthetic N(0,1) pools with a shuffled block table."""
    hq, hkv, hd = 64, 8, 128
    nb = -(-ctx // 16)
    g = torch.Generator(device="cpu").manual_seed(11)
    kp = torch.randn((nb + 8, hkv, 16, hd), generator=g).to(torch.bfloat16).to(dev)
    vp = torch.randn((nb + 8, hkv, 16, hd), generator=g).to(torch.bfloat16).to(dev)
    bt = torch.randperm(nb + 8, generator=g)[:nb].to(torch.int32).reshape(1, nb).contiguous().to(dev)
    q = torch.randn((1, hq, hd), generator=g).to(torch.bfloat16).to(dev)
    cl = torch.full((1,), ctx, dtype=torch.int32).to(dev)
    ws = pkv.decode_workspace(q, hkv, nb)
    scale = 1.0 / math.sqrt(hd)
    out = pkv.paged_attn_decode(q, kp, vp, bt, cl, scale, workspace=ws)
    flush_buf = torch.ones(flush_bytes // 4, dtype=torch.int32, device=dev) if flush_bytes else None
    stream = torch.cuda.current_stream(dev)
    times = []
    for r in range(runs + 2):
        if flush_buf is not None:
            torch.amax(flush_buf)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pkv.paged_attn_decode(q, kp, vp, bt, cl, scale, out=out, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        if r >= 2:
            times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    kv_bytes = ctx * 2 * hkv * hd * 2
    del flush_buf
    return {"config": f"1 sequence at {ctx} positions, {hq}/{hkv} heads x {hd}, bf16", "ms": ms,
            "kv_gbs": kv_bytes / (ms * 1e-3) / 1e9, "kv_frac_hbm_peak": kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def small_configs_oracle(small):
    """The oracle on the two small configs, with every host thread BLAS offers and with one thread
    (median of 3 runs each): the tiny decode after the oracle's own cache write, and the four
    chunks of the chunked prefill, each written before its attention."""
    import oracle

    c1, c2 = small["c1"], small["c2"]

    def run_c1():
        slots = oracle.slot_mapping(c1.block_tables, c1.new_cu_lens, c1.new_start_pos, 16)
        kp, vp = oracle.cache_write(c1.key_pool, c1.value_pool, c1.key_new, c1.value_new, slots)
        oracle.decode(c1.query, kp, vp, c1.block_tables, c1.context_lens, c1.scale, "f32")

    def run_c2():
        kp, vp = c2.key_pool, c2.value_pool
        for s, e in c2.notes["chunks"]:
            cu = np.array([0, e - s], np.int32)
            off = np.array([s], np.int32)
            slots = oracle.slot_mapping(c2.block_tables, cu, off, 16)
            kp, vp = oracle.cache_write(kp, vp, c2.key_new[s:e], c2.value_new[s:e], slots)
            oracle.prefill_chunk(c2.query[s:e], cu, off, kp, vp, c2.block_tables, c2.scale, "bf16")

    def med3(fn):
        ts = []
        for _ in range(3):
            t = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t)
        return float(np.median(ts))

    def measure():
        t1, t2 = med3(run_c1), med3(run_c2)
        return {"cores": blas_threads(), "tiny_decode": {"s": t1, "gbs": small["c1_bytes"] / t1 / 1e9},
                "chunked_prefill": {"s": t2, "gflops": small["c2_flop"] / t2 / 1e9}}

    res = {"all_threads": measure()}
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        return res
    with threadpool_limits(limits=1):
        res["one_thread"] = measure()
    return res


def cpu_baseline(dec, pre, kp, vp, has_write, args, torch):
    """The fp64 oracle on this host: decode of every sequence, prefill of a row sample."""
    import oracle

    kpool = kp.cpu().view(torch.int16).numpy().view(np.uint16) if dec.dtype == "bf16" else kp.cpu().numpy()
    vpool = vp.cpu().view(torch.int16).numpy().view(np.uint16) if dec.dtype == "bf16" else vp.cpu().numpy()
    t = time.perf_counter()
    oracle.decode(dec.query, kpool, vpool, dec.block_tables, dec.context_lens, dec.scale, dec.dtype)
    dt_dec = time.perf_counter() - t
    dec_bytes, _, _ = decode_algorithmic_bytes(dec)
    res = {"value": dec_bytes / dt_dec / 1e9, "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
           "sample": f"decode of all {dec.num_seqs} sequences ({dt_dec:.1f}s)",
           "host_cpus": len(os.sched_getaffinity(0))}
    if pre is not None:
        rows = np.linspace(0, int(pre.cu_q_lens[-1]) - 1, args.cpu_sample_rows).astype(int)
        t = time.perf_counter()
        oracle.prefill_chunk(pre.query, pre.cu_q_lens, pre.chunk_offsets, kpool, vpool, pre.block_tables, pre.scale,
                             pre.dtype, rows=rows)
        dt_pre = time.perf_counter() - t
        o = int(pre.chunk_offsets[0])
        fl = 4 * pre.head_dim * pre.num_q_heads * int(sum(o + r + 1 for r in rows))
        res["prefill_gflops"] = fl / dt_pre / 1e9
        res["sample"] += f"; prefill of {len(rows)} of {int(pre.cu_q_lens[-1])} rows ({dt_pre:.1f}s)"
    return res


if __name__ == "__main__":
    main()
