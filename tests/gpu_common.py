"""Helpers shared by the GPU test modules.

Call modes.  Every attention and write entry point has two kernel instances: with a non-NULL
err_flag the kernels check each block id and slot before touching memory (the checked
instances); with err_flag == NULL they do not (the release instances, which production callers
and bench.py run, and which hold the prefill's unmasked fast gather).  GPU parity tests run in
both modes through the `mode` parameter: `new_err(dev, mode)` gives a zeroed device flag or
None, and `flag(err)` reads it (0 in release mode, where nothing can be flagged).

Reference results of the full-size mixed step (127 decode sequences and the 512-row chunk after
its cache write) are computed by the oracle once per test process and shared by every module
that checks that workload.
"""
from __future__ import annotations

import functools

import numpy as np

import oracle
from oracle import fp8 as ofp8
import workloads as wl

MODES = ("checked", "release")
MAX_ABS, MEAN_ABS = 1e-2, 1e-3


def new_err(dev, mode="checked"):
    import torch
    if mode == "checked":
        return torch.zeros(1, dtype=torch.int32, device=dev)
    if mode == "release":
        return None
    raise ValueError(mode)


def flag(err) -> int:
    return 0 if err is None else int(err.item())


def to_dev(a, dev, bf16=False):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if bf16 else t).to(dev)


def close(got, ref, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    """Element-by-element comparison at the bf16-input tolerance; returns (max-abs, mean-abs)."""
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    assert d.max() <= max_abs and d.mean() <= mean_abs, f"{what}: max-abs {d.max():.3e} mean-abs {d.mean():.3e}"
    return float(d.max()), float(d.mean())


@functools.lru_cache(maxsize=1)
def mixed_step_case():
    """The mixed-step workload with poisoned dead slots, and the oracle's pools after the chunk's
    cache write (slots from the oracle's own slot mapping)."""
    dec, pre = wl.mixed_step(poison=True)
    slots = oracle.slot_mapping(pre.block_tables, pre.new_cu_lens, pre.new_start_pos, 16)
    rk, rv = oracle.cache_write(pre.key_pool, pre.value_pool, pre.key_new, pre.value_new, slots)
    return dec, pre, slots, rk, rv


@functools.lru_cache(maxsize=1)
def mixed_step_reference():
    """Oracle outputs of the mixed step: decode of all 127 sequences and all 512 chunk rows."""
    dec, pre, _, rk, rv = mixed_step_case()
    ref_dec = oracle.decode(dec.query, rk, rv, dec.block_tables, dec.context_lens, dec.scale, "bf16")
    ref_pre = oracle.prefill_chunk(pre.query, pre.cu_q_lens, pre.chunk_offsets, rk, rv, pre.block_tables, pre.scale,
                                   "bf16")
    return ref_dec, ref_pre


def compact(codes, tables, lens, seqs):
    """The blocks the listed sequences read, packed into a small pool, and their tables rewritten
    to it (so the oracle converts only what it needs)."""
    nb = [-(-int(lens[s]) // 16) for s in seqs]
    ids = np.unique(np.concatenate([tables[s, :n] for s, n in zip(seqs, nb)]))
    where = {int(b): i for i, b in enumerate(ids)}
    t = np.full((len(seqs), max(max(nb), 1)), wl.UNUSED_BLOCK_ID, np.int32)
    for r, (s, n) in enumerate(zip(seqs, nb)):
        t[r, :n] = [where[int(b)] for b in tables[s, :n]]
    return codes[ids], t


def fp8_decode_reference(dec, rk, rv, k_scale, v_scale, batch=16):
    """Oracle decode of every sequence of `dec` over E4M3 code pools rk / rv (exact attention over
    value(code) * scale), a batch of sequences at a time to bound the fp64 copies."""
    out = np.zeros((dec.num_seqs, dec.num_q_heads, dec.head_dim))
    ctx = dec.context_lens
    for lo in range(0, dec.num_seqs, batch):
        seqs = list(range(lo, min(lo + batch, dec.num_seqs)))
        kc, t = compact(rk, dec.block_tables, ctx, seqs)
        vc, _ = compact(rv, dec.block_tables, ctx, seqs)
        out[seqs] = oracle.decode(dec.query[seqs], ofp8.dequantize(kc, k_scale), ofp8.dequantize(vc, v_scale), t,
                                  ctx[seqs], dec.scale, "bf16", kv_dtype="f64")
    return out


def fp8_prefill_reference(pre, rk, rv, k_scale, v_scale):
    """Oracle chunk attention of every row of `pre` (one sequence) over E4M3 code pools."""
    plen = pre.chunk_offsets + np.diff(pre.cu_q_lens)
    kc, t = compact(rk, pre.block_tables, plen, [0])
    vc, _ = compact(rv, pre.block_tables, plen, [0])
    return oracle.prefill_chunk(pre.query, pre.cu_q_lens, pre.chunk_offsets, ofp8.dequantize(kc, k_scale),
                                ofp8.dequantize(vc, v_scale), t, pre.scale, "bf16", kv_dtype="f64")
