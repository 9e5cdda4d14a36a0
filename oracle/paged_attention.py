"""fp64 reference for the paged-KV attention hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (cited by page title and section):

* [vLLM-internals] "Phase 17 · 04 — vLLM serving internals"
  (aiengineeringfromscratch.com), section on PagedAttention as a virtual
  memory system: the cache is cut into fixed 16-token blocks and each
  sequence has a block table from logical token positions to physical
  block ids.
* [C13-L2] "C13 推理 · 第2课 服务端:连续批处理与 PagedAttention"
  (geekvape-learning), section "改进二:PagedAttention", figure "按块表取 K"
  and its dimension table: one pool per layer of shape blocks x block size
  x D (D = KV heads x head dim); a request's keys are the pool rows gathered
  through its table (table entries are indices, the gathered rows are the
  values), and values are gathered the same way.
* [Chunked-Prefill] "Chunked Prefill" (Ultralytics glossary), sections on
  prefill/decode and on how chunked prefill works, with its PyTorch example
  and printed result: prefill stores the prompt's K/V in the cache; decode
  reads the whole cache; each chunk attends, under a causal mask over
  absolute positions, to the cached K/V of every earlier chunk plus its own
  tokens, which gives exactly the one-pass prefill result.
* [Engine-core] "第2章:推理引擎核心技术" (aiinfra.vidrealm.tech), §1.2 (the
  block-table example: logical block j holds tokens 16j..16j+15) and §1.4
  (the paged kernel loops over a request's pages, looks up each physical
  page and accumulates with an online softmax).

Readings where the pages are silent (each is listed in the design notes):

* pool layout is ``[num_blocks, Hkv, block_size, hd]``: the page's pool of
  blocks x block size x D with each block's rows grouped by KV head; a slot
  ``block*block_size + offset`` holds one token, whose row of KV head ``g`` is
  ``pool[block, g, offset]``;
* query head ``h`` uses KV head ``h // (Hq // Hkv)``;
* ``context_lens`` counts the current token, so decode attends to
  positions ``[0, ctx)``; ``ctx == 0`` gives a zero row;
* a negative slot means "skip this token"; duplicate slots are a caller
  error;
* bf16 inputs enter as the exact bf16 values, widened to fp64.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------------------------
# Representation
# ----------------------------------------------------------------------------------------------


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored elements: ``dtype`` "f32" (float32), "bf16" (uint16 bit patterns)
    or "f64" (values already exact, e.g. a dequantised FP8 pool)."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------------------------
# Addressing: block table, slot mapping, write, gather
# ----------------------------------------------------------------------------------------------


def physical_block(block_table_row: np.ndarray, position: int, block_size: int) -> int:
    """Physical block holding absolute token ``position``: the table entry of logical block
    ``position // block_size`` ([Engine-core] §1.2; [vLLM-internals] PagedAttention section)."""
    return int(block_table_row[position // block_size])


def slot_mapping(block_tables: np.ndarray, cu_new_lens: np.ndarray, start_pos: np.ndarray,
                 block_size: int) -> np.ndarray:
    """Flat pool row of every new token.

    Sequence ``s`` contributes tokens ``cu_new_lens[s] .. cu_new_lens[s+1]-1`` at absolute
    positions ``start_pos[s] + i``.  The row is ``block * block_size + position % block_size``
    where ``block`` is the physical block of that position.
    """
    total = int(cu_new_lens[-1])
    out = np.empty(total, dtype=np.int32)
    for s in range(len(start_pos)):
        for i in range(int(cu_new_lens[s + 1] - cu_new_lens[s])):
            p = int(start_pos[s]) + i
            out[int(cu_new_lens[s]) + i] = physical_block(block_tables[s], p, block_size) * block_size + p % block_size
    return out


def cache_write(key_pool: np.ndarray, value_pool: np.ndarray, key: np.ndarray, value: np.ndarray,
                slots: np.ndarray):
    """Return copies of the pools with token ``t``'s K and V rows stored at slot ``slots[t]``
    (block ``slot // block_size``, offset ``slot % block_size``, every KV head).

    The copy is exact (same storage type, bit for bit).  Negative slots are skipped.  Slots must
    be unique and inside the pool ([Chunked-Prefill]: prefill stores the K/V it computes in the
    cache, which grows block by block).
    """
    nblk, hkv, b, hd = key_pool.shape
    live = slots[slots >= 0]
    if live.size and (live.max() >= nblk * b):
        raise ValueError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slots")
    kp = key_pool.copy()
    vp = value_pool.copy()
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        kp[sl // b, :, sl % b] = key[t]
        vp[sl // b, :, sl % b] = value[t]
    return kp, vp


def gather(pool: np.ndarray, block_table_row: np.ndarray, length: int) -> np.ndarray:
    """Contiguous ``[length, Hkv, hd]`` view of one sequence's first ``length`` tokens: the pool
    blocks named by the first ``ceil(length / block_size)`` table entries, concatenated in
    logical order and cut to ``length`` rows ([C13-L2] figure "按块表取 K").  Later table entries
    are never read."""
    _, hkv, b, hd = pool.shape
    nb = -(-int(length) // b)
    if nb == 0:
        return np.zeros((0, hkv, hd), pool.dtype)
    # Block j as [token, Hkv, hd] rows: its [Hkv, token, hd] array with the two axes swapped.
    blocks = [pool[int(block_table_row[j])].transpose(1, 0, 2) for j in range(nb)]
    return np.concatenate(blocks, axis=0)[:length]


# ----------------------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------------------


def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head used by query head ``q_head``: consecutive groups of ``Hq/Hkv`` query heads share one."""
    return q_head // (num_q_heads // num_kv_heads)


def visible_keys(row: int, offset: int, chunk_len: int, causal: bool) -> int:
    """Number of keys (positions ``0 .. n-1``) chunk row ``row`` sees: its absolute position is
    ``offset + row``; causal rows see keys up to and including that position, non-causal rows see
    every key of the chunk ([Chunked-Prefill] example: lower-triangular mask shifted by the chunk
    start)."""
    return offset + row + 1 if causal else offset + chunk_len


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, visible: np.ndarray) -> np.ndarray:
    """Exact softmax attention of query rows ``q [R, hd]`` over keys ``K [n, hd]`` / values
    ``V [n, hd]``; row ``r`` sees keys ``0 .. visible[r]-1``.  A row that sees no key is zero."""
    R = q.shape[0]
    out = np.zeros((R, V.shape[1]), dtype=np.float64)
    if K.shape[0] == 0:
        return out
    x = scale * (q @ K.T)
    seen = np.arange(K.shape[0])[None, :] < np.asarray(visible)[:, None]
    x = np.where(seen, x, -np.inf)
    rows = np.asarray(visible) > 0
    m = np.max(x[rows], axis=1, keepdims=True)
    w = np.exp(x[rows] - m)
    out[rows] = (w @ V) / np.sum(w, axis=1, keepdims=True)
    return out


def decode(query: np.ndarray, key_pool: np.ndarray, value_pool: np.ndarray, block_tables: np.ndarray,
           context_lens: np.ndarray, scale: float, dtype: str, kv_dtype: str | None = None) -> np.ndarray:
    """One-token decode: ``out[s, h]`` is softmax attention of query ``(s, h)`` over the
    sequence's cached positions ``0 .. ctx_s-1`` of KV head ``kv_head_of(h)`` ([Chunked-Prefill]:
    decode reads the whole cache each step; [Engine-core] §1.4: the paged kernel walks the
    request's pages through the table).  ``kv_dtype`` is the pools' storage type when it differs
    from the query's."""
    kv_dtype = kv_dtype or dtype
    B, hq, hd = query.shape
    hkv = key_pool.shape[1]
    q = as_f64(query, dtype)
    out = np.zeros((B, hq, hd), dtype=np.float64)
    for s in range(B):
        n = int(context_lens[s])
        if n == 0:
            continue
        K = as_f64(gather(key_pool, block_tables[s], n), kv_dtype)
        V = as_f64(gather(value_pool, block_tables[s], n), kv_dtype)
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            out[s, h] = softmax_attention(q[s, h][None, :], K[:, g], V[:, g], scale, np.array([n]))[0]
    return out


def prefill_chunk(query: np.ndarray, cu_q_lens: np.ndarray, chunk_offsets: np.ndarray, key_pool: np.ndarray,
                  value_pool: np.ndarray, block_tables: np.ndarray, scale: float, dtype: str,
                  causal: bool = True, rows=None, kv_dtype: str | None = None) -> np.ndarray:
    """Chunked-prefill attention ([Chunked-Prefill], section on how chunked prefill works).

    Sequence ``s`` has chunk rows ``cu_q_lens[s] .. cu_q_lens[s+1]-1`` at absolute positions
    ``chunk_offsets[s] + i``; its cache already holds positions ``0 .. offset+L-1`` (earlier
    chunks plus this chunk).  Row ``i`` attends to ``visible_keys(i, ...)`` keys.  ``rows``
    optionally restricts the computation to a subset of packed row indices (others stay zero).
    ``kv_dtype`` is the pools' storage type when it differs from the query's.
    """
    kv_dtype = kv_dtype or dtype
    total, hq, hd = query.shape
    hkv = key_pool.shape[1]
    out = np.zeros((total, hq, hd), dtype=np.float64)
    want = None if rows is None else set(int(r) for r in rows)
    for s in range(len(chunk_offsets)):
        lo, hi = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        L = hi - lo
        if L == 0:
            continue
        o = int(chunk_offsets[s])
        idx = [i for i in range(L) if want is None or (lo + i) in want]
        if not idx:
            continue
        K = as_f64(gather(key_pool, block_tables[s], o + L), kv_dtype)
        V = as_f64(gather(value_pool, block_tables[s], o + L), kv_dtype)
        q = as_f64(query[lo:hi][idx], dtype)
        vis = np.array([visible_keys(i, o, L, causal) for i in idx])
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            out[[lo + i for i in idx], h] = softmax_attention(q[:, h], K[:, g], V[:, g], scale, vis)
    return out


# ----------------------------------------------------------------------------------------------
# Split-KV partition and combine (decode over long contexts)
# ----------------------------------------------------------------------------------------------


def decode_split_partials(query: np.ndarray, key_pool: np.ndarray, value_pool: np.ndarray,
                          block_tables: np.ndarray, context_lens: np.ndarray, scale: float, dtype: str,
                          split_tokens: int):
    """Per (sequence, query head, split) partial state over positions
    ``[p*split_tokens, min((p+1)*split_tokens, ctx))``: ``m`` = max score, ``l`` = sum of
    ``exp(score - m)``, ``o`` = sum of ``exp(score - m) * v``.  Returns a dict keyed by
    ``(s, h)`` of ``(o [n_split, hd], m [n_split], l [n_split])``."""
    B, hq, hd = query.shape
    hkv = key_pool.shape[1]
    q = as_f64(query, dtype)
    res = {}
    for s in range(B):
        n = int(context_lens[s])
        K = as_f64(gather(key_pool, block_tables[s], n), dtype)
        V = as_f64(gather(value_pool, block_tables[s], n), dtype)
        nsplit = -(-n // split_tokens)
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            o = np.zeros((nsplit, hd))
            m = np.zeros(nsplit)
            l = np.zeros(nsplit)
            for p in range(nsplit):
                a, b = p * split_tokens, min((p + 1) * split_tokens, n)
                x = scale * (K[a:b, g] @ q[s, h])
                m[p] = x.max()
                w = np.exp(x - m[p])
                l[p] = w.sum()
                o[p] = w @ V[a:b, g]
            res[(s, h)] = (o, m, l)
    return res


def combine_splits(o: np.ndarray, m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """Merge split partials: rescale each by ``exp(m_p - M)`` with ``M = max m`` and divide the
    summed outputs by the summed normalisers.  No splits gives a zero row."""
    if len(m) == 0:
        return np.zeros(o.shape[1] if o.ndim == 2 else 0)
    M = np.max(m)
    f = np.exp(m - M)
    return (f @ o) / (f @ l)
