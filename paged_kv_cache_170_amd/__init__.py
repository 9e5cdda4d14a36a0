"""Python binding of libpagedkv.so (paged-KV attention for MI355X / gfx950).

Argument marshalling only: every function checks tensor devices, dtypes and
shapes, takes raw pointers and the current HIP stream, and calls the C entry
point of the same name.  All computation happens in the HIP kernels.  The
library is loaded on import; if it has not been built, the import fails
loudly (there is no fallback).

Tensors: pools are ``[num_blocks, num_kv_heads, 16, head_dim]`` (K and V
separate, same dtype: each block's 16 token rows grouped by KV head); block tables, context lengths, slot mappings and
offsets are int32 device tensors.  FP8 pools hold E4M3 codes as
``torch.float8_e4m3fn`` (or ``torch.uint8``) tensors and come with one fp32
scale per pool (the ``*_fp8`` calls).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIB_PATH)

OK, INVALID_ARG, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP_ERROR, NO_SPACE, SCRATCH_TOO_SMALL = 0, 1, 2, 3, 4, 5, 6
NOALLOC_SCRATCH_BYTES = 64 << 20
DTYPE_F32, DTYPE_BF16, DTYPE_FP8_E4M3 = 0, 1, 2
FLAG_BAD_BLOCK, FLAG_BAD_SLOT, FLAG_BAD_LENGTH, FLAG_SYNC_TIMEOUT = 1, 2, 4, 8
BLOCK_SIZE = 16

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "pkv_status_string": (ctypes.c_char_p, [_i32]),
    "pkv_slot_mapping": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]),
    "pkv_cache_write": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "pkv_paged_gather": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                _vp, _vp]),
    "pkv_decode_split_tokens": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_prefix_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attn_decode_prefix": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                            _f32, _i32, _vp, _i32, _i32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_paged_attn_decode_prefix_fp8": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                                _i32, _f32, _f32, _f32, _vp, _i32, _i32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_paged_attn_decode": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _f32,
                                     _i32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_paged_attn_decode_noalloc": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                             _f32, _i32, _i32, _vp, _vp]),
    "pkv_paged_attn_prefill_chunk": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_prefill_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_cache_write_fp8": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                   _f32, _vp, _vp]),
    "pkv_paged_attn_decode_fp8": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                         _f32, _f32, _f32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_paged_attn_prefill_chunk_fp8": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                                _i32, _i32, _i32, _i32, _f32, _f32, _f32, _vp, _sz, _vp, _vp]),
    "pkv_paged_attn_mixed": (_i32, [_vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                    _vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32, _f32, _f32, _i32, _i32, _vp, _sz,
                                    _vp, _sz, _vp, _vp]),
    "pkv_compose_step": (_i32, [_i32, _vp, _i32, _i32, _i32, _vp, _vp]),
    "pkv_sched_state_bytes": (_sz, [_i32, _i32, _i32, _i64]),
    "pkv_sched_init": (_i32, [_vp, _sz, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _vp]),
    "pkv_sched_add_request": (_i32, [_vp, _i32, _i32, ctypes.c_double, _vp]),
    "pkv_sched_plan": (_i32, [_vp, ctypes.c_double, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "pkv_sched_complete": (_i32, [_vp, ctypes.c_double]),
    "pkv_sched_table": (_vp, [_vp]),
    "pkv_sched_num_done": (_i32, [_vp]),
    "pkv_sched_request_times": (_i32, [_vp, _i32, _vp, _vp, _vp]),
    "pkv_sched_itl": (_i64, [_vp, _vp, _i64]),
    "pkv_stream_read_probe": (_i32, [_vp, _sz, _vp, _vp]),
    "pkv_mfma_peak_probe": (_i32, [_i32, _vp, _vp]),
    "pkv_device_cu_count": (_i32, []),
    "pkv_copy_blocks": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "pkv_bm_state_bytes": (_sz, [_i32]),
    "pkv_bm_init": (_i32, [_vp, _sz, _i32, _i32, _vp]),
    "pkv_bm_add_sequence": (_i32, [_vp, _vp, _i32, _vp, _i32, _vp]),
    "pkv_bm_append": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "pkv_bm_fork": (_i32, [_vp, _vp, _i32, _vp, _i32]),
    "pkv_bm_free_sequence": (_i32, [_vp, _vp, _i32]),
    "pkv_bm_num_free": (_i32, [_vp]),
    "pkv_bm_refcount": (_i32, [_vp, _i32]),
    "pkv_bm_block_hash": (ctypes.c_uint64, [_vp, _i32]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class PagedKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


def status_string(status: int) -> str:
    return _lib.pkv_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise PagedKVError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DTYPE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need_fp8_pools(key_pool: torch.Tensor, value_pool: torch.Tensor):
    if _dtype_code(key_pool) != DTYPE_FP8_E4M3:
        raise ValueError("FP8 pools must be float8_e4m3fn (or uint8 code) tensors")
    return _pool_dims(key_pool, value_pool)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("every tensor must be on the GPU")


def _need_i32(*ts):
    for t in ts:
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError("index tensors must be contiguous int32")


def _pool_dims(key_pool: torch.Tensor, value_pool: torch.Tensor):
    if key_pool.shape != value_pool.shape or key_pool.dtype != value_pool.dtype or key_pool.dim() != 4:
        raise ValueError("key_pool and value_pool must both be [num_blocks, num_kv_heads, 16, head_dim], same dtype")
    if not (key_pool.is_contiguous() and value_pool.is_contiguous()):
        raise ValueError("pools must be contiguous")
    nblk, hkv, bs, hd = key_pool.shape
    return nblk, bs, hkv, hd


def slot_mapping(block_tables: torch.Tensor, cu_new_lens: torch.Tensor, start_pos: torch.Tensor, max_new_len: int,
                 num_blocks: int, err_flag: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 total: int | None = None) -> torch.Tensor:
    """Slot (flat pool row) of each new token; see pkv_slot_mapping."""
    _need_gpu(block_tables, cu_new_lens, start_pos, err_flag)
    _need_i32(block_tables, cu_new_lens, start_pos, err_flag)
    num_seqs = start_pos.shape[0]
    if out is None:
        if total is None:
            total = int(cu_new_lens[-1].item())
        out = torch.empty(total, dtype=torch.int32, device=block_tables.device)
    _check(_lib.pkv_slot_mapping(_ptr(out), _ptr(block_tables), block_tables.shape[1], _ptr(cu_new_lens),
                                 _ptr(start_pos), num_seqs, int(max_new_len), int(num_blocks), BLOCK_SIZE,
                                 _ptr(err_flag), _stream(block_tables.device)), "pkv_slot_mapping")
    return out


def cache_write(key: torch.Tensor, value: torch.Tensor, key_pool: torch.Tensor, value_pool: torch.Tensor,
                slot_mapping: torch.Tensor, err_flag: torch.Tensor | None = None) -> None:
    """Copy token rows key[t], value[t] into pool slots slot_mapping[t] (negative slots skipped)."""
    _need_gpu(key, value, key_pool, value_pool, slot_mapping, err_flag)
    _need_i32(slot_mapping, err_flag)
    nblk, bs, hkv, hd = _pool_dims(key_pool, value_pool)
    for t in (key, value):
        if t.dtype != key_pool.dtype or t.dim() != 3 or tuple(t.shape[1:]) != (hkv, hd):
            raise ValueError("key/value must be [T, num_kv_heads, head_dim] in the pool dtype")
        if t.stride(2) != 1 or t.stride(1) != hd:
            raise ValueError("key/value rows must be contiguous")
    T = key.shape[0]
    if value.shape[0] != T or slot_mapping.shape[0] < T:
        raise ValueError("token counts differ")
    _check(_lib.pkv_cache_write(_ptr(key), _ptr(value), key.stride(0), value.stride(0), _ptr(key_pool),
                                _ptr(value_pool), _ptr(slot_mapping), T, nblk, hkv, hd, bs,
                                _dtype_code(key_pool), _ptr(err_flag), _stream(key.device)), "pkv_cache_write")


def cache_write_fp8(key: torch.Tensor, value: torch.Tensor, key_pool: torch.Tensor, value_pool: torch.Tensor,
                    slot_mapping: torch.Tensor, k_scale: float, v_scale: float,
                    err_flag: torch.Tensor | None = None) -> None:
    """Quantise token rows key[t], value[t] (bf16 or fp32) into E4M3 pool slots slot_mapping[t];
    see pkv_cache_write_fp8."""
    _need_gpu(key, value, key_pool, value_pool, slot_mapping, err_flag)
    _need_i32(slot_mapping, err_flag)
    nblk, bs, hkv, hd = _need_fp8_pools(key_pool, value_pool)
    for t in (key, value):
        if t.dtype not in (torch.float32, torch.bfloat16) or t.dim() != 3 or tuple(t.shape[1:]) != (hkv, hd):
            raise ValueError("key/value must be [T, num_kv_heads, head_dim] in bf16 or fp32")
        if t.stride(2) != 1 or t.stride(1) != hd:
            raise ValueError("key/value rows must be contiguous")
    if key.dtype != value.dtype:
        raise ValueError("key and value must have the same dtype")
    T = key.shape[0]
    if value.shape[0] != T or slot_mapping.shape[0] < T:
        raise ValueError("token counts differ")
    _check(_lib.pkv_cache_write_fp8(_ptr(key), _ptr(value), key.stride(0), value.stride(0), _ptr(key_pool),
                                    _ptr(value_pool), _ptr(slot_mapping), T, nblk, hkv, hd, bs, _dtype_code(key),
                                    float(k_scale), float(v_scale), _ptr(err_flag), _stream(key.device)),
           "pkv_cache_write_fp8")


def copy_blocks(key_pool: torch.Tensor, value_pool: torch.Tensor, src: torch.Tensor, dst: torch.Tensor,
                err_flag: torch.Tensor | None = None) -> None:
    """Copy whole blocks src[i] -> dst[i] in both pools (copy-on-write); see pkv_copy_blocks."""
    _need_gpu(key_pool, value_pool, src, dst, err_flag)
    _need_i32(src, dst, err_flag)
    nblk, bs, hkv, hd = _pool_dims(key_pool, value_pool)
    if src.shape != dst.shape or src.dim() != 1:
        raise ValueError("src and dst must be 1-D and the same length")
    _check(_lib.pkv_copy_blocks(_ptr(key_pool), _ptr(value_pool), _ptr(src), _ptr(dst), src.shape[0], nblk, hkv, hd,
                                bs, _dtype_code(key_pool), _ptr(err_flag), _stream(key_pool.device)),
           "pkv_copy_blocks")


def compose_step(num_decode: int, prefill_remaining, token_budget: int, max_chunk: int = 0):
    """Token-budget composition of one step (decode tokens first, then prompt chunks in queue
    order); returns (decode tokens scheduled, chunk length per waiting prompt).  Host code."""
    import numpy as np
    rem = np.ascontiguousarray(prefill_remaining, dtype=np.int32)
    chunks = np.zeros(rem.shape[0], dtype=np.int32)
    nd = ctypes.c_int32(0)
    _check(_lib.pkv_compose_step(int(num_decode), ctypes.c_void_p(rem.ctypes.data) if rem.size else None,
                                 rem.shape[0], int(token_budget), int(max_chunk),
                                 ctypes.c_void_p(chunks.ctypes.data) if rem.size else None, ctypes.byref(nd)),
           "pkv_compose_step")
    return nd.value, chunks


class BlockManager:
    """Host-side block manager over one pool (see the pkv_bm_* calls): block tables are rows of a
    caller-owned int32 numpy array [max_seqs, max_blocks]; the state is a numpy buffer."""

    def __init__(self, num_blocks: int, free_order=None):
        import numpy as np
        self._np = np
        n = int(_lib.pkv_bm_state_bytes(num_blocks))
        if n == 0:
            raise ValueError("bad num_blocks")
        self._state = np.zeros((n + 7) // 8, dtype=np.uint64)
        fo = None
        if free_order is not None:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            if fo.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
        self.num_blocks = num_blocks
        _check(_lib.pkv_bm_init(self._sp(), n, num_blocks, BLOCK_SIZE, self._ap(fo)), "pkv_bm_init")

    def _sp(self):
        return ctypes.c_void_p(self._state.ctypes.data)

    @staticmethod
    def _ap(a):
        return None if a is None else ctypes.c_void_p(a.ctypes.data)

    def _row(self, row):
        if row.dtype != self._np.int32 or not row.flags["C_CONTIGUOUS"] or row.ndim != 1:
            raise ValueError("table rows must be contiguous 1-D int32 numpy arrays")
        return row

    def add_sequence(self, tokens, table_row) -> int:
        """Fill table_row for a new prompt; returns the number of cached (reused) leading tokens."""
        tok = self._np.ascontiguousarray(tokens, dtype=self._np.int32)
        row = self._row(table_row)
        cached = ctypes.c_int32(0)
        _check(_lib.pkv_bm_add_sequence(self._sp(), self._ap(tok), tok.shape[0], self._ap(row), row.shape[0],
                                        ctypes.byref(cached)), "pkv_bm_add_sequence")
        return cached.value

    def append(self, table_row, ctx: int, num_new: int):
        """Extend a sequence; returns (slots, copy pairs as an [n, 2] int32 array)."""
        row = self._row(table_row)
        slots = self._np.empty(max(num_new, 1), dtype=self._np.int32)
        cs, cd, nc = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
        _check(_lib.pkv_bm_append(self._sp(), self._ap(row), row.shape[0], int(ctx), int(num_new), self._ap(slots),
                                  ctypes.byref(cs), ctypes.byref(cd), ctypes.byref(nc)), "pkv_bm_append")
        pairs = self._np.array([[cs.value, cd.value]], dtype=self._np.int32)[: nc.value]
        return slots[:num_new], pairs

    def fork(self, parent_row, ctx: int, child_row) -> None:
        _check(_lib.pkv_bm_fork(self._sp(), self._ap(self._row(parent_row)), int(ctx), self._ap(self._row(child_row)),
                                child_row.shape[0]), "pkv_bm_fork")

    def free_sequence(self, table_row, ctx: int) -> None:
        _check(_lib.pkv_bm_free_sequence(self._sp(), self._ap(self._row(table_row)), int(ctx)),
               "pkv_bm_free_sequence")

    def num_free(self) -> int:
        return int(_lib.pkv_bm_num_free(self._sp()))

    def refcount(self, block: int) -> int:
        return int(_lib.pkv_bm_refcount(self._sp(), int(block)))

    def block_hash(self, block: int) -> int:
        return int(_lib.pkv_bm_block_hash(self._sp(), int(block)))


SCHED_NAIVE, SCHED_STATIC, SCHED_CONTINUOUS, SCHED_CHUNKED = 0, 1, 2, 3


class Scheduler:
    """Iteration-level scheduler over synthetic requests (see the pkv_sched_* calls); host code.
    Block-table rows come from `block_manager` (a BlockManager over the pool the kernels use)."""

    def __init__(self, mode: int, max_requests: int, max_running: int, max_blocks: int, block_manager: BlockManager,
                 token_budget: int = 0, max_chunk: int = 0, max_itl_samples: int = 1 << 20):
        import numpy as np
        self._np = np
        n = int(_lib.pkv_sched_state_bytes(max_requests, max_running, max_blocks, max_itl_samples))
        if n == 0:
            raise ValueError("bad scheduler sizes")
        self._state = np.zeros((n + 7) // 8, dtype=np.uint64)
        self._bm = block_manager  # kept alive: the scheduler holds a pointer to its state
        self.max_running, self.max_blocks = max_running, max_blocks
        _check(_lib.pkv_sched_init(self._sp(), n, int(mode), max_requests, max_running, max_blocks, max_itl_samples,
                                   int(token_budget), int(max_chunk), block_manager._sp()), "pkv_sched_init")
        ptr = _lib.pkv_sched_table(self._sp())
        self.table = np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctypes.c_int32)),
                                           shape=(max_running, max_blocks))
        mr = max_running
        self._out = {k: np.zeros(mr, dtype=np.int32) for k in ("dec_row", "dec_ctx", "chunk_row", "chunk_offset",
                                                                "chunk_len")}

    def _sp(self):
        return ctypes.c_void_p(self._state.ctypes.data)

    @staticmethod
    def _ap(a):
        return ctypes.c_void_p(a.ctypes.data)

    def add_request(self, prompt_len: int, output_len: int, arrival: float) -> int:
        rid = ctypes.c_int32(0)
        _check(_lib.pkv_sched_add_request(self._sp(), int(prompt_len), int(output_len), float(arrival),
                                          ctypes.byref(rid)), "pkv_sched_add_request")
        return rid.value

    def plan(self, now: float) -> dict:
        """The step starting at `now`: decode (row, ctx) and chunk (row, offset, len) arrays."""
        nd, nc, nxt = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_double(0)
        o = self._out
        _check(_lib.pkv_sched_plan(self._sp(), float(now), ctypes.byref(nd), self._ap(o["dec_row"]),
                                   self._ap(o["dec_ctx"]), ctypes.byref(nc), self._ap(o["chunk_row"]),
                                   self._ap(o["chunk_offset"]), self._ap(o["chunk_len"]), ctypes.byref(nxt)),
               "pkv_sched_plan")
        d, c = nd.value, nc.value
        return {"dec_row": o["dec_row"][:d].copy(), "dec_ctx": o["dec_ctx"][:d].copy(),
                "chunk_row": o["chunk_row"][:c].copy(), "chunk_offset": o["chunk_offset"][:c].copy(),
                "chunk_len": o["chunk_len"][:c].copy(), "next_arrival": nxt.value}

    def complete(self, now: float) -> None:
        _check(_lib.pkv_sched_complete(self._sp(), float(now)), "pkv_sched_complete")

    def num_done(self) -> int:
        return int(_lib.pkv_sched_num_done(self._sp()))

    def request_times(self, rid: int):
        a, f, e = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
        _check(_lib.pkv_sched_request_times(self._sp(), int(rid), ctypes.byref(a), ctypes.byref(f), ctypes.byref(e)),
               "pkv_sched_request_times")
        return a.value, f.value, e.value

    def itl(self):
        n = int(_lib.pkv_sched_itl(self._sp(), None, 0))
        out = self._np.zeros(max(n, 1), dtype=self._np.float64)
        _lib.pkv_sched_itl(self._sp(), self._ap(out), n)
        return out[:n]


def paged_gather(key_pool: torch.Tensor, value_pool: torch.Tensor, block_tables: torch.Tensor,
                 lengths: torch.Tensor, cu_out: torch.Tensor, max_len: int, total: int,
                 err_flag: torch.Tensor | None = None):
    """Contiguous copies of each sequence's first lengths[s] rows (diagnostic of the block indexing)."""
    _need_gpu(key_pool, value_pool, block_tables, lengths, cu_out, err_flag)
    _need_i32(block_tables, lengths, cu_out, err_flag)
    nblk, bs, hkv, hd = _pool_dims(key_pool, value_pool)
    kout = torch.empty((total, hkv, hd), dtype=key_pool.dtype, device=key_pool.device)
    vout = torch.empty_like(kout)
    _check(_lib.pkv_paged_gather(_ptr(kout), _ptr(vout), _ptr(key_pool), _ptr(value_pool), _ptr(block_tables),
                                 block_tables.shape[1], _ptr(lengths), _ptr(cu_out), lengths.shape[0], int(max_len),
                                 nblk, hkv, hd, bs, _dtype_code(key_pool), _ptr(err_flag),
                                 _stream(key_pool.device)), "pkv_paged_gather")
    return kout, vout


def decode_split_tokens(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                        max_blocks_per_seq: int) -> int:
    return int(_lib.pkv_decode_split_tokens(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_blocks_per_seq: int, split_tokens: int = 0) -> int:
    return int(_lib.pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                               split_tokens))


def decode_workspace(query: torch.Tensor, num_kv_heads: int, max_blocks_per_seq: int,
                     split_tokens: int = 0) -> torch.Tensor:
    """Allocate a decode workspace for these shapes (a byte tensor on the query's device)."""
    n = decode_workspace_bytes(query.shape[0], query.shape[1], num_kv_heads, query.shape[2], max_blocks_per_seq,
                               split_tokens)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=query.device)


def paged_attn_decode(query: torch.Tensor, key_pool: torch.Tensor, value_pool: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                      out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                      workspace: torch.Tensor | None = None, split_tokens: int = 0,
                      err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """One-token decode over the paged cache; see pkv_paged_attn_decode."""
    _need_gpu(query, key_pool, value_pool, block_tables, context_lens, out, workspace, err_flag)
    _need_i32(block_tables, context_lens, err_flag)
    nblk, bs, hkv, hd = _pool_dims(key_pool, value_pool)
    if query.dim() != 3 or query.shape[2] != hd or query.dtype != key_pool.dtype or not query.is_contiguous():
        raise ValueError("query must be contiguous [num_seqs, num_q_heads, head_dim] in the pool dtype")
    B, hq, _ = query.shape
    if context_lens.shape[0] != B or block_tables.shape[0] != B:
        raise ValueError("batch sizes differ")
    if out is None:
        out = torch.empty((B, hq, hd), dtype=out_dtype, device=query.device)
    elif not out.is_contiguous() or tuple(out.shape) != (B, hq, hd):
        raise ValueError("out must be contiguous [num_seqs, num_q_heads, head_dim]")
    if workspace is None:
        workspace = decode_workspace(query, hkv, block_tables.shape[1], split_tokens)
    _check(_lib.pkv_paged_attn_decode(_ptr(out), _dtype_code(out), _ptr(query), _ptr(key_pool), _ptr(value_pool),
                                      _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, hq, hkv, hd,
                                      nblk, float(scale), _dtype_code(key_pool), int(split_tokens),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _ptr(err_flag), _stream(query.device)), "pkv_paged_attn_decode")
    return out


def paged_attn_decode_noalloc(query: torch.Tensor, key_pool: torch.Tensor, value_pool: torch.Tensor,
                              block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                              out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                              split_tokens: int = 0, err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """pkv_paged_attn_decode with the library's static scratch instead of a workspace; see
    pkv_paged_attn_decode_noalloc.  Pass `out` to keep the call free of allocations (only the
    output is allocated here when it is not given)."""
    _need_gpu(query, key_pool, value_pool, block_tables, context_lens, out, err_flag)
    _need_i32(block_tables, context_lens, err_flag)
    nblk, bs, hkv, hd = _pool_dims(key_pool, value_pool)
    if query.dim() != 3 or query.shape[2] != hd or query.dtype != key_pool.dtype or not query.is_contiguous():
        raise ValueError("query must be contiguous [num_seqs, num_q_heads, head_dim] in the pool dtype")
    B, hq, _ = query.shape
    if context_lens.shape[0] != B or block_tables.shape[0] != B:
        raise ValueError("batch sizes differ")
    if out is None:
        out = torch.empty((B, hq, hd), dtype=out_dtype, device=query.device)
    elif not out.is_contiguous() or tuple(out.shape) != (B, hq, hd):
        raise ValueError("out must be contiguous [num_seqs, num_q_heads, head_dim]")
    _check(_lib.pkv_paged_attn_decode_noalloc(_ptr(out), _dtype_code(out), _ptr(query), _ptr(key_pool),
                                              _ptr(value_pool), _ptr(block_tables), block_tables.shape[1],
                                              _ptr(context_lens), B, hq, hkv, hd, nblk, float(scale),
                                              _dtype_code(key_pool), int(split_tokens), _ptr(err_flag),
                                              _stream(query.device)), "pkv_paged_attn_decode_noalloc")
    return out


def decode_prefix_workspace(query: torch.Tensor, num_kv_heads: int, max_blocks_per_seq: int,
                            split_tokens: int = 0) -> torch.Tensor:
    """Allocate a workspace for pkv_paged_attn_decode_prefix (a byte tensor on the query's device)."""
    n = int(_lib.pkv_decode_prefix_workspace_bytes(query.shape[0], query.shape[1], num_kv_heads, query.shape[2],
                                                   max_blocks_per_seq, split_tokens))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=query.device)


def paged_attn_decode_prefix(query: torch.Tensor, key_pool: torch.Tensor, value_pool: torch.Tensor,
                             block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                             prefix_members: torch.Tensor, prefix_blocks: int, out: torch.Tensor | None = None,
                             out_dtype: torch.dtype = torch.float32, workspace: torch.Tensor | None = None,
                             split_tokens: int = 0, err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """Decode with a shared prefix attended once per KV head; see pkv_paged_attn_decode_prefix."""
    _need_gpu(query, key_pool, value_pool, block_tables, context_lens, prefix_members, out, workspace, err_flag)
    _need_i32(block_tables, context_lens, prefix_members, err_flag)
    if prefix_members.dim() != 1 or not prefix_members.is_contiguous():
        raise ValueError("prefix_members must be a contiguous 1-D int32 tensor")
    nblk, bs, hkv, hd = _pool_dims(key_pool, value_pool)
    if query.dim() != 3 or query.shape[2] != hd or query.dtype != key_pool.dtype or not query.is_contiguous():
        raise ValueError("query must be contiguous [num_seqs, num_q_heads, head_dim] in the pool dtype")
    B, hq, _ = query.shape
    if context_lens.shape[0] != B or block_tables.shape[0] != B:
        raise ValueError("batch sizes differ")
    if out is None:
        out = torch.empty((B, hq, hd), dtype=out_dtype, device=query.device)
    elif not out.is_contiguous() or tuple(out.shape) != (B, hq, hd):
        raise ValueError("out must be contiguous [num_seqs, num_q_heads, head_dim]")
    if workspace is None:
        workspace = decode_prefix_workspace(query, hkv, block_tables.shape[1], split_tokens)
    _check(_lib.pkv_paged_attn_decode_prefix(_ptr(out), _dtype_code(out), _ptr(query), _ptr(key_pool),
                                             _ptr(value_pool), _ptr(block_tables), block_tables.shape[1],
                                             _ptr(context_lens), B, hq, hkv, hd, nblk, float(scale),
                                             _dtype_code(key_pool), _ptr(prefix_members), prefix_members.shape[0],
                                             int(prefix_blocks), int(split_tokens), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _ptr(err_flag),
                                             _stream(query.device)), "pkv_paged_attn_decode_prefix")
    return out


def paged_attn_decode_prefix_fp8(query: torch.Tensor, key_pool: torch.Tensor, value_pool: torch.Tensor,
                                 block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, k_scale: float,
                                 v_scale: float, prefix_members: torch.Tensor, prefix_blocks: int,
                                 out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                                 workspace: torch.Tensor | None = None, split_tokens: int = 0,
                                 err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """Shared-prefix decode over E4M3 pools; see pkv_paged_attn_decode_prefix_fp8."""
    _need_gpu(query, key_pool, value_pool, block_tables, context_lens, prefix_members, out, workspace, err_flag)
    _need_i32(block_tables, context_lens, prefix_members, err_flag)
    if prefix_members.dim() != 1 or not prefix_members.is_contiguous():
        raise ValueError("prefix_members must be a contiguous 1-D int32 tensor")
    nblk, bs, hkv, hd = _need_fp8_pools(key_pool, value_pool)
    if query.dim() != 3 or query.shape[2] != hd or query.dtype != torch.bfloat16 or not query.is_contiguous():
        raise ValueError("query must be contiguous bf16 [num_seqs, num_q_heads, head_dim]")
    B, hq, _ = query.shape
    if context_lens.shape[0] != B or block_tables.shape[0] != B:
        raise ValueError("batch sizes differ")
    if out is None:
        out = torch.empty((B, hq, hd), dtype=out_dtype, device=query.device)
    elif not out.is_contiguous() or tuple(out.shape) != (B, hq, hd):
        raise ValueError("out must be contiguous [num_seqs, num_q_heads, head_dim]")
    if workspace is None:
        workspace = decode_prefix_workspace(query, hkv, block_tables.shape[1], split_tokens)
    _check(_lib.pkv_paged_attn_decode_prefix_fp8(_ptr(out), _dtype_code(out), _ptr(query), _ptr(key_pool),
                                                 _ptr(value_pool), _ptr(block_tables), block_tables.shape[1],
                                                 _ptr(context_lens), B, hq, hkv, hd, nblk, float(scale),
                                                 float(k_scale), float(v_scale), _ptr(prefix_members),
                                                 prefix_members.shape[0], int(prefix_blocks), int(split_tokens),
                                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                 _ptr(err_flag), _stream(query.device)),
           "pkv_paged_attn_decode_prefix_fp8")
    return out


def paged_attn_decode_fp8(query: torch.Tensor, key_pool: torch.Tensor, value_pool: torch.Tensor,
                          block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, k_scale: float,
                          v_scale: float, out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                          workspace: torch.Tensor | None = None, split_tokens: int = 0,
                          err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """One-token decode over E4M3 pools with per-pool scales; see pkv_paged_attn_decode_fp8."""
    _need_gpu(query, key_pool, value_pool, block_tables, context_lens, out, workspace, err_flag)
    _need_i32(block_tables, context_lens, err_flag)
    nblk, bs, hkv, hd = _need_fp8_pools(key_pool, value_pool)
    if query.dim() != 3 or query.shape[2] != hd or query.dtype != torch.bfloat16 or not query.is_contiguous():
        raise ValueError("query must be contiguous bf16 [num_seqs, num_q_heads, head_dim]")
    B, hq, _ = query.shape
    if context_lens.shape[0] != B or block_tables.shape[0] != B:
        raise ValueError("batch sizes differ")
    if out is None:
        out = torch.empty((B, hq, hd), dtype=out_dtype, device=query.device)
    elif not out.is_contiguous() or tuple(out.shape) != (B, hq, hd):
        raise ValueError("out must be contiguous [num_seqs, num_q_heads, head_dim]")
    if workspace is None:
        workspace = decode_workspace(query, hkv, block_tables.shape[1], split_tokens)
    _check(_lib.pkv_paged_attn_decode_fp8(_ptr(out), _dtype_code(out), _ptr(query), _ptr(key_pool),
                                          _ptr(value_pool), _ptr(block_tables), block_tables.shape[1],
                                          _ptr(context_lens), B, hq, hkv, hd, nblk, float(scale), float(k_scale),
                                          float(v_scale), int(split_tokens), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _ptr(err_flag),
                                          _stream(query.device)), "pkv_paged_attn_decode_fp8")
    return out


def prefill_workspace_bytes(num_seqs: int, max_q_len: int, num_q_heads: int, head_dim: int,
                            max_blocks_per_seq: int) -> int:
    return int(_lib.pkv_prefill_workspace_bytes(num_seqs, max_q_len, num_q_heads, head_dim, max_blocks_per_seq))


def prefill_workspace(query: torch.Tensor, num_seqs: int, max_q_len: int, max_blocks_per_seq: int):
    """Allocate the chunked-prefill workspace for these shapes (None when none is needed)."""
    n = prefill_workspace_bytes(num_seqs, max_q_len, query.shape[1], query.shape[2], max_blocks_per_seq)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=query.device)


def _ws_args(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def paged_attn_prefill_chunk(query: torch.Tensor, cu_q_lens: torch.Tensor, chunk_offsets: torch.Tensor,
                             key_pool: torch.Tensor, value_pool: torch.Tensor, block_tables: torch.Tensor,
                             max_q_len: int, scale: float, causal: bool = True, out: torch.Tensor | None = None,
                             out_dtype: torch.dtype = torch.float32, workspace: torch.Tensor | None = None,
                             err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """Chunked-prefill attention over the paged cache; see pkv_paged_attn_prefill_chunk."""
    _need_gpu(query, cu_q_lens, chunk_offsets, key_pool, value_pool, block_tables, out, workspace, err_flag)
    _need_i32(cu_q_lens, chunk_offsets, block_tables, err_flag)
    nblk, bs, hkv, hd = _pool_dims(key_pool, value_pool)
    if query.dim() != 3 or query.shape[2] != hd or query.dtype != key_pool.dtype or not query.is_contiguous():
        raise ValueError("query must be contiguous [rows, num_q_heads, head_dim] in the pool dtype")
    rows, hq, _ = query.shape
    num_seqs = chunk_offsets.shape[0]
    if cu_q_lens.shape[0] != num_seqs + 1 or block_tables.shape[0] != num_seqs:
        raise ValueError("batch sizes differ")
    if out is None:
        out = torch.empty((rows, hq, hd), dtype=out_dtype, device=query.device)
    elif not out.is_contiguous() or tuple(out.shape) != (rows, hq, hd):
        raise ValueError("out must be contiguous [rows, num_q_heads, head_dim]")
    if workspace is None:
        workspace = prefill_workspace(query, num_seqs, int(max_q_len), block_tables.shape[1])
    _check(_lib.pkv_paged_attn_prefill_chunk(_ptr(out), _dtype_code(out), _ptr(query), _ptr(cu_q_lens),
                                             _ptr(chunk_offsets), _ptr(key_pool), _ptr(value_pool),
                                             _ptr(block_tables), block_tables.shape[1], num_seqs, int(max_q_len), hq,
                                             hkv, hd, nblk, int(bool(causal)), float(scale), _dtype_code(key_pool),
                                             *_ws_args(workspace), _ptr(err_flag), _stream(query.device)),
           "pkv_paged_attn_prefill_chunk")
    return out


def paged_attn_prefill_chunk_fp8(query: torch.Tensor, cu_q_lens: torch.Tensor, chunk_offsets: torch.Tensor,
                                 key_pool: torch.Tensor, value_pool: torch.Tensor, block_tables: torch.Tensor,
                                 max_q_len: int, scale: float, k_scale: float, v_scale: float, causal: bool = True,
                                 out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                                 workspace: torch.Tensor | None = None,
                                 err_flag: torch.Tensor | None = None) -> torch.Tensor:
    """Chunked-prefill attention over E4M3 pools with per-pool scales; see
    pkv_paged_attn_prefill_chunk_fp8."""
    _need_gpu(query, cu_q_lens, chunk_offsets, key_pool, value_pool, block_tables, out, err_flag)
    _need_i32(cu_q_lens, chunk_offsets, block_tables, err_flag)
    nblk, bs, hkv, hd = _need_fp8_pools(key_pool, value_pool)
    if query.dim() != 3 or query.shape[2] != hd or query.dtype != torch.bfloat16 or not query.is_contiguous():
        raise ValueError("query must be contiguous bf16 [rows, num_q_heads, head_dim]")
    rows, hq, _ = query.shape
    num_seqs = chunk_offsets.shape[0]
    if cu_q_lens.shape[0] != num_seqs + 1 or block_tables.shape[0] != num_seqs:
        raise ValueError("batch sizes differ")
    if out is None:
        out = torch.empty((rows, hq, hd), dtype=out_dtype, device=query.device)
    elif not out.is_contiguous() or tuple(out.shape) != (rows, hq, hd):
        raise ValueError("out must be contiguous [rows, num_q_heads, head_dim]")
    if workspace is None:
        workspace = prefill_workspace(query, num_seqs, int(max_q_len), block_tables.shape[1])
    _check(_lib.pkv_paged_attn_prefill_chunk_fp8(_ptr(out), _dtype_code(out), _ptr(query), _ptr(cu_q_lens),
                                                 _ptr(chunk_offsets), _ptr(key_pool), _ptr(value_pool),
                                                 _ptr(block_tables), block_tables.shape[1], num_seqs,
                                                 int(max_q_len), hq, hkv, hd, nblk, int(bool(causal)), float(scale),
                                                 float(k_scale), float(v_scale), *_ws_args(workspace), _ptr(err_flag),
                                                 _stream(query.device)), "pkv_paged_attn_prefill_chunk_fp8")
    return out


def paged_attn_mixed(key_pool: torch.Tensor, value_pool: torch.Tensor, scale: float,
                     dec_query: torch.Tensor | None = None, dec_block_tables: torch.Tensor | None = None,
                     context_lens: torch.Tensor | None = None, pre_query: torch.Tensor | None = None,
                     cu_q_lens: torch.Tensor | None = None, chunk_offsets: torch.Tensor | None = None,
                     pre_block_tables: torch.Tensor | None = None, max_q_len: int = 0, causal: bool = True,
                     k_scale: float = 1.0, v_scale: float = 1.0, dec_out: torch.Tensor | None = None,
                     pre_out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                     workspace: torch.Tensor | None = None, pre_workspace: torch.Tensor | None = None,
                     split_tokens: int = 0, err_flag: torch.Tensor | None = None):
    """Decode tokens and prefill chunks of one step in one fused launch; see pkv_paged_attn_mixed.
    Returns (decode output or None, prefill output or None).  bf16 or E4M3 pools (with scales)."""
    _need_gpu(key_pool, value_pool, dec_query, dec_block_tables, context_lens, pre_query, cu_q_lens, chunk_offsets,
              pre_block_tables, dec_out, pre_out, workspace, err_flag)
    _need_i32(dec_block_tables, context_lens, cu_q_lens, chunk_offsets, pre_block_tables, err_flag)
    nblk, bs, hkv, hd = _pool_dims(key_pool, value_pool)
    code = _dtype_code(key_pool)
    if code not in (DTYPE_BF16, DTYPE_FP8_E4M3):
        raise ValueError("pools must be bf16 or FP8 E4M3")
    hq = None
    nd = 0
    if dec_query is not None:
        if dec_query.dim() != 3 or dec_query.shape[2] != hd or dec_query.dtype != torch.bfloat16 \
                or not dec_query.is_contiguous():
            raise ValueError("dec_query must be contiguous bf16 [num_seqs, num_q_heads, head_dim]")
        nd, hq = dec_query.shape[0], dec_query.shape[1]
        if context_lens.shape[0] != nd or dec_block_tables.shape[0] != nd:
            raise ValueError("decode batch sizes differ")
        if dec_out is None:
            dec_out = torch.empty((nd, hq, hd), dtype=out_dtype, device=dec_query.device)
        if workspace is None:
            workspace = decode_workspace(dec_query, hkv, dec_block_tables.shape[1], split_tokens)
    npre = 0
    if pre_query is not None:
        if pre_query.dim() != 3 or pre_query.shape[2] != hd or pre_query.dtype != torch.bfloat16 \
                or not pre_query.is_contiguous():
            raise ValueError("pre_query must be contiguous bf16 [rows, num_q_heads, head_dim]")
        if hq is not None and pre_query.shape[1] != hq:
            raise ValueError("decode and prefill queries must have the same head count")
        hq = pre_query.shape[1]
        npre = chunk_offsets.shape[0]
        if cu_q_lens.shape[0] != npre + 1 or pre_block_tables.shape[0] != npre:
            raise ValueError("prefill batch sizes differ")
        if pre_out is None:
            pre_out = torch.empty((pre_query.shape[0], hq, hd), dtype=out_dtype, device=pre_query.device)
        if pre_workspace is None:
            pre_workspace = prefill_workspace(pre_query, npre, int(max_q_len), pre_block_tables.shape[1])
    if hq is None:
        return None, None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    out_code = _dtype_code(dec_out if dec_out is not None else pre_out)
    _check(_lib.pkv_paged_attn_mixed(_ptr(dec_out), _ptr(dec_query), _ptr(dec_block_tables),
                                     0 if dec_block_tables is None else dec_block_tables.shape[1], _ptr(context_lens),
                                     nd, _ptr(pre_out), _ptr(pre_query), _ptr(cu_q_lens), _ptr(chunk_offsets),
                                     _ptr(pre_block_tables), 0 if pre_block_tables is None else pre_block_tables.shape[1],
                                     npre, int(max_q_len), int(bool(causal)), _ptr(key_pool), _ptr(value_pool), nblk, hq,
                                     hkv, hd, float(scale), code, float(k_scale), float(v_scale), out_code,
                                     int(split_tokens), _ptr(workspace), ws_bytes, *_ws_args(pre_workspace),
                                     _ptr(err_flag), _stream(key_pool.device)), "pkv_paged_attn_mixed")
    return dec_out, pre_out


def mfma_peak_probe(iters: int, sink: torch.Tensor) -> int:
    """Pure bf16 MFMA work on every SIMD (matrix-core reference); returns the flops of the call.
    `sink` is a device float tensor (written only in a case that never happens)."""
    _need_gpu(sink)
    _check(_lib.pkv_mfma_peak_probe(int(iters), _ptr(sink), _stream(sink.device)), "pkv_mfma_peak_probe")
    return int(_lib.pkv_device_cu_count()) * 8 * int(iters) * 4 * 32768


def stream_read_probe(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Read every byte of `buf` once (bandwidth reference); folds into the uint32-sized `sink`."""
    _need_gpu(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.pkv_stream_read_probe(_ptr(buf), nbytes, _ptr(sink), _stream(buf.device)), "pkv_stream_read_probe")
