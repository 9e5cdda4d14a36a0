"""GPU test of the decode that allocates nothing (needs an MI355X).

pkv_paged_attn_decode_noalloc runs the kernels of pkv_paged_attn_decode with its workspace in the
library's static device scratch instead of a caller's buffer, so on the same inputs its output
must be bit-identical to pkv_paged_attn_decode's (same split size, same plan), and within the
oracle's tolerance.  Two calls in a row, the second with a smaller input, show that the scratch
the first call left behind does not leak into the second.  Both call modes run (checked kernels
with an err_flag, and the release kernels, err_flag NULL).  Calls go through the C ABI via the
ctypes binding, with preallocated outputs.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_common import MODES, close, flag, mixed_step_case, mixed_step_reference, new_err, to_dev

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


def _both(pkv, dev, mode, q, kp, vp, bt, ctx, scale, split=0):
    """(workspace decode, no-alloc decode) outputs on the host, same inputs and split size."""
    err = new_err(dev, mode)
    ref = pkv.paged_attn_decode(q, kp, vp, bt, ctx, scale, split_tokens=split, err_flag=err)
    out = torch.full_like(ref, float("nan"))
    got = pkv.paged_attn_decode_noalloc(q, kp, vp, bt, ctx, scale, out=out, split_tokens=split, err_flag=err)
    assert got is out
    torch.cuda.synchronize()
    assert flag(err) == 0
    return ref.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("mode", MODES)
def test_noalloc_decode_matches_the_workspace_decode(pkv, mode):
    dev = torch.device("cuda:0")
    # First call: the mixed step's 127-sequence decode (multi-split, ~17 MB of partials) after the
    # chunk's cache write, as the benchmark runs it.
    dec, pre, slots, rk, rv = mixed_step_case()
    need = pkv.decode_workspace_bytes(dec.num_seqs, dec.num_q_heads, dec.num_kv_heads, dec.head_dim,
                                      dec.max_blocks_per_seq)
    _say(f"case no-alloc decode ({mode}): mixed step, 127 sequences, workspace {need / 2**20:.1f} MiB of "
         f"{pkv.NOALLOC_SCRATCH_BYTES / 2**20:.0f} MiB scratch")
    assert need <= pkv.NOALLOC_SCRATCH_BYTES
    kp, vp = to_dev(rk, dev, True), to_dev(rv, dev, True)
    a, b = _both(pkv, dev, mode, to_dev(dec.query, dev, True), kp, vp, to_dev(dec.block_tables, dev),
                 to_dev(dec.context_lens, dev), dec.scale)
    assert a.tobytes() == b.tobytes(), "no-alloc decode differs from the workspace decode (mixed step)"
    ref_dec, _ = mixed_step_reference()
    mx, mean = close(b, ref_dec, "no-alloc decode vs oracle (mixed step)")
    _say(f"  max-abs {mx:.2e} mean-abs {mean:.2e}")
    del kp, vp
    # Second call, smaller: fewer sequences, other head counts, split 128 (more splits per
    # sequence than the first call had), one empty context.
    c = wl.random_case(501, kind="decode", dtype="bf16", num_seqs=5, num_q_heads=16, num_kv_heads=2, head_dim=128,
                       max_ctx=900, min_ctx=0, new_tokens=False, poison=True)
    c.context_lens[2] = 0
    _say(f"case no-alloc decode ({mode}): second call, 5 sequences, contexts {c.context_lens.tolist()}")
    kp, vp = to_dev(c.key_pool, dev, True), to_dev(c.value_pool, dev, True)
    a, b = _both(pkv, dev, mode, to_dev(c.query, dev, True), kp, vp, to_dev(c.block_tables, dev),
                 to_dev(c.context_lens, dev), c.scale, split=128)
    assert a.tobytes() == b.tobytes(), "no-alloc decode differs from the workspace decode (second call)"
    ref = oracle.decode(c.query, c.key_pool, c.value_pool, c.block_tables, c.context_lens, c.scale, "bf16")
    close(b, ref, "no-alloc decode vs oracle (second call)")
    assert (b[2] == 0).all()


def test_noalloc_decode_rejects_shapes_beyond_the_scratch(pkv):
    """Shapes whose workspace exceeds the scratch are refused on the host (nothing is launched)."""
    dev = torch.device("cuda:0")
    B, hq, hkv, hd, maxb = 1024, 64, 8, 128, 1024
    need = pkv.decode_workspace_bytes(B, hq, hkv, hd, maxb)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, hq, hd), dtype=torch.bfloat16, device=dev)
    kp = torch.zeros((4, hkv, 16, hd), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, maxb), dtype=torch.int32, device=dev)
    ctx = torch.ones(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, hq, hd), dtype=torch.float32, device=dev)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attn_decode_noalloc(q, kp, kp, bt, ctx, hd ** -0.5, out=out)
    assert e.value.status == pkv.SCRATCH_TOO_SMALL
