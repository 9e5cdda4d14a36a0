"""bf16 outputs on every output path (needs an MI355X).

Every attention call takes an output dtype, and the kernels write either the fp32 result or that
same value rounded to bf16 (the output dtype is a run-time flag inside one kernel instance).  So
for identical inputs the bf16 output must equal the fp32 output rounded to nearest-even, bit for
bit, whatever path wrote the row.  The fp32 outputs themselves are checked against the oracle by
the parity tests; this module covers the rounding and the store of each path:

* decode: rows of one split written by the attention kernel, rows merged by the split reduce,
  the plan-free small-batch form, bf16 and E4M3 pools;
* prefill: one key split (rows written by the attention kernel), several key splits (rows written
  by the merge kernel), rows packed by KV head, bf16 and E4M3 pools;
* the fused mixed launch (both of its outputs).

Inputs: seeded N(0,1) bf16 pools with a shuffled block table (E4M3 pools: the same values cast to
E4M3 at scale 2^-5).
"""
import math
import sys

import numpy as np
import pytest

from gpu_common import MODES, flag, new_err

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

SCALE8 = 2.0 ** -5


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_170_amd as m
    return m


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def _rne_bits(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().float().to(torch.bfloat16).view(torch.int16).numpy()


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().view(torch.int16).numpy()


def _same(fp32_out, bf16_out, what):
    assert fp32_out.dtype == torch.float32 and bf16_out.dtype == torch.bfloat16
    assert torch.isfinite(fp32_out).all(), what
    a, b = _rne_bits(fp32_out), _bits(bf16_out)
    bad = np.flatnonzero(a.ravel() != b.ravel())
    assert bad.size == 0, f"{what}: {bad.size} of {a.size} bf16 outputs differ from the rounded fp32 output"


class Pools:
    """Seeded pools sized for `ctx` positions per sequence, one shuffled table per sequence."""

    def __init__(self, dev, seed, num_seqs, ctx_max, hkv, hd):
        g = torch.Generator(device="cpu").manual_seed(seed)
        nb = -(-ctx_max // 16)
        self.nblk = nb * num_seqs + 5
        self.kp = torch.randn((self.nblk, hkv, 16, hd), generator=g).to(torch.bfloat16).to(dev)
        self.vp = torch.randn((self.nblk, hkv, 16, hd), generator=g).to(torch.bfloat16).to(dev)
        perm = torch.randperm(self.nblk, generator=g)[: nb * num_seqs]
        self.bt = perm.to(torch.int32).reshape(num_seqs, nb).contiguous().to(dev)
        self.kp8 = (self.kp.float() / SCALE8).to(torch.float8_e4m3fn)
        self.vp8 = (self.vp.float() / SCALE8).to(torch.float8_e4m3fn)
        self.g = g


def _decode_pair(pkv, P, q, ctx, scale, fp8, err, split_tokens=0):
    outs = []
    for od in (torch.float32, torch.bfloat16):
        if fp8:
            o = pkv.paged_attn_decode_fp8(q, P.kp8, P.vp8, P.bt, ctx, scale, SCALE8, SCALE8, out_dtype=od,
                                          split_tokens=split_tokens, err_flag=err)
        else:
            o = pkv.paged_attn_decode(q, P.kp, P.vp, P.bt, ctx, scale, out_dtype=od, split_tokens=split_tokens,
                                      err_flag=err)
        outs.append(o)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("shape", ["splits", "single", "small_batch"])
def test_decode_bf16_output_is_the_rounded_fp32_output(pkv, dev, mode, fp8, shape):
    # splits: long contexts over several 512-position splits (rows merged by the split reduce);
    # single: every context inside one split (rows written by the attention kernel); small_batch:
    # a few sequences, one work item per workgroup (no plan pass).
    num_seqs, ctx_lo, ctx_hi, split = {"splits": (96, 600, 3000, 512), "single": (96, 1, 500, 512),
                                       "small_batch": (3, 1, 2500, 0)}[shape]
    hq, hkv, hd = 32, 4, 128
    _say(f"decode bf16 out: {shape} fp8={fp8} {mode}")
    P = Pools(dev, 41, num_seqs, ctx_hi, hkv, hd)
    ctx = torch.randint(ctx_lo, ctx_hi + 1, (num_seqs,), generator=P.g).to(torch.int32).to(dev)
    q = torch.randn((num_seqs, hq, hd), generator=P.g).to(torch.bfloat16).to(dev)
    err = new_err(dev, mode)
    o32, o16 = _decode_pair(pkv, P, q, ctx, 1.0 / math.sqrt(hd), fp8, err, split)
    _same(o32, o16, f"decode {shape}")
    assert flag(err) == 0


def _prefill_pair(pkv, P, q, cu, offs, maxl, scale, fp8, err):
    outs = []
    for od in (torch.float32, torch.bfloat16):
        if fp8:
            o = pkv.paged_attn_prefill_chunk_fp8(q, cu, offs, P.kp8, P.vp8, P.bt, maxl, scale, SCALE8, SCALE8,
                                                 causal=True, out_dtype=od, err_flag=err)
        else:
            o = pkv.paged_attn_prefill_chunk(q, cu, offs, P.kp, P.vp, P.bt, maxl, scale, causal=True, out_dtype=od,
                                             err_flag=err)
        outs.append(o)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("shape", ["one_split", "key_splits", "packed"])
def test_prefill_bf16_output_is_the_rounded_fp32_output(pkv, dev, mode, fp8, shape):
    # one_split: 1,024 rows over 64 query heads give a row tile per CU (one key split, rows written
    # by the attention kernel); key_splits: 512 rows at offset 4,096 (splits merged by the merge
    # kernel); packed: short chunks, rows packed by KV head.
    num_seqs, chunk, offset = {"one_split": (1, 1024, 512), "key_splits": (1, 512, 4096),
                               "packed": (8, 24, 700)}[shape]
    hq, hkv, hd = 64, 8, 128
    _say(f"prefill bf16 out: {shape} fp8={fp8} {mode}")
    P = Pools(dev, 42, num_seqs, offset + chunk, hkv, hd)
    q = torch.randn((num_seqs * chunk, hq, hd), generator=P.g).to(torch.bfloat16).to(dev)
    cu = torch.arange(0, num_seqs * chunk + 1, chunk, dtype=torch.int32).to(dev)
    offs = torch.full((num_seqs,), offset, dtype=torch.int32).to(dev)
    # The workspace holds key-split partials only: none for one split, some for several.
    ws = pkv.prefill_workspace_bytes(num_seqs, chunk, hq, hd, P.bt.shape[1])
    if shape == "one_split":
        assert ws == 0
    if shape == "key_splits":
        assert ws > 0
    err = new_err(dev, mode)
    o32, o16 = _prefill_pair(pkv, P, q, cu, offs, chunk, 1.0 / math.sqrt(hd), fp8, err)
    _same(o32, o16, f"prefill {shape}")
    assert flag(err) == 0


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("fp8", [False, True])
def test_fused_mixed_bf16_outputs_are_the_rounded_fp32_outputs(pkv, dev, mode, fp8):
    hq, hkv, hd = 64, 8, 128
    nd, chunk, offset = 40, 256, 2048
    _say(f"fused mixed bf16 out: fp8={fp8} {mode}")
    P = Pools(dev, 43, nd + 1, offset + chunk, hkv, hd)
    dec_bt, pre_bt = P.bt[:nd].contiguous(), P.bt[nd:].contiguous()
    ctx = torch.randint(1, offset + chunk + 1, (nd,), generator=P.g).to(torch.int32).to(dev)
    dq = torch.randn((nd, hq, hd), generator=P.g).to(torch.bfloat16).to(dev)
    pq = torch.randn((chunk, hq, hd), generator=P.g).to(torch.bfloat16).to(dev)
    cu = torch.tensor([0, chunk], dtype=torch.int32).to(dev)
    offs = torch.tensor([offset], dtype=torch.int32).to(dev)
    kp, vp = (P.kp8, P.vp8) if fp8 else (P.kp, P.vp)
    ks = SCALE8 if fp8 else 1.0
    err = new_err(dev, mode)
    outs = []
    for od in (torch.float32, torch.bfloat16):
        outs.append(pkv.paged_attn_mixed(kp, vp, 1.0 / math.sqrt(hd), dec_query=dq, dec_block_tables=dec_bt,
                                         context_lens=ctx, pre_query=pq, cu_q_lens=cu, chunk_offsets=offs,
                                         pre_block_tables=pre_bt, max_q_len=chunk, k_scale=ks, v_scale=ks,
                                         out_dtype=od, err_flag=err))
    torch.cuda.synchronize()
    (d32, p32), (d16, p16) = outs
    _same(d32, d16, "fused decode rows")
    _same(p32, p16, "fused chunk rows")
    assert flag(err) == 0
