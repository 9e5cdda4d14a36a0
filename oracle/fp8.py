"""Plain reference of the FP8 KV pool: E4M3 codes, per-tensor scales, quantise on write.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never imports this module.

Sources.  The pages say the served model runs in FP8 ("Phase 17 · 04 — vLLM serving internals",
the opening benchmark and the memory section) but never say how a KV cache would be stored in
FP8.  The format itself is the 8-bit E4M3 encoding of the OCP "8-bit Floating Point
Specification (OFP8)": 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
holds the subnormals m * 2^-9; the code S.1111.111 is NaN; there are no infinities; the largest
finite magnitude is 448 (S.1111.110).

Readings (each is listed in the design notes):

* one fp32 scale per pool (K and V separately), chosen by the caller; a stored code c stands for
  value(c) * scale;
* the write multiplies each input element (bf16 or fp32, widened exactly to fp32) by the fp32
  reciprocal of the scale (1 / scale rounded to nearest in fp32) in fp32 arithmetic, then rounds
  the product to the nearest E4M3 value, ties to the even code; finite magnitudes at or above 448
  and infinities saturate to +-448; NaN stays NaN (S.1111.111); the sign of zero is kept;
* attention over an FP8 pool is exact softmax attention over the dequantised values
  value(c) * scale (queries stay bf16).

The encoder below finds the nearest code by searching the table of all finite E4M3 values, which
is a different method from the bit arithmetic of the GPU encoder.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def e4m3_value(code: int) -> float:
    """Exact value of one E4M3 code (OFP8 definition)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Magnitudes of the non-negative finite codes 0x00 .. 0x7E, in increasing order (code = index).
_POS = np.array([e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
assert np.all(np.diff(_POS) > 0)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact fp64 values of an array of codes (uint8)."""
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each value, ties to the even code, saturating at 448; NaN -> NaN.

    For each magnitude, the two neighbouring entries of the table of finite magnitudes are found
    by binary search and the closer one is taken (the even code on a tie)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    nan = np.isnan(v)
    a_safe = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_POS, a_safe, side="left")          # first magnitude >= a (<= 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a_safe - _POS[lo], _POS[hi] - a_safe
    pick_lo = (dlo < dhi) | ((dlo == dhi) & (lo % 2 == 0))
    code = np.where(_POS[hi] == a_safe, hi, np.where(pick_lo, lo, hi)).astype(np.uint8)
    code = code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return np.where(nan, np.uint8(NAN_CODE), code).astype(np.uint8)


def reciprocal_f32(scale: float) -> np.float32:
    """1 / scale rounded to nearest in fp32."""
    return np.float32(1.0) / np.float32(scale)


def quantize(x_f32: np.ndarray, scale: float) -> np.ndarray:
    """Codes of fp32 elements for a pool with this scale: product with the fp32 reciprocal, taken
    in fp32, then rounded to E4M3."""
    with np.errstate(over="ignore", invalid="ignore"):  # overflow to inf saturates; NaN stays NaN
        prod = np.asarray(x_f32, dtype=np.float32) * reciprocal_f32(scale)  # one IEEE fp32 multiply each
    return e4m3_encode(prod.astype(np.float64))


def quantize_bf16_bits(bits: np.ndarray, scale: float) -> np.ndarray:
    """quantize() of bf16 elements given as uint16 bit patterns, evaluated once for each of the
    65,536 patterns and looked up (the same function, cheaper on large pools)."""
    every = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    return quantize(every, scale)[np.asarray(bits, dtype=np.uint16)]


def cache_write_fp8(key_pool: np.ndarray, value_pool: np.ndarray, key_f32: np.ndarray, value_f32: np.ndarray,
                    slots: np.ndarray, k_scale: float, v_scale: float):
    """Copies of the code pools ``[N_blk, Hkv, 16, hd]`` (uint8) with token ``t``'s quantised K and
    V rows stored at slot ``slots[t]`` (its block, its offset, every KV head); negative slots are
    skipped, slots must be unique."""
    nblk, hkv, b, hd = key_pool.shape
    live = slots[slots >= 0]
    if live.size and live.max() >= nblk * b:
        raise ValueError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slots")
    kp, vp = key_pool.copy(), value_pool.copy()
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        kp[sl // b, :, sl % b] = quantize(key_f32[t].reshape(-1), k_scale).reshape(hkv, hd)
        vp[sl // b, :, sl % b] = quantize(value_f32[t].reshape(-1), v_scale).reshape(hkv, hd)
    return kp, vp


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """fp64 values a code pool stands for: value(code) * scale."""
    return e4m3_decode(codes) * float(np.float32(scale))
