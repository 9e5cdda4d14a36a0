"""Pins of the FP8 (E4M3) reference in oracle/fp8.py: the OFP8 special values
(tests/golden/e4m3_spec_values.json), a round trip over every code, torch's own float8_e4m3fn
conversion, ties, saturation, NaN and signed zero, closed forms for power-of-two scales and the
format's error bound."""
import json
import os

import numpy as np
import pytest
import torch

from oracle.fp8 import (E4M3_MAX, NAN_CODE, dequantize, e4m3_decode, e4m3_encode, e4m3_value, quantize,
                        quantize_bf16_bits)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_spec_values():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_spec_values.json")))
    for code, val in g["values"]:
        assert e4m3_value(int(code, 16)) == val
        assert int(e4m3_encode(np.array([val]))[0]) == int(code, 16) or val == 0.0
    for code in g["nan_codes"]:
        assert np.isnan(e4m3_value(int(code, 16)))


def test_every_code_round_trips():
    for c in range(256):
        v = e4m3_value(c)
        if np.isnan(v):
            continue
        got = int(e4m3_encode(np.array([v]))[0])
        assert got == c, (hex(c), v, hex(got))  # includes -0.0 -> 0x80


def test_against_torch_float8_cast():
    """torch's float8_e4m3fn conversion rounds to nearest even; below the saturation point the two
    encoders must agree bit for bit, including on exact midpoints between codes."""
    rng = np.random.default_rng(7)
    mags = np.concatenate([
        rng.uniform(0, 440, 4000), np.exp2(rng.uniform(-12, 8.7, 4000)),
        (e4m3_decode(np.arange(0, 0x7E)) + e4m3_decode(np.arange(1, 0x7F))) / 2,  # midpoints
    ])
    vals = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    vals = vals[np.abs(vals) < E4M3_MAX]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3_encode(vals.astype(np.float64))
    assert np.array_equal(got, ref)


def test_ties_saturation_nan_zero():
    enc = lambda x: int(e4m3_encode(np.array([x], dtype=np.float64))[0])
    assert enc(1.0625) == 0x38   # halfway 1.0 / 1.125 -> even mantissa 0
    assert enc(1.1875) == 0x3A   # halfway 1.125 / 1.25 -> even mantissa 2
    assert enc(2.0 ** -10) == 0x00  # halfway 0 / 2^-9
    assert enc(3 * 2.0 ** -10) == 0x02  # halfway 2^-9 / 2^-8
    assert enc(-2.0 ** -11) == 0x80  # rounds to negative zero
    assert enc(447.0) == 0x7E and enc(463.9) == 0x7E and enc(1e6) == 0x7E and enc(np.inf) == 0x7E
    assert enc(-1e6) == 0xFE and enc(-np.inf) == 0xFE
    assert enc(np.nan) == NAN_CODE


def test_power_of_two_scale_is_exact_rescaling():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(3000).astype(np.float32)
    for k in (-6, 0, 3):
        assert np.array_equal(quantize(x, 2.0 ** k), e4m3_encode(x.astype(np.float64) * 2.0 ** -k))


def test_quantisation_error_bound_and_monotonicity():
    """Within the normal range the relative error is at most half a mantissa step, 2^-4; below it
    the absolute error is at most half the subnormal step, 2^-10 * scale."""
    rng = np.random.default_rng(4)
    scale = 0.0123
    x = (rng.standard_normal(20000) * 2).astype(np.float32)
    back = dequantize(quantize(x, scale), scale)
    xs = x.astype(np.float64)
    r = np.abs(xs) / scale
    normal = (r >= 2.0 ** -6) & (r < E4M3_MAX)
    sub = r < 2.0 ** -6
    assert normal.sum() > 15000 and (r >= E4M3_MAX).sum() > 0
    assert np.all(np.abs(back - xs)[normal] <= np.abs(xs[normal]) * (2.0 ** -4) * (1 + 1e-6))
    assert np.all(np.abs(back - xs)[sub] <= 2.0 ** -10 * scale * (1 + 1e-6))
    sat = r >= E4M3_MAX * (1 + 2.0 ** -4)
    assert np.all(back[sat] == np.sign(xs[sat]) * E4M3_MAX * float(np.float32(scale)))
    order = np.argsort(xs)
    vals = e4m3_decode(quantize(xs[order].astype(np.float32), scale))
    assert np.all(np.diff(vals) >= 0)


def test_bf16_table_form_equals_direct_form():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 65536, 50000, dtype=np.uint32).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    for scale in (0.0123, 1.0, 3.5):
        assert np.array_equal(quantize_bf16_bits(bits, scale), quantize(f, scale))
