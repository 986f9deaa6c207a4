"""Pins for oracle/fp8.py.

* library routine: torch's float8_e4m3fn dtype (decode of all 256 codes,
  and the float64 -> e4m3fn cast for in-range values);
* brute force: nearest representable value by exhaustive search with
  ties to the even code;
* closed forms from the OCP E4M3FN definition: 448, 2^-6, 2^-9, NaN codes;
* round trip code -> value -> code for every non-NaN code.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.fp8 import e4m3_decode, e4m3_encode, quantize_kv_fp8, dequantize_kv_fp8


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(ref[~nan_ref]))


def test_decode_closed_forms():
    assert e4m3_decode(0x7E) == 448.0 and e4m3_decode(0xFE) == -448.0
    assert e4m3_decode(0x01) == 2.0 ** -9
    assert e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert e4m3_decode(0x08) == 2.0 ** -6
    assert e4m3_decode(0x38) == 1.0
    assert np.isnan(e4m3_decode(0x7F)) and np.isnan(e4m3_decode(0xFF))
    assert np.sum(np.isnan(e4m3_decode(np.arange(256)))) == 2
    assert e4m3_decode(0x00) == 0.0 and np.signbit(e4m3_decode(0x80))


def test_roundtrip_every_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert int(e4m3_encode(e4m3_decode(c))) == c


def _brute_encode(x):
    """Exhaustive nearest finite value, ties to the even code, saturating."""
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1, x) < 0 else 0
    a = min(abs(x), 448.0)
    best, best_err = None, None
    for c in range(0x7F):            # 0x00 .. 0x7E: non-negative finite codes
        err = abs(a - float(e4m3_decode(c)))
        if best is None or err < best_err or (err == best_err and c % 2 == 0):
            best, best_err = c, err
    return sign | best


def test_encode_matches_brute_force():
    rng = np.random.default_rng(7)
    xs = np.concatenate([
        rng.standard_normal(3000) * 50,
        rng.standard_normal(1000) * 0.01,
        rng.uniform(-600, 600, 500),
        (e4m3_decode(np.arange(0, 0x7E)) + e4m3_decode(np.arange(1, 0x7F))) / 2,   # midpoints
        -(e4m3_decode(np.arange(0, 0x7E)) + e4m3_decode(np.arange(1, 0x7F))) / 2,
        [0.0, -0.0, 448.0, 449.0, 464.0, 479.9, 480.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -11],
    ])
    ours = e4m3_encode(xs)
    for x, c in zip(xs, ours):
        assert int(c) == _brute_encode(float(x)), x


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(8)
    xs = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(5000) * 0.005])
    xs = xs[np.abs(xs) <= 448.0]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(xs), ref)


def test_ties_to_even_and_saturation():
    assert int(e4m3_encode(1.0625)) == 0x38       # between 1.0 (0x38) and 1.125 (0x39)
    assert int(e4m3_encode(1.1875)) == 0x3A       # between 1.125 and 1.25 (0x3A)
    assert int(e4m3_encode(2.0 ** -10)) == 0x00   # half the smallest subnormal
    assert int(e4m3_encode(3 * 2.0 ** -10)) == 0x02
    assert int(e4m3_encode(464.0)) == 0x7E
    assert int(e4m3_encode(1e30)) == 0x7E and int(e4m3_encode(-1e30)) == 0xFE
    assert int(e4m3_encode(float("nan"))) == 0x7F


def test_quantize_per_head_scales_and_error_bound():
    rng = np.random.default_rng(9)
    kv = rng.standard_normal((2, 3, 50, 16)).astype(np.float32)
    kv[:, 1] *= 10
    kv[:, 2] = 0
    codes, scales = quantize_kv_fp8(kv)
    assert scales.dtype == np.float32 and codes.dtype == np.uint8
    for h in range(2):
        amax = np.abs(kv[:, h]).max()
        assert scales[h] == np.float32(amax / np.float32(448.0))
        # the largest element lands on the largest code
        idx = np.unravel_index(np.argmax(np.abs(kv[:, h])), kv[:, h].shape)
        assert codes[:, h][idx] & 0x7F == 0x7E
    assert scales[2] == 1.0 and np.all(codes[:, 2] == 0)
    deq = dequantize_kv_fp8(codes, scales)
    x = kv.astype(np.float64)
    for h in range(3):
        s = float(scales[h])
        y = np.abs(x[:, h]) / s
        # half a quantisation step: 2^-4 relative for normals, 2^-10 absolute for subnormals
        bound = np.maximum(y * 2.0 ** -4, 2.0 ** -10) * s * (1 + 1e-6)
        assert np.all(np.abs(deq[:, h] - x[:, h]) <= bound)


def test_encode_with_given_scales_round_trips_every_code():
    """With a power-of-two scale the division is exact, so the value s*decode(c)
    of every finite code c must encode back to c (negative zero to 0x80)."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for s in (0.25, 1.0, 8.0):
        vals = (e4m3_decode(codes) * s).astype(np.float32).reshape(1, 1, -1, 1)
        scales = np.array([s], dtype=np.float32)
        assert np.array_equal(oracle.encode_kv_fp8(vals, scales).reshape(-1), codes)


def test_encode_with_given_scales_saturates_and_uses_each_heads_scale():
    x = np.array([[[[1000.0, -1000.0, 3.0, -3.0]], [[1000.0, -1000.0, 3.0, -3.0]]]], dtype=np.float32)
    c = oracle.encode_kv_fp8(x, np.array([1.0, 2.0], dtype=np.float32))
    # 3 = 1.5 * 2^1: exponent field 1 + 7 = 0b1000, mantissa 0b100
    assert list(c[0, 0, 0]) == [0x7E, 0xFE, 0x44, 0xC4]
    # 3 / 2 = 1.5 * 2^0: exponent field 0b0111
    assert list(c[0, 1, 0]) == [0x7E, 0xFE, 0x3C, 0xBC]


def test_encode_with_the_quantisers_own_scales_gives_its_codes():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3, 17, 8)).astype(np.float32)
    codes, scales = quantize_kv_fp8(x)
    assert np.array_equal(oracle.encode_kv_fp8(x, scales), codes)
