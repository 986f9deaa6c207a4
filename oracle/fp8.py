"""OCP fp8-e4m3fn codec and per-KV-head cache quantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring): no code shared with the
GPU path.

The pages motivate an 8-bit KV cache (the 65B example with 8-bit cache
quantisation, [P seg. 1]; deployments that quantise the cache to 4 or 8 bits,
[P seg. 24]) but fix no format.  Readings taken:

* Format: OCP "E4M3FN" -- 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448;
  subnormals are m/8 * 2^-6 (step 2^-9).  Written here from that definition.
* Encoding: round to nearest, ties to even, saturating to +-448.
* Scales: one float32 scale per KV head, separately for K and for V, shared
  by every sequence of the batch: s_h = amax_h / 448 over all (b, n, d) of
  that head (s_h = 1 when the head is all zero).  A stored code c stands for
  the value s_h * decode(c).
* The two steps that decide a code -- the scale s_h = amax/448 and the
  scaled value x / s_h -- are done in IEEE float32 (one correctly rounded
  division each), the precision the quantising kernel uses, so that both
  sides take the same integer decision.  Everything else is exact.
"""

import math

import numpy as np

__all__ = [
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_encode",
    "kv_fp8_scales",
    "quantize_kv_fp8",
    "encode_kv_fp8",
    "dequantize_kv_fp8",
]

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6
_SUB_STEP = 2.0 ** -9


def _decode_scalar(code):
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * _MIN_NORMAL
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_DECODE_TABLE = np.array([_decode_scalar(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes):
    """Value of each e4m3fn code (uint8 array or int) as float64."""
    return _DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def _encode_scalar(x):
    x = float(x)
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if a >= E4M3_MAX:
        return sign | 0x7E
    if a < _MIN_NORMAL:
        # subnormal range: multiples of 2^-9; n == 8 is the smallest normal,
        # whose code is also 8, so the code is n itself.
        return sign | int(round(a / _SUB_STEP))
    _, k = math.frexp(a)          # a = f * 2^k, f in [0.5, 1)
    exp = k - 1                   # a in [2^exp, 2^(exp+1))
    n = int(round(a / 2.0 ** (exp - 3)))   # 8 <= n <= 16, ties to even
    code = (exp + 7) * 8 + (n - 8)         # n == 16 carries into the exponent
    return sign | min(code, 0x7E)


def e4m3_encode(x):
    """Round-to-nearest-even, saturating e4m3fn encoding of float values."""
    arr = np.asarray(x, dtype=np.float64)
    flat = arr.reshape(-1)
    out = np.fromiter((_encode_scalar(v) for v in flat), dtype=np.uint8,
                      count=flat.size)
    return out.reshape(arr.shape)


def kv_fp8_scales(kv):
    """Per-KV-head scales of a KV tensor [B, Hkv, n, d]: s_h = amax_h / 448
    over all (b, n, d) of head h, one float32 division (1 for an all-zero
    head).  kv holds the exact float32 or bfloat16 values."""
    x32 = np.asarray(kv, dtype=np.float32)
    hkv = x32.shape[1]
    scales = np.empty(hkv, dtype=np.float32)
    for h in range(hkv):
        amax = np.float32(np.max(np.abs(x32[:, h]))) if x32[:, h].size else np.float32(0)
        scales[h] = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(E4M3_MAX))
    return scales


def quantize_kv_fp8(kv):
    """Quantise a KV tensor [B, Hkv, n, d] to e4m3fn codes with per-head scales.

    kv holds the exact values the quantiser receives (float32 or bfloat16
    values, here as any float array).  Returns (codes uint8 [B, Hkv, n, d],
    scales float32 [Hkv]): the scales of kv_fp8_scales, and each value x of
    head h encoded as e4m3fn(x / s_h), the division in float32 (IEEE,
    correctly rounded).
    """
    scales = kv_fp8_scales(kv)
    return encode_kv_fp8(kv, scales), scales


def encode_kv_fp8(kv, scales):
    """Codes of a KV tensor [B, Hkv, n, d] under per-head scales that are
    already set (rows appended to an 8-bit cache after its scales were fixed):
    code = e4m3fn(x / s_h), the division in float32, saturating like
    e4m3_encode.  kv holds the exact float32 or bfloat16 values."""
    x32 = np.asarray(kv, dtype=np.float32)
    s32 = np.asarray(scales, dtype=np.float32)
    codes = np.empty(x32.shape, dtype=np.uint8)
    for h in range(x32.shape[1]):
        codes[:, h] = e4m3_encode(x32[:, h] / s32[h])
    return codes


def dequantize_kv_fp8(codes, scales):
    """Exact float64 values s_h * decode(code) of a quantised KV tensor."""
    vals = e4m3_decode(codes)
    return vals * np.asarray(scales, dtype=np.float64)[None, :, None, None]
