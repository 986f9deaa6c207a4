"""Rotary position embedding (RoPE) of queries and keys.

TEST INFRASTRUCTURE ONLY (see the package docstring): float64 numpy, no code
shared with the GPU path.

What the pages fix: the model uses RoPE, with a base theta that grows with
each length-extension stage (640K, then 5M, then 80M for the 1M-token stage)
([S App. E]; [P seg. 20]).  They do not state the pairing of channels or
where in the block the rotation sits.

Readings taken:
* the original rotary formulation with interleaved pairs: channels (2i,
  2i+1) of a head form a pair, rotated by the angle pos * theta^(-2i/d);
* the angle is the exact real number pos * theta^(-2i/d) (float64 here; no
  single-precision rounding of large angles);
* queries and keys are rotated right after their projection, at their
  absolute positions (values never are).
"""

import math

import numpy as np

__all__ = ["rope_inv_freq", "apply_rope"]


def rope_inv_freq(d, theta):
    """theta^(-2i/d) for the d/2 channel pairs i = 0 .. d/2-1."""
    if d % 2 or not theta > 0:
        raise ValueError("d must be even and theta > 0")
    return np.array([theta ** (-2.0 * i / d) for i in range(d // 2)])


def apply_rope(x, pos0, theta):
    """Rotate x [..., N, d] (last axis: channels of one head) for positions
    pos0 .. pos0 + N - 1: pair (2i, 2i+1) at position p becomes
    (x0 cos a - x1 sin a, x0 sin a + x1 cos a), a = p * theta^(-2i/d)."""
    x = np.asarray(x, dtype=np.float64)
    N, d = x.shape[-2], x.shape[-1]
    inv = rope_inv_freq(d, theta)
    out = np.empty_like(x)
    for n in range(N):
        p = pos0 + n
        for i in range(d // 2):
            a = p * inv[i]
            c, s = math.cos(a), math.sin(a)
            x0, x1 = x[..., n, 2 * i], x[..., n, 2 * i + 1]
            out[..., n, 2 * i] = x0 * c - x1 * s
            out[..., n, 2 * i + 1] = x0 * s + x1 * c
    return out
