"""Pins for the generation-time parts of the oracle: the self-decoder's ring
cache decode (oracle.swa_ring_decode_attention) and the token-by-token block
(oracle.yoco_block_generate).

* ring decode == row pos of the full-sequence sliding-window attention,
  bitwise, for a ring filled with the last W positions (slot t mod W) --
  before, at and after the ring wraps;
* slots outside the window are never read (they hold NaN);
* W = 1 returns the current token's V exactly;
* brute force: a scalar Python loop over the window;
* token-by-token generation reproduces the full forward's rows bitwise
  (causality), and leaves in each ring the last W positions' K/V.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.block import _heads, _norm_rows, linear_rows
from test_oracle_block import make_params

RNG = np.random.default_rng(77)


def _ring_from_sequence(k, v, pos, W):
    """Ring of W slots holding positions max(0, pos-W+1)..pos (slot t mod W);
    slots never written hold NaN."""
    B, Hkv, _, d = k.shape
    kr = np.full((B, Hkv, W, d), np.nan)
    vr = np.full((B, Hkv, W, d), np.nan)
    for t in range(max(0, pos - W + 1), pos + 1):
        kr[:, :, t % W] = k[:, :, t]
        vr[:, :, t % W] = v[:, :, t]
    return kr, vr


@pytest.mark.parametrize("W", [1, 4, 7, 16])
def test_ring_decode_equals_window_row_bitwise(W):
    B, Hq, Hkv, N, d = 2, 4, 2, 40, 8
    q = RNG.standard_normal((B, Hq, N, d))
    k = RNG.standard_normal((B, Hkv, N, d))
    v = RNG.standard_normal((B, Hkv, N, d))
    o_full, lse_full = oracle.swa_attention(q, k, v, W)
    for pos in sorted({0, 1, W - 2, W - 1, W, W + 1, 2 * W + 3, N - 1} - {-1}):
        if pos < 0 or pos >= N:
            continue
        kr, vr = _ring_from_sequence(k, v, pos, W)
        o, lse = oracle.swa_ring_decode_attention(q[:, :, pos], kr, vr, pos)
        assert np.array_equal(o, o_full[:, :, pos]), (W, pos)
        assert np.array_equal(lse, lse_full[:, :, pos]), (W, pos)
        assert np.all(np.isfinite(o))   # the NaN slots were never read


def test_ring_window_slots():
    assert oracle.ring_window(0, 4) == [(0, 0)]
    assert oracle.ring_window(2, 4) == [(0, 0), (1, 1), (2, 2)]
    assert oracle.ring_window(5, 4) == [(2, 2), (3, 3), (4, 0), (5, 1)]
    assert oracle.ring_window(9, 1) == [(9, 0)]
    with pytest.raises(ValueError):
        oracle.ring_window(-1, 4)


def test_window_one_returns_current_value():
    B, Hq, Hkv, W, d = 1, 4, 2, 1, 8
    q = RNG.standard_normal((B, Hq, d))
    kr = RNG.standard_normal((B, Hkv, W, d))
    vr = RNG.standard_normal((B, Hkv, W, d))
    o, lse = oracle.swa_ring_decode_attention(q, kr, vr, pos=17)
    for h in range(Hq):
        assert np.array_equal(o[0, h], vr[0, h // 2, 0])
        assert lse[0, h] == pytest.approx(np.dot(q[0, h], kr[0, h // 2, 0]) / math.sqrt(d), abs=1e-14)


def test_ring_decode_brute_force():
    B, Hq, Hkv, W, d, pos = 1, 2, 1, 5, 3, 12
    q = RNG.standard_normal((B, Hq, d))
    kr = RNG.standard_normal((B, Hkv, W, d))
    vr = RNG.standard_normal((B, Hkv, W, d))
    o, lse = oracle.swa_ring_decode_attention(q, kr, vr, pos)
    for h in range(Hq):
        z = []
        for t in range(pos - W + 1, pos + 1):
            s = t % W
            z.append(sum(q[0, h, i] * kr[0, 0, s, i] for i in range(d)) / math.sqrt(d))
        m = max(z)
        w = [math.exp(x - m) for x in z]
        tot = sum(w)
        ref = [sum(w[j] * vr[0, 0, (pos - W + 1 + j) % W, i] for j in range(W)) / tot for i in range(d)]
        assert np.allclose(o[0, h], ref, atol=1e-13, rtol=0)
        assert lse[0, h] == pytest.approx(m + math.log(tot), abs=1e-13)


@pytest.mark.parametrize("W,N,ffn_dim", [(5, 23, None), (32, 9, None), (4, 13, 24)])
def test_generation_equals_full_forward_bitwise(W, N, ffn_dim):
    p = make_params(W=W, ffn_dim=ffn_dim)
    x = RNG.standard_normal((2, N, 32))
    full, (kg, vg) = oracle.yoco_block(x, p)
    gen, (kg2, vg2), rings = oracle.yoco_block_generate(x, p)
    assert np.array_equal(gen, full)
    assert np.array_equal(kg2, kg) and np.array_equal(vg2, vg)
    # each ring holds the last W positions' K/V of its layer (slot t mod W):
    # recompute the self-decoder layer inputs of the full forward
    h = np.array(x, dtype=np.float64)
    for layer, ((wq, wk, wv, wo), (kr, vr)) in enumerate(zip(zip(p.swa_wq, p.swa_wk, p.swa_wv, p.swa_wo), rings)):
        n = _norm_rows(h, p.eps)
        k = _heads(linear_rows(n, wk), p.n_kv_heads, p.head_dim)
        v = _heads(linear_rows(n, wv), p.n_kv_heads, p.head_dim)
        for t in range(max(0, N - W), N):
            assert np.array_equal(kr[:, :, t % W], k[:, :, t])
            assert np.array_equal(vr[:, :, t % W], v[:, :, t])
        q = _heads(linear_rows(n, wq), p.n_heads, p.head_dim)
        o, _ = oracle.swa_attention(q, k, v, W)
        from oracle.block import _merge, _ffn_rows
        h = h + linear_rows(_merge(o), wo)
        h = _ffn_rows(h, p.ffn("swa", layer), p.eps)


def test_generation_catches_a_wrong_slot():
    """A ring indexed by t mod (W+1) instead of t mod W breaks the identity."""
    p = make_params(W=4)
    x = RNG.standard_normal((1, 11, 32))
    full, _ = oracle.yoco_block(x, p)
    import oracle.block as blk
    orig = blk.ring_window
    try:
        blk.ring_window = lambda pos, W: [(t, t % (W + 1)) for t in range(max(0, pos - W + 1), pos + 1)]
        with pytest.raises((IndexError, AssertionError)):
            gen, _, _ = blk.yoco_block_generate(x, p)
            assert np.array_equal(gen, full)
    finally:
        blk.ring_window = orig
