"""Pins for oracle/block.py: the tiny YOCO block.

* early exit: the last position's output with the cross-decoder run on every
  position equals, bitwise, running it on the last position only;
* sharing: cross layers reading one cache equal layers reading their own
  duplicated copies, bitwise;
* causality of the whole block, bitwise;
* library routine: an independent float64 torch composition (rms_norm,
  linear, scaled_dot_product_attention with explicit masks).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.block import BlockParams, linear_rows

RNG = np.random.default_rng(2024)


def make_params(D=32, Hq=4, Hkv=2, d=8, Ls=2, Lc=2, W=5, std=None):
    std = std or 1 / math.sqrt(D)
    r = lambda *s: RNG.standard_normal(s) * std  # noqa: E731
    return BlockParams(
        n_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=W,
        swa_wq=[r(Hq * d, D) for _ in range(Ls)], swa_wk=[r(Hkv * d, D) for _ in range(Ls)],
        swa_wv=[r(Hkv * d, D) for _ in range(Ls)], swa_wo=[r(D, Hq * d) for _ in range(Ls)],
        glob_wk=r(Hkv * d, D), glob_wv=r(Hkv * d, D),
        cross_wq=[r(Hq * d, D) for _ in range(Lc)], cross_wo=[r(D, Hq * d) for _ in range(Lc)])


def test_early_exit_is_bitwise_exact():
    p = make_params()
    x = RNG.standard_normal((2, 23, 32))
    full, _ = oracle.yoco_block(x, p)
    last, _ = oracle.yoco_block_early_exit(x, p)
    assert np.array_equal(full[:, -1], last)


def test_sharing_equals_duplicated_caches_bitwise():
    p = make_params()
    x = RNG.standard_normal((1, 17, 32))
    out, (kg, vg) = oracle.yoco_block(x, p)
    # rebuild the cross-decoder with a private copy of the cache for each layer
    xs = x.copy()
    # recompute the self-decoder output through the early-exit path's helper
    from oracle.block import _self_decoder_and_projection, _norm_rows, _heads, _merge
    xs, k1, v1 = _self_decoder_and_projection(xs, p)
    for wq, wo in zip(p.cross_wq, p.cross_wo):
        kc, vc = k1.copy(), v1.copy()
        q = _heads(linear_rows(_norm_rows(xs, p.eps), wq), p.n_heads, p.head_dim)
        o, _ = oracle.cross_prefill_attention(q, kc, vc)
        xs = xs + linear_rows(_merge(o), wo)
    assert np.array_equal(out, xs)


@pytest.mark.parametrize("t_star", [3, 15])
def test_block_causality_bitwise(t_star):
    p = make_params()
    x = RNG.standard_normal((1, 20, 32))
    x2 = x.copy()
    x2[:, t_star + 1:] = 1e4
    a, (ka, va) = oracle.yoco_block(x, p)
    b, (kb, vb) = oracle.yoco_block(x2, p)
    assert np.array_equal(a[:, :t_star + 1], b[:, :t_star + 1])
    assert np.array_equal(ka[:, :, :t_star + 1], kb[:, :, :t_star + 1])


def _torch_block(x, p):
    t = lambda a: torch.from_numpy(np.asarray(a))  # noqa: E731
    X = t(x)
    B, N, D = X.shape
    Hq, Hkv, d, W = p.n_heads, p.n_kv_heads, p.head_dim, p.window
    g = Hq // Hkv
    ii = torch.arange(N)
    swa = (ii[None, :] <= ii[:, None]) & (ii[None, :] > ii[:, None] - W)
    causal = ii[None, :] <= ii[:, None]
    F = torch.nn.functional
    split = lambda y, h: y.view(B, N, h, d).permute(0, 2, 1, 3)  # noqa: E731
    for wq, wk, wv, wo in zip(p.swa_wq, p.swa_wk, p.swa_wv, p.swa_wo):
        n = F.rms_norm(X, (D,), eps=p.eps)
        q, k, v = split(F.linear(n, t(wq)), Hq), split(F.linear(n, t(wk)), Hkv), split(F.linear(n, t(wv)), Hkv)
        o = F.scaled_dot_product_attention(q, k.repeat_interleave(g, 1), v.repeat_interleave(g, 1), attn_mask=swa)
        X = X + F.linear(o.permute(0, 2, 1, 3).reshape(B, N, Hq * d), t(wo))
    n = F.rms_norm(X, (D,), eps=p.eps)
    K, V = split(F.linear(n, t(p.glob_wk)), Hkv), split(F.linear(n, t(p.glob_wv)), Hkv)
    for wq, wo in zip(p.cross_wq, p.cross_wo):
        q = split(F.linear(F.rms_norm(X, (D,), eps=p.eps), t(wq)), Hq)
        o = F.scaled_dot_product_attention(q, K.repeat_interleave(g, 1), V.repeat_interleave(g, 1), attn_mask=causal)
        X = X + F.linear(o.permute(0, 2, 1, 3).reshape(B, N, Hq * d), t(wo))
    return X.numpy()


def test_block_matches_independent_torch_composition():
    p = make_params(D=48, Hq=6, Hkv=2, d=8, Ls=2, Lc=3, W=7)
    x = RNG.standard_normal((2, 30, 48))
    out, _ = oracle.yoco_block(x, p)
    assert np.max(np.abs(out - _torch_block(x, p))) < 1e-11
