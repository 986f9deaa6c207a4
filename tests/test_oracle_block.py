"""Pins for oracle/block.py: the tiny YOCO block.

* early exit: the last position's output with the cross-decoder run on every
  position equals, bitwise, running it on the last position only;
* sharing: cross layers reading one cache equal layers reading their own
  duplicated copies, bitwise;
* causality of the whole block, bitwise;
* library routine: an independent float64 torch composition (rms_norm,
  linear, scaled_dot_product_attention with explicit masks, silu for the
  SwiGLU feed-forward), with and without the feed-forward;
* the SwiGLU pieces: silu against torch's over the whole float64 range, and
  the feed-forward's early-exit and causality identities.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.block import BlockParams, linear_rows

RNG = np.random.default_rng(2024)


def make_params(D=32, Hq=4, Hkv=2, d=8, Ls=2, Lc=2, W=5, std=None, ffn_dim=None):
    std = std or 1 / math.sqrt(D)
    r = lambda *s: RNG.standard_normal(s) * std  # noqa: E731
    ffn = (lambda: (r(ffn_dim, D), r(ffn_dim, D), r(D, ffn_dim) * math.sqrt(D / ffn_dim))) if ffn_dim else None
    return BlockParams(
        n_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=W,
        swa_wq=[r(Hq * d, D) for _ in range(Ls)], swa_wk=[r(Hkv * d, D) for _ in range(Ls)],
        swa_wv=[r(Hkv * d, D) for _ in range(Ls)], swa_wo=[r(D, Hq * d) for _ in range(Ls)],
        glob_wk=r(Hkv * d, D), glob_wv=r(Hkv * d, D),
        cross_wq=[r(Hq * d, D) for _ in range(Lc)], cross_wo=[r(D, Hq * d) for _ in range(Lc)],
        swa_ffn=[ffn() for _ in range(Ls)] if ffn else [],
        cross_ffn=[ffn() for _ in range(Lc)] if ffn else [])


@pytest.mark.parametrize("ffn_dim", [None, 24])
def test_early_exit_is_bitwise_exact(ffn_dim):
    p = make_params(ffn_dim=ffn_dim)
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


@pytest.mark.parametrize("ffn_dim", [None, 40])
@pytest.mark.parametrize("t_star", [3, 15])
def test_block_causality_bitwise(t_star, ffn_dim):
    p = make_params(ffn_dim=ffn_dim)
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
    def ffn(X, w):
        if w is None:
            return X
        n = F.rms_norm(X, (D,), eps=p.eps)
        return X + F.linear(F.silu(F.linear(n, t(w[0]))) * F.linear(n, t(w[1])), t(w[2]))

    for layer, (wq, wk, wv, wo) in enumerate(zip(p.swa_wq, p.swa_wk, p.swa_wv, p.swa_wo)):
        n = F.rms_norm(X, (D,), eps=p.eps)
        q, k, v = split(F.linear(n, t(wq)), Hq), split(F.linear(n, t(wk)), Hkv), split(F.linear(n, t(wv)), Hkv)
        o = F.scaled_dot_product_attention(q, k.repeat_interleave(g, 1), v.repeat_interleave(g, 1), attn_mask=swa)
        X = X + F.linear(o.permute(0, 2, 1, 3).reshape(B, N, Hq * d), t(wo))
        X = ffn(X, p.swa_ffn[layer] if p.swa_ffn else None)
    n = F.rms_norm(X, (D,), eps=p.eps)
    K, V = split(F.linear(n, t(p.glob_wk)), Hkv), split(F.linear(n, t(p.glob_wv)), Hkv)
    for layer, (wq, wo) in enumerate(zip(p.cross_wq, p.cross_wo)):
        q = split(F.linear(F.rms_norm(X, (D,), eps=p.eps), t(wq)), Hq)
        o = F.scaled_dot_product_attention(q, K.repeat_interleave(g, 1), V.repeat_interleave(g, 1), attn_mask=causal)
        X = X + F.linear(o.permute(0, 2, 1, 3).reshape(B, N, Hq * d), t(wo))
        X = ffn(X, p.cross_ffn[layer] if p.cross_ffn else None)
    return X.numpy()


@pytest.mark.parametrize("ffn_dim", [None, 56])
def test_block_matches_independent_torch_composition(ffn_dim):
    p = make_params(D=48, Hq=6, Hkv=2, d=8, Ls=2, Lc=3, W=7, ffn_dim=ffn_dim)
    x = RNG.standard_normal((2, 30, 48))
    out, _ = oracle.yoco_block(x, p)
    assert np.max(np.abs(out - _torch_block(x, p))) < 1e-11


def test_feed_forward_changes_the_block():
    """The feed-forward is really applied (a dropped term would leave the
    block equal to the attention-only one)."""
    p = make_params(ffn_dim=24)
    x = RNG.standard_normal((1, 9, 32))
    with_ffn, _ = oracle.yoco_block(x, p)
    p.swa_ffn, p.cross_ffn = [], []
    without, _ = oracle.yoco_block(x, p)
    assert np.max(np.abs(with_ffn - without)) > 1e-2


def test_silu_matches_torch_over_the_float64_range():
    z = np.concatenate([np.linspace(-800, 800, 3201), RNG.standard_normal(200) * 6, [0.0, -0.0, 1e-300, -1e-300]])
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    with np.errstate(over="raise", invalid="raise", divide="raise"):
        got = oracle.silu(z)
    assert np.allclose(got, ref, rtol=1e-15, atol=1e-300)
    # closed forms: silu(0) = 0, silu(z) -> z for z >> 0, -> 0 for z << 0
    assert oracle.silu(0.0) == 0.0 and oracle.silu(800.0) == 800.0 and oracle.silu(-800.0) == 0.0


def test_swiglu_row_brute_force():
    D, F = 5, 3
    wg, wu, wd = RNG.standard_normal((F, D)), RNG.standard_normal((F, D)), RNG.standard_normal((D, F))
    x = RNG.standard_normal(D)
    ms = sum(v * v for v in x) / D
    n = [v / math.sqrt(ms + 1e-6) for v in x]
    hid = []
    for j in range(F):
        a = sum(wg[j, i] * n[i] for i in range(D))
        b = sum(wu[j, i] * n[i] for i in range(D))
        hid.append(a / (1 + math.exp(-a)) * b)
    ref = [x[i] + sum(wd[i, j] * hid[j] for j in range(F)) for i in range(D)]
    assert np.allclose(oracle.swiglu_ffn_row(x, (wg, wu, wd), 1e-6), ref, atol=1e-13)


# ---------------------------------------------------------------------------
# The block with a gated-retention self-decoder
# ---------------------------------------------------------------------------
def make_gret_params(D=32, H=4, Hkv=2, d=8, Ls=2, Lc=2, ffn_dim=None, tau=4.0):
    p = make_params(D=D, Hq=H, Hkv=Hkv, d=d, Ls=Ls, Lc=Lc, ffn_dim=ffn_dim)
    std = 1 / math.sqrt(D)
    r = lambda *s: RNG.standard_normal(s) * std  # noqa: E731
    p.self_kind = "gret"
    p.swa_wk = [r(H * d, D) for _ in range(Ls)]
    p.swa_wv = [r(H * d, D) for _ in range(Ls)]
    p.gret_wz = [r(H, D) * 6 for _ in range(Ls)]        # gate logits of order +-6: decays from ~0 to ~1
    p.gret_wg = [r(H * d, D) for _ in range(Ls)]
    p.gret_tau = tau
    return p


@pytest.mark.parametrize("ffn_dim", [None, 24])
def test_gret_block_early_exit_and_generation_are_bitwise(ffn_dim):
    p = make_gret_params(ffn_dim=ffn_dim)
    x = RNG.standard_normal((2, 21, 32))
    full, (kf, vf) = oracle.yoco_block(x, p)
    last, _ = oracle.yoco_block_early_exit(x, p)
    gen, (kg, vg), _ = oracle.yoco_block_generate(x, p)
    assert np.array_equal(full[:, -1], last)
    assert np.array_equal(full, gen) and np.array_equal(kf, kg) and np.array_equal(vf, vg)


def test_gret_block_causality_bitwise():
    p = make_gret_params(ffn_dim=16)
    x = RNG.standard_normal((1, 18, 32))
    x2 = x.copy()
    x2[:, 10:] = -1e4
    a, _ = oracle.yoco_block(x, p)
    b, _ = oracle.yoco_block(x2, p)
    assert np.array_equal(a[:, :10], b[:, :10])


def _torch_gret_block(x, p):
    """Independent composition: gated retention in its parallel form with an
    explicit decay matrix built from torch's logsigmoid, GroupNorm from
    torch.nn.functional.group_norm, swish from silu."""
    t = lambda a: torch.from_numpy(np.asarray(a))  # noqa: E731
    X = t(x)
    B, N, D = X.shape
    H, Hkv, d = p.n_heads, p.n_kv_heads, p.head_dim
    g = H // Hkv
    F = torch.nn.functional
    split = lambda y, h: y.view(B, N, h, d).permute(0, 2, 1, 3)  # noqa: E731
    causal = torch.arange(N)[None, :] <= torch.arange(N)[:, None]
    for layer in range(len(p.swa_wq)):
        n = F.rms_norm(X, (D,), eps=p.eps)
        q, k, v = (split(F.linear(n, t(w[layer])), H) for w in (p.swa_wq, p.swa_wk, p.swa_wv))
        lg = F.logsigmoid(F.linear(n, t(p.gret_wz[layer]))).permute(0, 2, 1) / p.gret_tau   # [B, H, N]
        c = torch.cumsum(lg, dim=-1)
        dec = torch.exp(c[..., :, None] - c[..., None, :]).masked_fill(~causal, 0.0)
        y = (q @ k.transpose(-1, -2) * dec) @ v                                            # [B, H, N, d]
        yn = F.group_norm(y.permute(0, 2, 1, 3).reshape(B * N, H * d), H, eps=p.eps).view(B, N, H * d)
        X = X + F.linear(F.silu(F.linear(n, t(p.gret_wg[layer]))) * yn, t(p.swa_wo[layer]))
        if p.swa_ffn:
            wg_, wu_, wd_ = p.swa_ffn[layer]
            n2 = F.rms_norm(X, (D,), eps=p.eps)
            X = X + F.linear(F.silu(F.linear(n2, t(wg_))) * F.linear(n2, t(wu_)), t(wd_))
    n = F.rms_norm(X, (D,), eps=p.eps)
    K, V = split(F.linear(n, t(p.glob_wk)), Hkv), split(F.linear(n, t(p.glob_wv)), Hkv)
    for layer, (wq, wo) in enumerate(zip(p.cross_wq, p.cross_wo)):
        qq = split(F.linear(F.rms_norm(X, (D,), eps=p.eps), t(wq)), H)
        o = F.scaled_dot_product_attention(qq, K.repeat_interleave(g, 1), V.repeat_interleave(g, 1), attn_mask=causal)
        X = X + F.linear(o.permute(0, 2, 1, 3).reshape(B, N, H * d), t(wo))
        if p.cross_ffn:
            wg_, wu_, wd_ = p.cross_ffn[layer]
            n2 = F.rms_norm(X, (D,), eps=p.eps)
            X = X + F.linear(F.silu(F.linear(n2, t(wg_))) * F.linear(n2, t(wu_)), t(wd_))
    return X.numpy()


@pytest.mark.parametrize("ffn_dim", [None, 40])
def test_gret_block_matches_independent_torch_composition(ffn_dim):
    p = make_gret_params(D=48, H=6, Hkv=2, d=8, Ls=2, Lc=2, ffn_dim=ffn_dim, tau=3.0)
    x = RNG.standard_normal((2, 26, 48))
    out, _ = oracle.yoco_block(x, p)
    assert np.max(np.abs(out - _torch_gret_block(x, p))) < 1e-10


def test_gret_self_decoder_differs_from_the_window_one():
    """The gated-retention branch is really taken (same weights, window layers
    instead: a different block)."""
    p = make_gret_params()
    x = RNG.standard_normal((1, 12, 32))
    a, _ = oracle.yoco_block(x, p)
    p.self_kind = "swa"
    p.n_kv_heads = p.n_heads   # window layers with the same [H*d, D] K/V weights
    p.glob_wk = np.vstack([p.glob_wk, p.glob_wk])
    p.glob_wv = np.vstack([p.glob_wv, p.glob_wv])
    b, _ = oracle.yoco_block(x, p)
    assert np.max(np.abs(a - b)) > 1e-2
