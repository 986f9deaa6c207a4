"""Pins for oracle/rope.py (rotary position embedding) and the block with RoPE.

* complex form: pair (x_2i, x_2i+1) as the complex number x_2i + i x_2i+1,
  multiplied by exp(i p theta^(-2i/d)) (torch complex arithmetic);
* the defining property: q_m . k_n depends on m - n only;
* each pair keeps its norm; position 0 is the identity; rotating by p then
  by -p returns the input; scalar 2x2 rotations on a tiny case;
* the block with RoPE: early exit, generation and causality identities
  still hold bitwise, and an independent torch composition agrees.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.rope import apply_rope, rope_inv_freq

RNG = np.random.default_rng(77)


def test_inverse_frequencies_closed_form():
    inv = rope_inv_freq(128, 10000.0)
    assert inv[0] == 1.0
    assert inv[1] == pytest.approx(10000.0 ** (-2 / 128), rel=1e-15)
    assert inv[-1] == pytest.approx(10000.0 ** (-126 / 128), rel=1e-15)
    with pytest.raises(ValueError):
        rope_inv_freq(7, 10.0)


@pytest.mark.parametrize("theta", [10000.0, 640e3, 80e6])
def test_matches_complex_rotation(theta):
    d, N, pos0 = 16, 9, 1000
    x = RNG.standard_normal((3, N, d))
    got = apply_rope(x, pos0, theta)
    z = torch.view_as_complex(torch.from_numpy(x.reshape(3, N, d // 2, 2)).contiguous())
    pos = torch.arange(pos0, pos0 + N, dtype=torch.float64)[:, None]
    inv = torch.tensor([theta ** (-2.0 * i / d) for i in range(d // 2)], dtype=torch.float64)
    ref = torch.view_as_real(z * torch.polar(torch.ones(N, d // 2, dtype=torch.float64), pos * inv)).reshape(3, N, d)
    assert np.allclose(got, ref.numpy(), atol=1e-12)


def test_scores_depend_on_the_offset_only():
    d, theta = 32, 10000.0
    q = RNG.standard_normal(d)
    k = RNG.standard_normal(d)
    def score(m, n):
        return float(apply_rope(q[None], m, theta)[0] @ apply_rope(k[None], n, theta)[0])
    for m, n in [(5, 2), (300, 17), (9, 9)]:
        for s in (1, 64, 1000):
            assert score(m + s, n + s) == pytest.approx(score(m, n), rel=1e-10, abs=1e-10)
    assert abs(score(5, 2) - score(5, 3)) > 1e-6


def test_norms_identity_and_inverse():
    d, theta = 64, 5e6
    x = RNG.standard_normal((2, 4, d))
    y = apply_rope(x, 123456, theta)
    assert np.allclose(np.hypot(y[..., 0::2], y[..., 1::2]), np.hypot(x[..., 0::2], x[..., 1::2]), atol=1e-12)
    assert np.array_equal(apply_rope(x, 0, theta)[..., 0, :], x[..., 0, :])
    back = np.stack([apply_rope(y[:, n:n + 1], -(123456 + n), theta)[:, 0] for n in range(4)], axis=1)
    assert np.allclose(back, x, atol=1e-9)


def test_scalar_rotations():
    d, theta, p = 4, 100.0, 3
    x = RNG.standard_normal(d)
    got = apply_rope(x[None], p, theta)[0]
    for i in range(d // 2):
        a = p * theta ** (-2 * i / d)
        R = [[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]]
        ref = [R[0][0] * x[2 * i] + R[0][1] * x[2 * i + 1], R[1][0] * x[2 * i] + R[1][1] * x[2 * i + 1]]
        assert got[2 * i] == pytest.approx(ref[0], abs=1e-14) and got[2 * i + 1] == pytest.approx(ref[1], abs=1e-14)


# ---------------------------------------------------------------- the block with RoPE
from test_oracle_block import make_params  # noqa: E402


def _rope_params(**kw):
    p = make_params(**kw)
    p.rope_theta = 500.0
    return p


def test_block_with_rope_early_exit_bitwise():
    p = _rope_params(ffn_dim=24)
    x = RNG.standard_normal((2, 19, 32))
    full, _ = oracle.yoco_block(x, p)
    last, _ = oracle.yoco_block_early_exit(x, p)
    assert np.array_equal(full[:, -1], last)


def test_block_with_rope_generation_bitwise():
    p = _rope_params(W=4)
    x = RNG.standard_normal((1, 11, 32))
    full, (kg, vg) = oracle.yoco_block(x, p)
    gen, (kg2, vg2), _ = oracle.yoco_block_generate(x, p)
    assert np.array_equal(gen, full) and np.array_equal(kg2, kg) and np.array_equal(vg2, vg)


def test_block_with_rope_is_causal_and_rope_matters():
    p = _rope_params()
    x = RNG.standard_normal((1, 16, 32))
    x2 = x.copy()
    x2[:, 9:] = 1e4
    a, _ = oracle.yoco_block(x, p)
    b, _ = oracle.yoco_block(x2, p)
    assert np.array_equal(a[:, :9], b[:, :9])
    p.rope_theta = 0.0
    c, _ = oracle.yoco_block(x, p)
    assert np.max(np.abs(a - c)) > 1e-3


def test_block_with_rope_matches_torch_composition():
    """The block with RoPE against an independent float64 torch composition
    (rotation as complex multiplication)."""
    p = _rope_params(D=48, Hq=6, Hkv=2, d=8, Ls=2, Lc=2, W=7, ffn_dim=40)
    x = RNG.standard_normal((2, 21, 48))
    out, _ = oracle.yoco_block(x, p)
    F = torch.nn.functional
    t = lambda a: torch.from_numpy(np.asarray(a))  # noqa: E731
    X = t(x)
    B, N, D = X.shape
    Hq, Hkv, d, W = p.n_heads, p.n_kv_heads, p.head_dim, p.window
    g = Hq // Hkv
    ii = torch.arange(N)
    swa = (ii[None, :] <= ii[:, None]) & (ii[None, :] > ii[:, None] - W)
    causal = ii[None, :] <= ii[:, None]
    inv = torch.tensor([p.rope_theta ** (-2.0 * i / d) for i in range(d // 2)], dtype=torch.float64)
    rot = torch.polar(torch.ones(N, d // 2, dtype=torch.float64), ii[:, None].double() * inv)

    def rope(y):   # y [B, H, N, d]
        z = torch.view_as_complex(y.reshape(*y.shape[:-1], d // 2, 2).contiguous())
        return torch.view_as_real(z * rot).reshape(y.shape)

    split = lambda y, h: y.view(B, N, h, d).permute(0, 2, 1, 3)  # noqa: E731
    merge = lambda o: o.permute(0, 2, 1, 3).reshape(B, N, Hq * d)  # noqa: E731

    def ffn(X, w):
        n = F.rms_norm(X, (D,), eps=p.eps)
        return X + F.linear(F.silu(F.linear(n, t(w[0]))) * F.linear(n, t(w[1])), t(w[2]))

    for layer, (wq, wk, wv, wo) in enumerate(zip(p.swa_wq, p.swa_wk, p.swa_wv, p.swa_wo)):
        n = F.rms_norm(X, (D,), eps=p.eps)
        q, k, v = rope(split(F.linear(n, t(wq)), Hq)), rope(split(F.linear(n, t(wk)), Hkv)), split(F.linear(n, t(wv)), Hkv)
        o = F.scaled_dot_product_attention(q, k.repeat_interleave(g, 1), v.repeat_interleave(g, 1), attn_mask=swa)
        X = ffn(X + F.linear(merge(o), t(wo)), p.swa_ffn[layer])
    n = F.rms_norm(X, (D,), eps=p.eps)
    K, V = rope(split(F.linear(n, t(p.glob_wk)), Hkv)), split(F.linear(n, t(p.glob_wv)), Hkv)
    for layer, (wq, wo) in enumerate(zip(p.cross_wq, p.cross_wo)):
        q = rope(split(F.linear(F.rms_norm(X, (D,), eps=p.eps), t(wq)), Hq))
        o = F.scaled_dot_product_attention(q, K.repeat_interleave(g, 1), V.repeat_interleave(g, 1), attn_mask=causal)
        X = ffn(X + F.linear(merge(o), t(wo)), p.cross_ffn[layer])
    assert np.max(np.abs(out - X.numpy())) < 1e-11
