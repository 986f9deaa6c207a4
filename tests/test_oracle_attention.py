"""Pins for oracle/attention.py against things other than itself.

* library routine: torch's scaled_dot_product_attention in float64 on the CPU
  with an explicit boolean mask built here from the mask definitions;
* brute force: scalar pure-Python loops on tiny inputs;
* closed forms: zero queries (uniform softmax), window 1, constant values,
  a single key, a planted dominant key;
* the method's invariants: causality and window locality (bitwise), grouped
  heads equal repeated heads, sliding window >= N equals causal, softmax rows
  sum to one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import attend_row

RNG = np.random.default_rng(1234)


def _rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def _sdpa(q, k, v, mask):
    """torch SDPA in float64 with K/V heads repeated for the query groups."""
    g = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(k).repeat_interleave(g, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(g, dim=1)
    mt = torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt).numpy()


def _swa_mask(n, w):
    t = np.arange(n)[:, None]
    s = np.arange(n)[None, :]
    return (s <= t) & (s > t - w)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,W", [
    (1, 4, 1, 37, 16, 5), (2, 6, 2, 50, 32, 1), (1, 3, 3, 40, 8, 64),
    (2, 8, 2, 65, 16, 16), (1, 4, 4, 33, 64, 33)])
def test_swa_matches_torch_sdpa(B, Hq, Hkv, N, d, W):
    q, k, v = _rand(B, Hq, N, d), _rand(B, Hkv, N, d), _rand(B, Hkv, N, d)
    o, lse = oracle.swa_attention(q, k, v, W)
    ref = _sdpa(q, k, v, _swa_mask(N, W))
    assert np.max(np.abs(o - ref)) < 1e-12
    # LSE against torch.logsumexp of the masked scores
    g = Hq // Hkv
    kk = np.repeat(k, g, axis=1)
    z = np.einsum("bhtd,bhsd->bhts", q, kk) / math.sqrt(d)
    z = np.where(_swa_mask(N, W)[None, None], z, -np.inf)
    lse_ref = torch.logsumexp(torch.from_numpy(z), dim=-1).numpy()
    assert np.max(np.abs(lse - lse_ref)) < 1e-12


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nkv,ncap,off,d", [
    (1, 4, 1, 30, 30, 30, 0, 16), (2, 6, 2, 9, 41, 48, 32, 32),
    (1, 3, 1, 1, 25, 25, 24, 8), (2, 8, 4, 17, 17, 20, 0, 64)])
def test_cross_prefill_matches_torch_sdpa(B, Hq, Hkv, Nq, Nkv, ncap, off, d):
    q = _rand(B, Hq, Nq, d)
    k, v = _rand(B, Hkv, ncap, d), _rand(B, Hkv, ncap, d)
    o, _ = oracle.cross_prefill_attention(q, k, v, n_kv=Nkv, q_offset=off)
    mask = np.arange(ncap)[None, :] <= (off + np.arange(Nq))[:, None]
    ref = _sdpa(q, k, v, mask)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_decode_matches_torch_sdpa_ragged():
    B, Hq, Hkv, ncap, d = 3, 8, 2, 70, 32
    ctx = np.array([70, 1, 33])
    q = _rand(B, Hq, d)
    k, v = _rand(B, Hkv, ncap, d), _rand(B, Hkv, ncap, d)
    o, lse = oracle.decode_attention(q, k, v, ctx)
    for b in range(B):
        mask = (np.arange(ncap) < ctx[b])[None, :]
        ref = _sdpa(q[b:b + 1, :, None, :], k[b:b + 1], v[b:b + 1], mask)[0, :, 0]
        assert np.max(np.abs(o[b] - ref)) < 1e-12


def _brute_row(qv, krows, vrows, scale):
    zs = [scale * sum(a * b for a, b in zip(qv, kr)) for kr in krows]
    m = max(zs)
    es = [math.exp(z - m) for z in zs]
    tot = sum(es)
    out = [sum(es[j] * vrows[j][c] for j in range(len(es))) / tot for c in range(len(qv))]
    return out, m + math.log(tot)


def test_brute_force_scalar_loops():
    B, Hq, Hkv, N, d, W = 1, 4, 2, 12, 4, 5
    q, k, v = _rand(B, Hq, N, d), _rand(B, Hkv, N, d), _rand(B, Hkv, N, d)
    o, lse = oracle.swa_attention(q, k, v, W)
    oc, lsec = oracle.cross_prefill_attention(q, k, v)
    scale = 1 / math.sqrt(d)
    for h in range(Hq):
        kvh = h // (Hq // Hkv)
        for t in range(N):
            keys = [s for s in range(N) if t - W < s <= t]
            ref, lref = _brute_row(q[0, h, t], [k[0, kvh, s] for s in keys],
                                   [v[0, kvh, s] for s in keys], scale)
            assert np.max(np.abs(o[0, h, t] - ref)) < 1e-12
            assert abs(lse[0, h, t] - lref) < 1e-12
            keys = list(range(t + 1))
            ref, lref = _brute_row(q[0, h, t], [k[0, kvh, s] for s in keys],
                                   [v[0, kvh, s] for s in keys], scale)
            assert np.max(np.abs(oc[0, h, t] - ref)) < 1e-12
            assert abs(lsec[0, h, t] - lref) < 1e-12


def test_zero_queries_give_window_mean_and_log_count():
    B, Hq, Hkv, N, d, W = 1, 2, 1, 20, 8, 6
    q = np.zeros((B, Hq, N, d))
    k, v = _rand(B, Hkv, N, d), _rand(B, Hkv, N, d)
    o, lse = oracle.swa_attention(q, k, v, W)
    for t in range(N):
        lo = max(0, t - W + 1)
        np.testing.assert_allclose(o[0, 0, t], v[0, 0, lo:t + 1].mean(axis=0), atol=1e-14)
        assert abs(lse[0, 0, t] - math.log(t + 1 - lo)) < 1e-14


def test_window_one_returns_own_value():
    q, k, v = _rand(1, 3, 15, 8), _rand(1, 3, 15, 8), _rand(1, 3, 15, 8)
    o, lse = oracle.swa_attention(q, k, v, 1)
    assert np.array_equal(o, v)
    np.testing.assert_allclose(lse, np.einsum("bhtd,bhtd->bht", q, k) / math.sqrt(8), atol=1e-14)


def test_constant_values_give_constant_output():
    q, k = _rand(2, 4, 25, 16) * 3, _rand(2, 2, 25, 16) * 3
    v = np.ones((2, 2, 25, 16))
    for o, _ in (oracle.swa_attention(q, k, v, 7), oracle.cross_prefill_attention(q, k, v)):
        assert np.max(np.abs(o - 1.0)) < 1e-14


def test_single_key_and_first_row():
    q, k, v = _rand(1, 2, 10, 8), _rand(1, 1, 10, 8), _rand(1, 1, 10, 8)
    o, lse = oracle.cross_prefill_attention(q, k, v)
    assert np.array_equal(o[0, :, 0], np.repeat(v[0, :, 0], 2, axis=0))
    od, _ = oracle.decode_attention(q[:, :, 5], k, v, [1])
    assert np.array_equal(od[0], np.repeat(v[0, :, 0], 2, axis=0))


def test_planted_key_dominates():
    B, Hq, Hkv, n, d = 1, 4, 1, 300, 32
    q = _rand(B, Hq, d)
    k, v = _rand(B, Hkv, n, d), _rand(B, Hkv, n, d)
    s_star = 123
    # one key aligned with all four queries, strongly: its logit is ~60 above the rest
    k[0, 0, s_star] = 60.0 * math.sqrt(d) * q[0].sum(axis=0) / np.dot(q[0].sum(0), q[0].sum(0)) * 4
    o, _ = oracle.decode_attention(q, k, v, [n])
    assert np.max(np.abs(o[0] - v[0, 0, s_star])) < 1e-6


def test_window_at_least_n_equals_causal_bitwise():
    q, k, v = _rand(2, 4, 30, 16), _rand(2, 2, 30, 16), _rand(2, 2, 30, 16)
    o1, l1 = oracle.swa_attention(q, k, v, 30)
    o2, l2 = oracle.swa_attention(q, k, v, 1000)
    o3, l3 = oracle.cross_prefill_attention(q, k, v)
    assert np.array_equal(o1, o3) and np.array_equal(o2, o3)
    assert np.array_equal(l1, l3)


def test_gqa_equals_mha_with_repeated_kv_bitwise():
    q, k, v = _rand(2, 6, 21, 16), _rand(2, 2, 21, 16), _rand(2, 2, 21, 16)
    o1, _ = oracle.swa_attention(q, k, v, 9)
    o2, _ = oracle.swa_attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 9)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("t_star", [0, 7, 18])
def test_causality_bitwise(t_star):
    N = 24
    q, k, v = _rand(1, 4, N, 16), _rand(1, 2, N, 16), _rand(1, 2, N, 16)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for t in (q2, k2, v2):
        t[:, :, t_star + 1:] = RNG.choice([-1e4, 1e4], size=t[:, :, t_star + 1:].shape)
    for fn in (lambda a, b, c: oracle.swa_attention(a, b, c, 8),
               lambda a, b, c: oracle.cross_prefill_attention(a, b, c)):
        o1, l1 = fn(q, k, v)
        o2, l2 = fn(q2, k2, v2)
        assert np.array_equal(o1[:, :, :t_star + 1], o2[:, :, :t_star + 1])
        assert np.array_equal(l1[:, :, :t_star + 1], l2[:, :, :t_star + 1])


def test_decode_ignores_rows_beyond_ctx_bitwise():
    q, k, v = _rand(2, 4, 16), _rand(2, 1, 40, 16), _rand(2, 1, 40, 16)
    o1, l1 = oracle.decode_attention(q, k, v, [25, 40])
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 25:] = 1e4
    v2[0, :, 25:] = np.nan
    o2, l2 = oracle.decode_attention(q, k2, v2, [25, 40])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_window_locality_bitwise():
    N, W = 30, 6
    q, k, v = _rand(1, 2, N, 8), _rand(1, 1, N, 8), _rand(1, 1, N, 8)
    o1, _ = oracle.swa_attention(q, k, v, W)
    t = 20
    k2, v2 = k.copy(), v.copy()
    k2[:, :, :t - W + 1] = 1e4
    v2[:, :, :t - W + 1] = -1e4
    o2, _ = oracle.swa_attention(q, k2, v2, W)
    assert np.array_equal(o1[:, :, t:], o2[:, :, t:])
    assert not np.array_equal(o1[:, :, t - 1], o2[:, :, t - 1])


def test_softmax_rows_sum_to_one():
    for n in (1, 2, 17, 500):
        qv = RNG.standard_normal(64) * 4
        kr, vr = RNG.standard_normal((n, 64)) * 4, RNG.standard_normal((n, 64))
        _, _, p = attend_row(qv, kr, vr, 1 / 8)
        assert abs(p.sum() - 1.0) < 1e-12
        assert np.all(p >= 0)


def test_row_subsets_are_exact_samples():
    q, k, v = _rand(2, 4, 40, 16), _rand(2, 2, 40, 16), _rand(2, 2, 40, 16)
    full, lfull = oracle.swa_attention(q, k, v, 11)
    rows = [0, 10, 39]
    part, lpart = oracle.swa_attention(q, k, v, 11, rows=rows, bh=[(1, 3), (0, 0)])
    for b, h in [(1, 3), (0, 0)]:
        assert np.array_equal(part[b, h, rows], full[b, h, rows])
    assert np.isnan(part[0, 1]).all()


def test_rejects_bad_arguments():
    q, k = _rand(1, 3, 5, 4), _rand(1, 2, 5, 4)
    with pytest.raises(ValueError):
        oracle.swa_attention(q, k, k, 2)
    with pytest.raises(ValueError):
        oracle.swa_attention(_rand(1, 2, 5, 4), k, k, 0)
    with pytest.raises(ValueError):
        oracle.cross_prefill_attention(_rand(1, 2, 5, 4), k, k, n_kv=5, q_offset=1)
    with pytest.raises(ValueError):
        oracle.decode_attention(_rand(1, 2, 4), k, k, [0])
