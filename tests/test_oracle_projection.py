"""Pins for oracle/projection.py.

* library routine: torch.nn.functional.rms_norm / linear in float64;
* closed forms: constant rows, the mean square of a normalised row;
* layout: selection-matrix weights put known inputs at known
  (KV head, channel) positions of the head-major cache.
"""
import math

import numpy as np
import torch

import oracle

RNG = np.random.default_rng(99)


def test_rmsnorm_matches_torch():
    x = RNG.standard_normal((7, 33)) * 3
    gamma = RNG.standard_normal(33)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(gamma), eps=1e-6)
    assert np.max(np.abs(oracle.rmsnorm(x, gamma) - ref.numpy())) < 1e-13


def test_rmsnorm_closed_forms():
    c = -2.5
    y = oracle.rmsnorm_row(np.full(10, c))
    assert np.allclose(y, c / math.sqrt(c * c + 1e-6), rtol=0, atol=1e-15)
    x = RNG.standard_normal(64)
    y = oracle.rmsnorm_row(x, eps=1e-6)
    ms = np.mean(x * x)
    assert abs(np.mean(y * y) - ms / (ms + 1e-6)) < 1e-13
    assert np.allclose(oracle.rmsnorm_row(5 * x, eps=0.0), oracle.rmsnorm_row(x, eps=0.0), atol=1e-14)


def test_global_kv_proj_matches_torch():
    B, N, D, Hkv, d = 2, 9, 40, 3, 8
    x = RNG.standard_normal((B, N, D))
    wk, wv = RNG.standard_normal((Hkv * d, D)) * 0.2, RNG.standard_normal((Hkv * d, D)) * 0.2
    k, v = oracle.global_kv_proj(x, wk, wv, Hkv, d)
    n = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), eps=1e-6)
    kr = torch.nn.functional.linear(n, torch.from_numpy(wk)).view(B, N, Hkv, d).permute(0, 2, 1, 3)
    vr = torch.nn.functional.linear(n, torch.from_numpy(wv)).view(B, N, Hkv, d).permute(0, 2, 1, 3)
    assert np.max(np.abs(k - kr.numpy())) < 1e-12
    assert np.max(np.abs(v - vr.numpy())) < 1e-12


def test_global_kv_proj_layout_with_selection_weights():
    B, N, D, Hkv, d = 1, 5, 12, 2, 3
    x = RNG.standard_normal((B, N, D))
    perm = RNG.permutation(D)[:Hkv * d]
    wk = np.zeros((Hkv * d, D))
    wk[np.arange(Hkv * d), perm] = 1.0
    wv = 2.0 * wk
    k, v = oracle.global_kv_proj(x, wk, wv, Hkv, d)
    n = oracle.rmsnorm(x)
    for h in range(Hkv):
        for c in range(d):
            for t in range(N):
                assert k[0, h, t, c] == n[0, t, perm[h * d + c]]
                assert v[0, h, t, c] == 2.0 * n[0, t, perm[h * d + c]]


def test_global_kv_proj_row_subset_is_exact():
    x = RNG.standard_normal((2, 11, 16))
    wk, wv = RNG.standard_normal((8, 16)), RNG.standard_normal((8, 16))
    kf, vf = oracle.global_kv_proj(x, wk, wv, 2, 4)
    ks, vs = oracle.global_kv_proj(x, wk, wv, 2, 4, rows=[3, 10])
    assert np.array_equal(ks[:, :, [3, 10]], kf[:, :, [3, 10]])
    assert np.isnan(ks[:, :, 0]).all()
