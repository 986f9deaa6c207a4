"""Pins for oracle/retention.py (gated retention).

* the pages' own invariant: the recurrent, parallel and chunkwise forms give
  the same result (any chunk size, with and without an initial state);
* library routines: torch logsigmoid for the log decay, torch group_norm and
  silu for the head normalisation and swish gate;
* closed forms: gate 1 (z -> +inf, or tau -> inf) is causal linear attention
  written out as tril(Q K^T) V; gate 0 (z -> -inf) keeps only the current
  token, o_n = (q_n . k_n) v_n; a constant gate g gives D[n, m] = g^(n-m);
* brute force: scalar loops on a tiny case;
* state hand-over: running N1 positions, then the rest from the returned
  state, equals one run over all N positions.
"""
import math

import numpy as np
import pytest
import torch

import oracle.retention as R

RNG = np.random.default_rng(4242)


def _inputs(B=2, H=3, N=19, dk=5, dv=4, zscale=2.0):
    q = RNG.standard_normal((B, H, N, dk))
    k = RNG.standard_normal((B, H, N, dk))
    v = RNG.standard_normal((B, H, N, dv))
    z = RNG.standard_normal((B, H, N)) * zscale + 1.0
    return q, k, v, z


@pytest.mark.parametrize("tau", [1.0, 16.0, 0.5])
@pytest.mark.parametrize("with_state", [False, True])
def test_three_forms_agree(tau, with_state):
    q, k, v, z = _inputs()
    s0 = RNG.standard_normal((2, 3, 5, 4)) if with_state else None
    o_r, st_r = R.gret_recurrent(q, k, v, z, tau, s0)
    o_p = R.gret_parallel(q, k, v, z, tau, s0)
    assert np.allclose(o_p, o_r, atol=1e-12, rtol=1e-12)
    for chunk in (1, 3, 4, 7, 19, 64):
        o_c, st_c = R.gret_chunkwise(q, k, v, z, tau, chunk, s0)
        assert np.allclose(o_c, o_r, atol=1e-12, rtol=1e-12), chunk
        assert np.allclose(st_c, st_r, atol=1e-12, rtol=1e-12), chunk


def test_log_decay_matches_torch_logsigmoid():
    z = np.concatenate([np.linspace(-60, 60, 241), RNG.standard_normal(50) * 5])
    for tau in (1.0, 4.0, 16.0):
        ref = torch.nn.functional.logsigmoid(torch.from_numpy(z)).numpy() / tau
        assert np.allclose(R.gret_log_decay(z, tau), ref, atol=1e-15, rtol=1e-13)
    with pytest.raises(ValueError):
        R.gret_log_decay(z, 0.0)


def test_gate_one_is_causal_linear_attention():
    q, k, v, _ = _inputs(B=1, H=2, N=11)
    z = np.full((1, 2, 11), 800.0)           # sigmoid = 1 exactly in float64
    o, _ = R.gret_recurrent(q, k, v, z, 1.0)
    for h in range(2):
        ref = np.tril(q[0, h] @ k[0, h].T) @ v[0, h]
        assert np.allclose(o[0, h], ref, atol=1e-12)
    # a huge temperature drives the decay to 1 as well
    zt = RNG.standard_normal((1, 2, 11))
    o_t, _ = R.gret_recurrent(q, k, v, zt, 1e15)
    for h in range(2):
        assert np.allclose(o_t[0, h], np.tril(q[0, h] @ k[0, h].T) @ v[0, h], atol=1e-9)


def test_gate_zero_keeps_the_current_token():
    q, k, v, _ = _inputs(B=1, H=2, N=9)
    z = np.full((1, 2, 9), -800.0)          # gamma = exp(-800) = 0 in float64
    o, _ = R.gret_recurrent(q, k, v, z, 1.0)
    for h in range(2):
        for n in range(9):
            assert np.allclose(o[0, h, n], np.dot(q[0, h, n], k[0, h, n]) * v[0, h, n], atol=1e-12)


def test_constant_gate_is_a_power_decay():
    q, k, v, _ = _inputs(B=1, H=1, N=10)
    g = 0.8
    zc = math.log(g / (1 - g))              # sigmoid(zc) = g, tau = 1
    o, _ = R.gret_recurrent(q, k, v, np.full((1, 1, 10), zc), 1.0)
    n = np.arange(10)
    D = np.where(n[:, None] >= n[None, :], g ** (n[:, None] - n[None, :]).clip(0), 0.0)
    assert np.allclose(o[0, 0], (q[0, 0] @ k[0, 0].T * D) @ v[0, 0], atol=1e-12)


def test_brute_force_scalar_loops():
    B, H, N, dk, dv, tau = 1, 1, 5, 2, 3, 2.0
    q, k, v, z = _inputs(B, H, N, dk, dv)
    o, st = R.gret_recurrent(q, k, v, z, tau)
    S = [[0.0] * dv for _ in range(dk)]
    for n in range(N):
        gam = (1.0 / (1.0 + math.exp(-z[0, 0, n]))) ** (1.0 / tau)
        for i in range(dk):
            for j in range(dv):
                S[i][j] = gam * S[i][j] + k[0, 0, n, i] * v[0, 0, n, j]
        for j in range(dv):
            ref = sum(q[0, 0, n, i] * S[i][j] for i in range(dk))
            assert abs(o[0, 0, n, j] - ref) < 1e-13
    assert np.allclose(st[0, 0], np.array(S), atol=1e-13)


@pytest.mark.parametrize("n1", [1, 8, 13])
def test_state_hand_over(n1):
    q, k, v, z = _inputs(N=21)
    tau = 4.0
    o_all, st_all = R.gret_chunkwise(q, k, v, z, tau, 8)
    o1, st1 = R.gret_chunkwise(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], z[:, :, :n1], tau, 8)
    o2, st2 = R.gret_chunkwise(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], z[:, :, n1:], tau, 8, st1)
    assert np.allclose(np.concatenate([o1, o2], axis=2), o_all, atol=1e-12)
    assert np.allclose(st2, st_all, atol=1e-12)


def test_group_norm_swish_matches_torch():
    B, H, N, dv = 2, 3, 7, 8
    y = RNG.standard_normal((B, H, N, dv)) * 3 + 0.5
    g = RNG.standard_normal((B, N, H * dv))
    out = R.gret_group_norm_swish(y, g)
    merged = torch.from_numpy(y.transpose(0, 2, 1, 3).reshape(B * N, H * dv))
    ref = torch.nn.functional.group_norm(merged, H, eps=1e-6).reshape(B, N, H * dv)
    ref = torch.nn.functional.silu(torch.from_numpy(g)) * ref
    assert np.allclose(out, ref.numpy(), atol=1e-12)
