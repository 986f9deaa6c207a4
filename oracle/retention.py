"""Gated retention, the self-decoder's other choice, in its three forms.

TEST INFRASTRUCTURE ONLY (see the package docstring): float64 numpy, no code
shared with the GPU path.

What the method computes (pages cited as in the package docstring):

* Gated retention is retention plus a data-dependent, head-wise scalar decay
  gate; the gate is a sigmoid of the input raised to the power one over a
  temperature, and the temperature pushes the decay towards 1 ([P seg. 16];
  [S §3 Gated Retention]).
* Three forms give the same result ([S §3]; [S App. B]; [P seg. 16]):
  recurrent (one d x d state per head, for decoding), parallel (for
  training), and chunkwise (parallel inside a chunk, recurrent across
  chunks; chunk size 256 in the paper, positions n = kB + r).
* Several heads run independently; their outputs are normalised per head
  (GroupNorm) and multiplied by a swish gate ([S §3 Gated Retention]).

Readings taken (the pages give the forms in words only; the symbols below
are the ones used here):
* gate: gamma_n = sigmoid(z_n) ** (1 / tau) for the per-head, per-position
  gate logit z_n (z_n = x_n . w_gamma is a position-wise product outside this
  path) and temperature tau > 0; log gamma_n = log sigmoid(z_n) / tau.
* recurrent form, state S (d_k x d_v, zero unless given), for n = 1..N:
      S_n = gamma_n S_{n-1} + k_n^T v_n,     o_n = q_n S_n
  (the current token enters the state before it is read, as causal
  attention includes the current position).
* no scale on q . k and no rotation of q, k (the pages name neither; after
  the per-head normalisation a scale would cancel).
* GroupNorm per head over its d_v channels, eps 1e-6, unit gain, zero bias;
  swish(x) = x * sigmoid(x).
"""

import math

import numpy as np

__all__ = [
    "gret_log_decay",
    "gret_recurrent",
    "gret_parallel",
    "gret_chunkwise",
    "gret_group_norm_swish",
]


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def gret_log_decay(z, tau):
    """log gamma = log(sigmoid(z)) / tau, evaluated without overflow."""
    z = _as64(z)
    if not tau > 0:
        raise ValueError("tau must be > 0")
    # log sigmoid(z) = -log(1 + exp(-z)) = min(z, 0) - log(1 + exp(-|z|))
    return (np.minimum(z, 0.0) - np.log1p(np.exp(-np.abs(z)))) / tau


def _shapes(q, k, v, z):
    B, H, N, dk = q.shape
    if k.shape != (B, H, N, dk) or v.shape[:3] != (B, H, N) or z.shape != (B, H, N):
        raise ValueError("q, k [B,H,N,dk], v [B,H,N,dv], z [B,H,N]")
    return B, H, N, dk, v.shape[3]


def gret_recurrent(q, k, v, z, tau, state0=None):
    """Recurrent form.  Returns (o [B,H,N,dv], final state [B,H,dk,dv])."""
    q, k, v, z = _as64(q), _as64(k), _as64(v), _as64(z)
    B, H, N, dk, dv = _shapes(q, k, v, z)
    lg = gret_log_decay(z, tau)
    o = np.empty((B, H, N, dv))
    st = np.zeros((B, H, dk, dv)) if state0 is None else _as64(state0).copy()
    for b in range(B):
        for h in range(H):
            S = st[b, h]
            for n in range(N):
                S = math.exp(lg[b, h, n]) * S + np.outer(k[b, h, n], v[b, h, n])
                o[b, h, n] = q[b, h, n] @ S
            st[b, h] = S
    return o, st


def gret_parallel(q, k, v, z, tau, state0=None):
    """Parallel form: o = (Q K^T * D) V + (decay from the start) * Q S_0, with
    D[n, m] = prod_{i=m+1..n} gamma_i for m <= n, else 0.  Returns o."""
    q, k, v, z = _as64(q), _as64(k), _as64(v), _as64(z)
    B, H, N, dk, dv = _shapes(q, k, v, z)
    lg = gret_log_decay(z, tau)
    o = np.empty((B, H, N, dv))
    for b in range(B):
        for h in range(H):
            c = np.cumsum(lg[b, h])                       # c[n] = sum_{i<=n} log gamma_i
            diff = c[:, None] - c[None, :]                # log prod_{i=m+1..n} gamma_i
            D = np.where(np.tril(np.ones((N, N), dtype=bool)), np.exp(np.minimum(diff, 0.0)), 0.0)
            o[b, h] = (q[b, h] @ k[b, h].T * D) @ v[b, h]
            if state0 is not None:
                o[b, h] += np.exp(c)[:, None] * (q[b, h] @ _as64(state0)[b, h])
    return o


def gret_chunkwise(q, k, v, z, tau, chunk, state0=None):
    """Chunkwise form with chunks of `chunk` positions (the last may be
    shorter): inside a chunk the parallel form, across chunks the state.
    With L_j the log decay accumulated from the chunk start through j:
        o_n = sum_{m in chunk, m <= n} (q_n . k_m) e^{L_n - L_m} v_m
              + e^{L_n} q_n R
        R  <- e^{L_last} R + sum_{m in chunk} e^{L_last - L_m} k_m^T v_m
    Returns (o [B,H,N,dv], final state [B,H,dk,dv])."""
    q, k, v, z = _as64(q), _as64(k), _as64(v), _as64(z)
    B, H, N, dk, dv = _shapes(q, k, v, z)
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    lg = gret_log_decay(z, tau)
    o = np.empty((B, H, N, dv))
    st = np.zeros((B, H, dk, dv)) if state0 is None else _as64(state0).copy()
    for b in range(B):
        for h in range(H):
            R = st[b, h]
            for c0 in range(0, N, chunk):
                c1 = min(c0 + chunk, N)
                L = np.cumsum(lg[b, h, c0:c1])
                Qc, Kc, Vc = q[b, h, c0:c1], k[b, h, c0:c1], v[b, h, c0:c1]
                n_c = c1 - c0
                mask = np.tril(np.ones((n_c, n_c), dtype=bool))
                Dc = np.where(mask, np.exp(np.minimum(L[:, None] - L[None, :], 0.0)), 0.0)
                o[b, h, c0:c1] = (Qc @ Kc.T * Dc) @ Vc + np.exp(L)[:, None] * (Qc @ R)
                R = math.exp(L[-1]) * R + Kc.T @ (np.exp(L[-1] - L)[:, None] * Vc)
            st[b, h] = R
    return o, st


def gret_group_norm_swish(y, g, eps=1e-6):
    """Per-head GroupNorm of y [B,H,N,dv] over its dv channels, times
    swish(g), with heads merged: g and the result are [B, N, H*dv]."""
    y, g = _as64(y), _as64(g)
    B, H, N, dv = y.shape
    if g.shape != (B, N, H * dv):
        raise ValueError("g must be [B, N, H*dv]")
    mu = y.mean(axis=3, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=3, keepdims=True)
    yn = (y - mu) / np.sqrt(var + eps)
    merged = yn.transpose(0, 2, 1, 3).reshape(B, N, H * dv)
    return g / (1.0 + np.exp(-g)) * merged
