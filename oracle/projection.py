"""RMSNorm and the one-time global key/value projection.

TEST INFRASTRUCTURE ONLY (see the package docstring): float64 numpy, no code
shared with the GPU path.

What the method computes:
* At the boundary between the two halves, the self-decoder's output is
  normalised once and projected by a single pair of matrices into the global
  keys and values that every cross-decoder layer reuses ([P seg. 12];
  [S §2]; [P seg. 8]).
* The pages say only "normalized".  Reading taken: RMSNorm (the Llama-style
  normalisation of the baseline the paper compares against, [S §4 Scaling
  model size]), y = x / sqrt(mean(x^2) + eps) * gamma, eps = 1e-6, gamma = 1
  unless given.
* Weight layout (a choice made here, stated so tests can build inputs):
  W_K and W_V are [Hkv*d, D] ("out x in"), K = norm(X) @ W_K^T.  Output
  column j = h*d + c goes to KV head h, channel c; caches are head-major
  [B, Hkv, N, d].

Every row is computed on its own with the same routines (a dot product for
the mean square, a matrix-vector product for the projection), so a row's
result never depends on which other rows are computed.
"""

import math

import numpy as np

__all__ = ["rmsnorm_row", "rmsnorm", "global_kv_proj"]


def rmsnorm_row(x_row, gamma=None, eps=1e-6):
    """RMSNorm of one vector: x / sqrt(mean(x^2) + eps) * gamma."""
    x_row = np.asarray(x_row, dtype=np.float64)
    ms = float(np.dot(x_row, x_row)) / x_row.shape[0]
    y = x_row / math.sqrt(ms + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    return y


def rmsnorm(x, gamma=None, eps=1e-6):
    """RMSNorm over the last axis, row by row."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty_like(flat)
    for r in range(flat.shape[0]):
        out[r] = rmsnorm_row(flat[r], gamma, eps)
    return out.reshape(x.shape)


def global_kv_proj(x, w_k, w_v, n_kv_heads, head_dim, gamma=None, eps=1e-6,
                   rows=None):
    """K, V = RMSNorm(x) @ W_K^T, RMSNorm(x) @ W_V^T, split into KV heads.

    x [B, N, D]; w_k, w_v [Hkv*d, D].  rows: token indices to compute (default
    all); uncomputed rows are NaN.  Returns (K, V), each [B, Hkv, N, d].
    """
    x = np.asarray(x, dtype=np.float64)
    w_k = np.asarray(w_k, dtype=np.float64)
    w_v = np.asarray(w_v, dtype=np.float64)
    B, N, D = x.shape
    width = n_kv_heads * head_dim
    if w_k.shape != (width, D) or w_v.shape != (width, D):
        raise ValueError("weights must be [Hkv*d, D]")
    if rows is None:
        rows = range(N)
    k_out = np.full((B, n_kv_heads, N, head_dim), np.nan)
    v_out = np.full((B, n_kv_heads, N, head_dim), np.nan)
    for b in range(B):
        for t in rows:
            n = rmsnorm_row(x[b, t], gamma, eps)
            k_out[b, :, t, :] = (w_k @ n).reshape(n_kv_heads, head_dim)
            v_out[b, :, t, :] = (w_v @ n).reshape(n_kv_heads, head_dim)
    return k_out, v_out
