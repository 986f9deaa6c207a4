"""The tiny YOCO block: self-decoder, one global KV projection, cross-decoder.

TEST INFRASTRUCTURE ONLY (see the package docstring): float64 numpy, no code
shared with the GPU path.

What the method computes:
* The L layers are split in half: a self-decoder below, a cross-decoder on
  top ([P seg. 8]; [S §2]).
* Self-decoder layer: efficient attention (here sliding-window) on the
  normalised input plus a residual ([P seg. 12]; [S §3]).
* At the halfway point the output is normalised once and projected by one
  pair of matrices into the global keys and values ([P seg. 12]).
* Cross-decoder layer: its own query projection, causal grouped-query
  attention over that one shared pair, plus a residual ([P seg. 12]).
* Early exit: prefill runs the self-decoder over the whole prompt, writes the
  shared KV, skips the cross-decoder for the prompt tokens and sends only
  the last position through it; the output is unchanged ([P seg. 14] and its
  Figure 3; [S §2]; [A]).
* Generation: one token per step; each self-decoder layer keeps a constant
  window-sized cache, the global cache grows by one row per token, and every
  cross-decoder layer reads the whole global cache ([P seg. 4], [P seg. 26];
  [S §2], [S §3]).  Causality makes token-by-token generation reproduce the
  rows of a full forward over the same sequence.
* A self-decoder layer follows its attention with a SwiGLU feed-forward
  ([P seg. 12]).
Readings taken: each attention keeps an output projection W_o; layers are
pre-norm residual, x + attention(norm x) then x + SwiGLU(norm x); the
cross-decoder layers carry the same feed-forward (the pages describe only
their attention); the feed-forward is optional here (BlockParams.swa_ffn /
cross_ffn; absent in the smallest pins) and, when present, is SwiGLU(n) =
W_down (silu(W_gate n) * (W_up n)) with silu(z) = z * sigmoid(z), its sizes
chosen by the caller (the pages give none); RoPE is optional
(BlockParams.rope_theta, see oracle/rope.py for its readings); the final norm before the output head is left out (the
head is not part of the path); the cross-decoder's residual stream continues
from the self-decoder output, the same tensor the global K/V are projected
from.

The self-decoder's layers may instead be gated retention ([S §3 Gated
Retention]; [P seg. 16]; the better-scoring layout of [S §4 Scaling model
size]), BlockParams.self_kind = "gret".  Readings taken for such a layer (the
pages give its parts in words only): from n = rmsnorm(x), q = W_q n,
k = W_k n, v = W_v n with n_heads heads each (no grouping, no rotation), the
per-head gate logits z = W_z n, the retention of oracle/retention.py with
temperature gret_tau, the per-head GroupNorm times swish(W_g n), then W_o and
the residual, then the feed-forward as for a window layer.  Generation keeps
one d x d state per head and layer in place of the window ring.

Position-wise products are computed row by row with one routine (a
matrix-vector product), so that a row's value is bitwise the same whether or
not other rows are computed -- this is what makes the early-exit identity
exact inside the oracle.
"""

from dataclasses import dataclass, field
from typing import List

import math

import numpy as np

from .attention import attend_row, cross_prefill_attention, ring_window, swa_attention
from .projection import global_kv_proj, rmsnorm_row
from .retention import gret_group_norm_swish, gret_log_decay, gret_recurrent
from .rope import apply_rope

__all__ = ["BlockParams", "linear_rows", "silu", "swiglu_hidden_row", "swiglu_ffn_row", "yoco_block", "yoco_block_early_exit",
           "yoco_block_generate"]


@dataclass
class BlockParams:
    """Weights of the tiny block; every matrix is [out, in]."""
    n_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    swa_wq: List[np.ndarray] = field(default_factory=list)   # [Hq*d, D]
    swa_wk: List[np.ndarray] = field(default_factory=list)   # [Hkv*d, D]
    swa_wv: List[np.ndarray] = field(default_factory=list)   # [Hkv*d, D]
    swa_wo: List[np.ndarray] = field(default_factory=list)   # [D, Hq*d]
    glob_wk: np.ndarray = None                               # [Hkv*d, D]
    glob_wv: np.ndarray = None                               # [Hkv*d, D]
    cross_wq: List[np.ndarray] = field(default_factory=list)  # [Hq*d, D]
    cross_wo: List[np.ndarray] = field(default_factory=list)  # [D, Hq*d]
    # optional SwiGLU feed-forward per layer: (w_gate [F, D], w_up [F, D], w_down [D, F])
    swa_ffn: List[tuple] = field(default_factory=list)
    cross_ffn: List[tuple] = field(default_factory=list)
    eps: float = 1e-6
    # rotary embedding base (0: none): queries and keys of every attention,
    # and the global keys, rotated at their absolute positions
    rope_theta: float = 0.0
    # self-decoder layer kind: "swa" (sliding-window attention) or "gret"
    # (gated retention: swa_wk / swa_wv are then [n_heads*d, D], and each
    # layer adds gate-logit weights [n_heads, D] and swish-gate weights
    # [n_heads*d, D]); gated retention takes no rotary embedding
    self_kind: str = "swa"
    gret_wz: List[np.ndarray] = field(default_factory=list)
    gret_wg: List[np.ndarray] = field(default_factory=list)
    gret_tau: float = 16.0

    def ffn(self, kind, layer):
        lst = self.swa_ffn if kind == "swa" else self.cross_ffn
        return lst[layer] if lst else None


def silu(z):
    """z * sigmoid(z), written so that no exponential overflows."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, z / (1.0 + e), z * e / (1.0 + e))


def _rope(t, pos0, p):
    """t [..., n, d] rotated for positions pos0.. when the block uses RoPE."""
    return apply_rope(t, pos0, p.rope_theta) if p.rope_theta > 0 else t


def swiglu_hidden_row(x_row, w_gate, w_up, gamma=None, eps=1e-6):
    """The feed-forward's hidden activations for one row: silu(W_gate n) * (W_up n),
    n = rmsnorm(x) * gamma."""
    n = rmsnorm_row(x_row, gamma, eps)
    return silu(w_gate @ n) * (w_up @ n)


def swiglu_ffn_row(x_row, ffn, eps):
    """x + W_down (silu(W_gate n) * (W_up n)), n = rmsnorm(x), for one row."""
    wg, wu, wd = ffn
    return x_row + wd @ swiglu_hidden_row(x_row, wg, wu, None, eps)


def _ffn_rows(x, ffn, eps):
    if ffn is None:
        return x
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty_like(flat)
    for r in range(flat.shape[0]):
        out[r] = swiglu_ffn_row(flat[r], ffn, eps)
    return out.reshape(x.shape)


def linear_rows(x, w):
    """y[..., :] = w @ x[..., :] computed one row at a time."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty((flat.shape[0], w.shape[0]))
    for r in range(flat.shape[0]):
        out[r] = w @ flat[r]
    return out.reshape(x.shape[:-1] + (w.shape[0],))


def _norm_rows(x, eps):
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty_like(flat)
    for r in range(flat.shape[0]):
        out[r] = rmsnorm_row(flat[r], None, eps)
    return out.reshape(x.shape)


def _heads(t, n_heads, head_dim):
    """[B, N, H*d] -> [B, H, N, d]."""
    B, N, _ = t.shape
    return t.reshape(B, N, n_heads, head_dim).transpose(0, 2, 1, 3)


def _merge(t):
    """[B, H, N, d] -> [B, N, H*d]."""
    B, H, N, d = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, N, H * d)


def _gret_layer_rows(x, p, layer):
    """The residual stream after gated-retention layer `layer` (before its
    feed-forward), every position at once."""
    H, d = p.n_heads, p.head_dim
    n = _norm_rows(x, p.eps)
    q = _heads(linear_rows(n, p.swa_wq[layer]), H, d)
    k = _heads(linear_rows(n, p.swa_wk[layer]), H, d)
    v = _heads(linear_rows(n, p.swa_wv[layer]), H, d)
    z = linear_rows(n, p.gret_wz[layer]).transpose(0, 2, 1)        # [B, H, N]
    y, _ = gret_recurrent(q, k, v, z, p.gret_tau)
    g = linear_rows(n, p.gret_wg[layer])                           # [B, N, H*d]
    return x + linear_rows(gret_group_norm_swish(y, g, p.eps), p.swa_wo[layer])


def _self_decoder_and_projection(x, p):
    Hq, Hkv, d = p.n_heads, p.n_kv_heads, p.head_dim
    x = np.array(x, dtype=np.float64)
    for layer, (wq, wk, wv, wo) in enumerate(zip(p.swa_wq, p.swa_wk, p.swa_wv, p.swa_wo)):
        if p.self_kind == "gret":
            x = _gret_layer_rows(x, p, layer)
            x = _ffn_rows(x, p.ffn("swa", layer), p.eps)
            continue
        n = _norm_rows(x, p.eps)
        q = _rope(_heads(linear_rows(n, wq), Hq, d), 0, p)
        k = _rope(_heads(linear_rows(n, wk), Hkv, d), 0, p)
        v = _heads(linear_rows(n, wv), Hkv, d)
        o, _ = swa_attention(q, k, v, p.window)
        x = x + linear_rows(_merge(o), wo)
        x = _ffn_rows(x, p.ffn("swa", layer), p.eps)
    k_glob, v_glob = global_kv_proj(x, p.glob_wk, p.glob_wv, Hkv, d, eps=p.eps)
    return x, _rope(k_glob, 0, p), v_glob


def yoco_block(x, p):
    """Full forward: every position goes through the cross-decoder.

    x [B, N, D].  Returns (x_out [B, N, D], (K, V) shared cache [B, Hkv, N, d]).
    """
    Hq, d = p.n_heads, p.head_dim
    x, k_glob, v_glob = _self_decoder_and_projection(x, p)
    for layer, (wq, wo) in enumerate(zip(p.cross_wq, p.cross_wo)):
        n = _norm_rows(x, p.eps)
        q = _rope(_heads(linear_rows(n, wq), Hq, d), 0, p)
        # every cross layer reads the same k_glob / v_glob objects
        o, _ = cross_prefill_attention(q, k_glob, v_glob)
        x = x + linear_rows(_merge(o), wo)
        x = _ffn_rows(x, p.ffn("cross", layer), p.eps)
    return x, (k_glob, v_glob)


def yoco_block_early_exit(x, p):
    """Early-exit prefill: the cross-decoder runs for the last position only.

    Returns (x_last [B, D], (K, V)).  Equal bitwise to yoco_block(x, p)[0][:, -1].
    """
    Hq, Hkv, d = p.n_heads, p.n_kv_heads, p.head_dim
    x, k_glob, v_glob = _self_decoder_and_projection(x, p)
    B, N, _ = x.shape
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    last = x[:, N - 1, :].copy()
    for layer, (wq, wo) in enumerate(zip(p.cross_wq, p.cross_wo)):
        ffn = p.ffn("cross", layer)
        new = np.empty_like(last)
        for b in range(B):
            n = rmsnorm_row(last[b], None, p.eps)
            q = _rope((wq @ n).reshape(Hq, 1, d), N - 1, p)[:, 0]
            o = np.empty((Hq, d))
            for h in range(Hq):
                o[h], _, _ = attend_row(q[h], k_glob[b, h // g, :N],
                                        v_glob[b, h // g, :N], scale)
            new[b] = last[b] + wo @ o.reshape(Hq * d)
            if ffn is not None:
                new[b] = swiglu_ffn_row(new[b], ffn, p.eps)
        last = new
    return last, (k_glob, v_glob)


def yoco_block_generate(x, p):
    """Token-by-token forward with generation-time caches.

    Position t is processed after positions 0..t-1 only.  Each self-decoder
    layer appends the token's K/V to its ring of W slots (slot t mod W) and
    attends over the window read back in position order; the hidden state
    after the self-decoder is normalised and projected into row t of the
    global cache; each cross-decoder layer attends over global rows 0..t.
    Returns (x_out [B, N, D], (K, V) [B, Hkv, N, d], rings) where rings[l] =
    (K ring, V ring) [B, Hkv, W, d] of self-decoder layer l after the last
    token.  Equal bitwise to yoco_block(x, p) (the same per-row arithmetic).
    """
    Hq, Hkv, d, W = p.n_heads, p.n_kv_heads, p.head_dim, p.window
    x = np.array(x, dtype=np.float64)
    B, N, D = x.shape
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    rings = [(np.zeros((B, Hkv, W, d)), np.zeros((B, Hkv, W, d))) for _ in p.swa_wq]
    states = [np.zeros((B, Hq, d, d)) for _ in p.swa_wq]      # gated-retention layers
    k_glob = np.zeros((B, Hkv, N, d))
    v_glob = np.zeros((B, Hkv, N, d))
    out = np.empty_like(x)
    for t in range(N):
        slots = [s for _, s in ring_window(t, W)]
        h_t = x[:, t, :].copy()
        for layer, ((wq, wk, wv, wo), (kr, vr)) in enumerate(zip(zip(p.swa_wq, p.swa_wk, p.swa_wv, p.swa_wo),
                                                                 rings)):
            ffn = p.ffn("swa", layer)
            new = np.empty_like(h_t)
            if p.self_kind == "gret":
                # one recurrent step per head: S <- gamma S + k^T v, y = q S
                for b in range(B):
                    n = rmsnorm_row(h_t[b], None, p.eps)
                    q, k, v = (wq @ n).reshape(Hq, d), (wk @ n).reshape(Hq, d), (wv @ n).reshape(Hq, d)
                    lg = gret_log_decay(p.gret_wz[layer] @ n, p.gret_tau)
                    y = np.empty((Hq, d))
                    for h in range(Hq):
                        S = math.exp(lg[h]) * states[layer][b, h] + np.outer(k[h], v[h])
                        states[layer][b, h] = S
                        y[h] = q[h] @ S
                    gn = gret_group_norm_swish(y[None, :, None, :], (p.gret_wg[layer] @ n)[None, None, :], p.eps)
                    new[b] = h_t[b] + wo @ gn[0, 0]
                    if ffn is not None:
                        new[b] = swiglu_ffn_row(new[b], ffn, p.eps)
                h_t = new
                continue
            for b in range(B):
                n = rmsnorm_row(h_t[b], None, p.eps)
                q = _rope((wq @ n).reshape(Hq, 1, d), t, p)[:, 0]
                kr[b, :, t % W] = _rope((wk @ n).reshape(Hkv, 1, d), t, p)[:, 0]
                vr[b, :, t % W] = (wv @ n).reshape(Hkv, d)
                o = np.empty((Hq, d))
                for h in range(Hq):
                    o[h], _, _ = attend_row(q[h], kr[b, h // g, slots], vr[b, h // g, slots], scale)
                new[b] = h_t[b] + wo @ o.reshape(Hq * d)
                if ffn is not None:
                    new[b] = swiglu_ffn_row(new[b], ffn, p.eps)
            h_t = new
        for b in range(B):
            k_row, v_row = global_kv_proj(h_t[b][None, None, :], p.glob_wk, p.glob_wv, Hkv, d, eps=p.eps)
            k_glob[b, :, t] = _rope(k_row[0, :, :1], t, p)[:, 0]
            v_glob[b, :, t] = v_row[0, :, 0]
        for layer, (wq, wo) in enumerate(zip(p.cross_wq, p.cross_wo)):
            ffn = p.ffn("cross", layer)
            new = np.empty_like(h_t)
            for b in range(B):
                n = rmsnorm_row(h_t[b], None, p.eps)
                q = _rope((wq @ n).reshape(Hq, 1, d), t, p)[:, 0]
                o = np.empty((Hq, d))
                for h in range(Hq):
                    o[h], _, _ = attend_row(q[h], k_glob[b, h // g, :t + 1], v_glob[b, h // g, :t + 1], scale)
                new[b] = h_t[b] + wo @ o.reshape(Hq * d)
                if ffn is not None:
                    new[b] = swiglu_ffn_row(new[b], ffn, p.eps)
            h_t = new
        out[:, t, :] = h_t
    return out, (k_glob, v_glob), rings
