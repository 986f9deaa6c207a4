"""Softmax attention over an explicit allowed-key set, one query row at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring): float64 numpy, no code
shared with the GPU path.

What the method computes (pages cited as in the package docstring):

* Every attention in YOCO is causal: a position never looks at later
  positions ([S §1 Architecture bullet]; [P seg. 8]: the whole stack stays
  causal).
* Self-decoder sliding-window attention restricts each query to a fixed
  window of the most recent positions ([S §3 Sliding-Window Attention]).
  Reading taken: a window of W keys *including* the query's own position,
  i.e. keys s with t - W < s <= t.  W >= N is then ordinary causal attention.
* Cross-decoder layers each have their own queries and attend causally to the
  one shared key/value pair produced by the global projection, with
  grouped-query heads ([P seg. 12]; [S §2]).
* Decoding produces one token per step and reads the entire cache each step
  ([P seg. 4], [P seg. 26]).
* During generation the self-decoder keeps only a window-sized cache: its
  memory is constant in the sequence length ([S §3 Sliding-Window
  Attention]; [S §2]).  Reading taken for its layout: a ring of W slots per
  layer and KV head, position t stored in slot t mod W, so that the slots
  always hold the last W positions.  Reading taken: the cache already holds the
  current token, so a decode query at step ctx-1 attends to keys 0..ctx-1.
* Grouped-query attention: several query heads share one KV head
  ([P seg. 4]; [S App. C]).  Reading taken: contiguous groups, query head h
  uses KV head h // (Hq // Hkv).
* Softmax scale 1/sqrt(d) (the textbook choice; the pages name no other).

The definition written out, for query row t with allowed key set A(t):
    z_s = scale * <q_t, k_s>          for s in A(t)
    m   = max_s z_s
    p_s = exp(z_s - m) / sum_r exp(z_r - m)
    o_t = sum_s p_s v_s
    lse = m + ln(sum_r exp(z_r - m))
Masked keys are left out of A(t) altogether; they are never added as -inf.
All three allowed sets are contiguous index ranges [lo, hi).
"""

import math

import numpy as np

__all__ = [
    "attend_row",
    "attention_rows",
    "swa_allowed",
    "causal_allowed",
    "swa_attention",
    "cross_prefill_attention",
    "decode_attention",
    "ring_window",
    "swa_ring_decode_attention",
]


def attend_row(q_vec, k_rows, v_rows, scale):
    """Attention of one query over the given key/value rows (all allowed).

    q_vec [d], k_rows/v_rows [n, d] float64, n >= 1.
    Returns (o [d], lse scalar, p [n]) with p the explicit softmax row.
    """
    z = scale * (k_rows @ q_vec)
    m = z.max()
    e = np.exp(z - m)
    s = e.sum()
    p = e / s
    o = p @ v_rows
    return o, m + math.log(s), p


def swa_allowed(t, window, n_keys):
    """Keys visible to position t under a window of W keys including t itself."""
    lo = max(0, t - window + 1)
    hi = min(t, n_keys - 1) + 1
    return lo, hi


def causal_allowed(pos, n_keys):
    """Keys visible to a query at absolute position pos under causal masking."""
    return 0, min(pos, n_keys - 1) + 1


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def attention_rows(q, k, v, allowed, scale=None, rows=None, bh=None):
    """Grouped-query attention with a per-row allowed range.

    q [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d]; allowed(i) -> (lo, hi) for query
    row i.  rows: query indices to compute (default all); bh: (b, h) pairs to
    compute (default all).  Rows that are not computed are NaN in the output.
    Returns (o [B, Hq, Nq, d], lse [B, Hq, Nq]).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if rows is None:
        rows = range(Nq)
    if bh is None:
        bh = [(b, h) for b in range(B) for h in range(Hq)]
    o = np.full(q.shape, np.nan)
    lse = np.full(q.shape[:3], np.nan)
    for b, h in bh:
        kvh = h // g
        for i in rows:
            lo, hi = allowed(i)
            if hi <= lo:
                raise ValueError(f"empty allowed set for row {i}")
            o[b, h, i], lse[b, h, i], _ = attend_row(
                q[b, h, i], k[b, kvh, lo:hi], v[b, kvh, lo:hi], scale)
    return o, lse


def swa_attention(q, k, v, window, scale=None, rows=None, bh=None):
    """Self-decoder sliding-window attention ([S §3 Sliding-Window Attention]).

    q [B, Hq, N, d], k/v [B, Hkv, N, d]; query t sees keys t-W < s <= t.
    """
    n_keys = np.shape(k)[2]
    if window < 1:
        raise ValueError("window must be >= 1")
    return attention_rows(q, k, v, lambda t: swa_allowed(t, window, n_keys),
                          scale, rows, bh)


def cross_prefill_attention(q, k, v, n_kv=None, q_offset=0, scale=None,
                            rows=None, bh=None):
    """Causal cross-attention of one cross-decoder layer over the shared cache.

    q [B, Hq, Nq, d] holds queries at absolute positions q_offset .. q_offset+Nq-1;
    k/v [B, Hkv, n_cap, d] is the shared global cache of which the first n_kv
    rows are valid ([P seg. 12]: per-layer queries, one shared K/V pair,
    causal).  Query i sees keys 0 .. q_offset + i.
    """
    Nq = np.shape(q)[2]
    if n_kv is None:
        n_kv = np.shape(k)[2]
    if q_offset < 0 or q_offset + Nq > n_kv:
        raise ValueError("queries must sit inside the valid cache rows")
    return attention_rows(q, k, v, lambda i: causal_allowed(q_offset + i, n_kv),
                          scale, rows, bh)


def decode_attention(q, k_cache, v_cache, ctx_lens, scale=None, bh=None):
    """One decode step of a cross-decoder layer ([P seg. 4], [P seg. 26]).

    q [B, Hq, d]; k_cache/v_cache [B, Hkv, n_cap, d]; ctx_lens [B] (>= 1).
    Query of sequence b sees cache rows 0 .. ctx_lens[b]-1.
    Returns (o [B, Hq, d], lse [B, Hq]).
    """
    q, k_cache, v_cache = _as64(q), _as64(k_cache), _as64(v_cache)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ctx_lens = [int(c) for c in np.broadcast_to(np.asarray(ctx_lens), (B,))]
    if bh is None:
        bh = [(b, h) for b in range(B) for h in range(Hq)]
    o = np.full(q.shape, np.nan)
    lse = np.full((B, Hq), np.nan)
    for b, h in bh:
        c = ctx_lens[b]
        if c < 1 or c > k_cache.shape[2]:
            raise ValueError("ctx must be in [1, n_cap]")
        kvh = h // g
        o[b, h], lse[b, h], _ = attend_row(
            q[b, h], k_cache[b, kvh, :c], v_cache[b, kvh, :c], scale)
    return o, lse


def merge_partial_attention(o_parts, lse_parts):
    """Attention over a union of disjoint key sets, from the results over each
    set: with L = log sum_s exp(lse_s),  o = sum_s exp(lse_s - L) o_s.

    This is the combine step of a decode whose cache is split across shards
    (each shard attends over its rows and reports o_s with its log-sum-exp);
    the pages split long sequences across devices ([S App. A]; [P seg. 14]),
    the merge itself is the softmax definition regrouped.
    o_parts [S, ..., d]; lse_parts [S, ...] (natural log).  Returns (o, L).
    """
    o_parts, lse_parts = _as64(o_parts), _as64(lse_parts)
    if o_parts.shape[:-1] != lse_parts.shape:
        raise ValueError("o_parts [S, ..., d] and lse_parts [S, ...]")
    m = lse_parts.max(axis=0)
    w = np.exp(lse_parts - m)
    tot = w.sum(axis=0)
    o = (w[..., None] * o_parts).sum(axis=0) / tot[..., None]
    return o, m + np.log(tot)


def ring_window(pos, window):
    """(position, slot) pairs a decode query at position pos reads from a ring
    of W slots, in position order: positions max(0, pos-W+1) .. pos, position
    t in slot t mod W."""
    if pos < 0 or window < 1:
        raise ValueError("pos must be >= 0 and window >= 1")
    return [(t, t % window) for t in range(max(0, pos - window + 1), pos + 1)]


def swa_ring_decode_attention(q, k_ring, v_ring, pos, scale=None, bh=None):
    """One decode step of a self-decoder sliding-window layer over its ring
    cache ([S §3 Sliding-Window Attention]).

    q [B, Hq, d] is the query of the token at position pos (the same for the
    whole batch); k_ring/v_ring [B, Hkv, W, d] hold position t in slot t mod W
    for the last W positions, the current one included.  The keys are
    gathered in position order, so the result equals row pos of
    swa_attention over the full sequence.
    Returns (o [B, Hq, d], lse [B, Hq]).
    """
    q, k_ring, v_ring = _as64(q), _as64(k_ring), _as64(v_ring)
    B, Hq, d = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    slots = [s for _, s in ring_window(pos, W)]
    if bh is None:
        bh = [(b, h) for b in range(B) for h in range(Hq)]
    o = np.full(q.shape, np.nan)
    lse = np.full((B, Hq), np.nan)
    for b, h in bh:
        kvh = h // g
        o[b, h], lse[b, h], _ = attend_row(
            q[b, h], k_ring[b, kvh, slots], v_ring[b, kvh, slots], scale)
    return o, lse
