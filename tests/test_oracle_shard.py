"""Pins for the sharded forms (one device's share of a sequence split across
devices):

* merge_partial_attention: decoding each disjoint shard of a cache and
  merging equals decoding the whole cache (the softmax over a union), for any
  split, in any shard order; one shard is the identity; a planted wrong weight
  (dropping a shard's log-sum-exp) is caught;
* a sliding-window shard computed over its rows plus a halo of the previous
  W - 1 rows equals those rows of the full sequence, bitwise (each row's
  arithmetic is the same).
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(909)


def _cache(B=2, Hq=4, Hkv=2, n=37, d=8):
    return (RNG.standard_normal((B, Hq, d)), RNG.standard_normal((B, Hkv, n, d)),
            RNG.standard_normal((B, Hkv, n, d)))


@pytest.mark.parametrize("cuts", [[37], [10, 37], [1, 2, 30, 37], [5, 6, 20, 21, 37]])
def test_merged_shards_equal_the_whole_cache(cuts):
    q, k, v = _cache()
    full_o, full_lse = oracle.decode_attention(q, k, v, [37])
    parts, lses = [], []
    lo = 0
    for hi in cuts:
        o, lse = oracle.decode_attention(q, k[:, :, lo:hi], v[:, :, lo:hi], [hi - lo])
        parts.append(o)
        lses.append(lse)
        lo = hi
    o, lse = oracle.merge_partial_attention(np.stack(parts), np.stack(lses))
    assert np.allclose(o, full_o, atol=1e-12) and np.allclose(lse, full_lse, atol=1e-12)
    # shard order does not matter
    o2, lse2 = oracle.merge_partial_attention(np.stack(parts[::-1]), np.stack(lses[::-1]))
    assert np.allclose(o2, o, atol=1e-14) and np.allclose(lse2, lse, atol=1e-14)
    if len(cuts) == 1:
        assert np.array_equal(o, parts[0]) and np.allclose(lse, lses[0], atol=1e-15)


def test_planted_wrong_weight_is_caught():
    q, k, v = _cache()
    a = oracle.decode_attention(q, k[:, :, :20], v[:, :, :20], [20])
    b = oracle.decode_attention(q, k[:, :, 20:], v[:, :, 20:], [17])
    full_o, _ = oracle.decode_attention(q, k, v, [37])
    # equal weights instead of the log-sum-exp weights
    wrong, _ = oracle.merge_partial_attention(np.stack([a[0], b[0]]), np.zeros((2,) + a[1].shape))
    assert np.max(np.abs(wrong - full_o)) > 1e-3


@pytest.mark.parametrize("W,start,N", [(5, 8, 6), (16, 40, 25), (3, 3, 1)])
def test_halo_window_shard_is_bitwise(W, start, N):
    B, Hq, Hkv, d, T = 1, 4, 2, 8, 80
    q = RNG.standard_normal((B, Hq, T, d))
    k = RNG.standard_normal((B, Hkv, T, d))
    v = RNG.standard_normal((B, Hkv, T, d))
    full, _ = oracle.swa_attention(q, k, v, W)
    h0 = max(0, start - (W - 1))
    # the shard's queries sit at offset start - h0 of its key rows [h0, start + N)
    shard = oracle.attention_rows(q[:, :, start:start + N], k[:, :, h0:start + N], v[:, :, h0:start + N],
                                  lambda i: oracle.swa_allowed(start - h0 + i, W, start + N - h0))[0]
    assert np.array_equal(shard, full[:, :, start:start + N])
