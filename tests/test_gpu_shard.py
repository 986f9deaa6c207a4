"""One device's share of a sequence split across devices, on the GPU:

* a sliding-window shard computed over its rows plus a halo of the previous
  rows (yoco_swa_attn_halo) equals those rows of the full sequence's
  yoco_swa_attn bitwise when the halo starts on a 64-row boundary, and the
  float64 oracle within the usual bounds otherwise;
* decoding each shard of a split cache (with its log-sum-exp) and merging
  (yoco_attn_merge) equals decoding the whole cache, within the bf16 / f32
  bounds, and the oracle;
* the 1M-token early-exit workload split 8 ways, at the real shard shapes.
"""
import numpy as np
import pytest
import torch

import oracle
import shared_kv_attention_amd as yk
from shared_kv_attention_amd.synth import randn
from _tol import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _tdt(dt):
    return torch.float32 if dt == "f32" else torch.bfloat16


@pytest.mark.parametrize("dt,W,C", [("bf16", 64, 256), ("bf16", 1024, 1024), ("f32", 128, 384)])
def test_halo_shards_are_bitwise_rows_of_the_full_sequence(dt, W, C):
    B, Hq, Hkv, d, N = 1, 8, 2, 128, 4 * C
    print(f"halo shards {dt} W={W} shard={C}", flush=True)
    q = randn((B, Hq, N, d), 7000 + W, dtype=dt, device=DEV)
    k = randn((B, Hkv, N, d), 7001 + W, dtype=dt, device=DEV)
    v = randn((B, Hkv, N, d), 7002 + W, dtype=dt, device=DEV)
    lse_full = torch.empty(B, Hq, N, dtype=torch.float32, device=DEV)
    full = yk.yoco_swa_attn(q, k, v, W, lse=lse_full)
    halo = (W - 1 + 63) // 64 * 64          # at least W - 1 rows, starting on a 64-row boundary
    for s in range(N // C):
        lo, hi = s * C, (s + 1) * C
        h0 = max(0, lo - halo)
        lse = torch.empty(B, Hq, C, dtype=torch.float32, device=DEV)
        o = yk.yoco_swa_attn_halo(q[:, :, lo:hi].contiguous(), k[:, :, h0:hi].contiguous(),
                                  v[:, :, h0:hi].contiguous(), W, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o, full[:, :, lo:hi]), f"shard {s}: output differs"
        assert torch.equal(lse, lse_full[:, :, lo:hi]), f"shard {s}: lse differs"


def test_unaligned_halo_matches_oracle():
    """A halo of exactly W - 1 rows starting off a tile boundary: the key
    tiles differ from the full sequence's, so only the oracle bound holds."""
    B, Hq, Hkv, d, N, W = 1, 4, 1, 64, 700, 100
    lo, hi = 333, 700
    q = randn((B, Hq, N, d), 7100, dtype="f32", device=DEV)
    k = randn((B, Hkv, N, d), 7101, dtype="f32", device=DEV)
    v = randn((B, Hkv, N, d), 7102, dtype="f32", device=DEV)
    h0 = lo - (W - 1)
    o = yk.yoco_swa_attn_halo(q[:, :, lo:hi].contiguous(), k[:, :, h0:hi].contiguous(), v[:, :, h0:hi].contiguous(), W)
    torch.cuda.synchronize()
    ref, _ = oracle.swa_attention(to64(q), to64(k), to64(v), W, rows=list(range(lo, hi)))
    check(to64(o), ref[:, :, lo:hi], "f32", "unaligned halo shard")


@pytest.mark.parametrize("dt,cuts", [("bf16", [1000, 1001, 5000, 8192]), ("f32", [64, 4096]),
                                     ("bf16", [2048, 4096, 6144, 8192])])
def test_sharded_decode_merge_equals_the_whole_cache(dt, cuts):
    B, Hq, Hkv, d, ctx = 3, 16, 4, 128, cuts[-1]
    print(f"sharded decode {dt} cuts={cuts}", flush=True)
    q = randn((B, Hq, d), 7200 + len(cuts), dtype=dt, device=DEV)
    k = randn((B, Hkv, ctx, d), 7201, dtype=dt, device=DEV)
    v = randn((B, Hkv, ctx, d), 7202, dtype=dt, device=DEV)
    full = yk.yoco_cross_attn_decode(q, k, v, ctx)
    parts, lses = [], []
    lo = 0
    for hi in cuts:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
        parts.append(yk.yoco_cross_attn_decode(q, k[:, :, lo:hi].contiguous(), v[:, :, lo:hi].contiguous(), hi - lo,
                                               lse=lse))
        lses.append(lse)
        lo = hi
    lse_m = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    merged = yk.yoco_attn_merge(torch.stack(parts), torch.stack(lses), lse=lse_m)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.decode_attention(to64(q), to64(k), to64(v), [ctx])
    check(to64(merged), ref_o, dt, "merged shards vs oracle", rel_axes=(2,))
    check(to64(full), ref_o, dt, "whole cache vs oracle", rel_axes=(2,))
    tol = 1e-3 if dt == "bf16" else 1e-5
    assert np.max(np.abs(to64(lse_m) - ref_lse)) <= tol
    # the merge of the oracle's own shard results from the GPU's shard outputs
    mo, ml = oracle.merge_partial_attention(np.stack([to64(p) for p in parts]), np.stack([to64(x) for x in lses]))
    assert np.max(np.abs(to64(merged) - mo)) <= (2e-2 if dt == "bf16" else 1e-5)


def test_one_million_tokens_split_eight_ways():
    """The 1M-token workload's shard shapes (8 devices): a 131072-row
    sliding-window shard with its 1024-row halo, bitwise equal to those rows
    of the full sequence; the last-token decode over 8 cache shards of 131072
    rows, merged, against the whole-cache decode and sampled oracle heads."""
    B, Hq, Hkv, d, N, W, P = 1, 32, 8, 128, 1 << 20, 1024, 8
    C = N // P
    q = randn((B, Hq, N, d), 7300, device=DEV)
    k = randn((B, Hkv, N, d), 7301, device=DEV)
    v = randn((B, Hkv, N, d), 7302, device=DEV)
    full = yk.yoco_swa_attn(q, k, v, W)
    s = 5
    lo, hi = s * C, (s + 1) * C
    o = yk.yoco_swa_attn_halo(q[:, :, lo:hi].contiguous(), k[:, :, lo - W:hi].contiguous(),
                              v[:, :, lo - W:hi].contiguous(), W)
    torch.cuda.synchronize()
    assert torch.equal(o, full[:, :, lo:hi])
    del full, o
    qd = q[:, :, N - 1].contiguous()
    whole = yk.yoco_cross_attn_decode(qd, k, v, N)
    parts, lses = [], []
    for i in range(P):
        lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
        parts.append(yk.yoco_cross_attn_decode(qd, k[:, :, i * C:(i + 1) * C].contiguous(),
                                               v[:, :, i * C:(i + 1) * C].contiguous(), C, lse=lse))
        lses.append(lse)
    merged = yk.yoco_attn_merge(torch.stack(parts), torch.stack(lses))
    torch.cuda.synchronize()
    check(to64(merged), to64(whole), "bf16", "merged 8 shards vs whole cache", rel_axes=(2,))
    bh = [(0, 0), (0, 13), (0, 31)]
    ref, _ = oracle.decode_attention(to64(qd), to64(k), to64(v), [N], bh=bh)
    for b, h in bh:
        check(to64(merged)[b, h][None], ref[b, h][None], "bf16", f"merged 1M decode head {h}")
