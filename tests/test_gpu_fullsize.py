"""Parity at the workloads' full sizes, in the launch configuration bench.py
times, on sampled outputs the oracle computes one by one (row sampling is
exact: the oracle computes every row independently)."""
import numpy as np
import pytest
import torch

import oracle
import shared_kv_attention_amd as yk
from shared_kv_attention_amd.synth import WORKLOADS, randn, seed_for
from tests._tol import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rows(n, w, extra):
    rows = {0, 1, w - 2, w - 1, w, w + 1, n // 2, n - 2, n - 1}
    rng = np.random.default_rng(extra)
    rows |= set(int(r) for r in rng.integers(0, n, 12))
    return sorted(r for r in rows if 0 <= r < n)


def test_prefill_3b_full_size_sampled():
    wl = WORKLOADS["prefill_3b_bf16"]
    B, N, D, Hq, Hkv, d, W = wl.batch, wl.seq, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.window
    print(f"full-size prefill N={N} Hq={Hq} Hkv={Hkv}", flush=True)
    q = randn((B, Hq, N, d), seed_for(wl.wid, 10), device=DEV)
    k = randn((B, Hkv, N, d), seed_for(wl.wid, 11), device=DEV)
    v = randn((B, Hkv, N, d), seed_for(wl.wid, 12), device=DEV)
    o = yk.yoco_swa_attn(q, k, v, W)
    x = randn((B, N, D), seed_for(wl.wid, 0), device=DEV)
    wk = randn((Hkv * d, D), seed_for(wl.wid, 1), std=wl.weight_std, device=DEV)
    wv = randn((Hkv * d, D), seed_for(wl.wid, 2), std=wl.weight_std, device=DEV)
    kc = torch.empty(B, Hkv, N, d, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    yk.yoco_global_kv_proj(x, wk, wv, kc, vc)
    qc = randn((B, Hq, N, d), seed_for(wl.wid, 200), device=DEV)
    oc = yk.yoco_cross_attn_prefill(qc, kc, vc)
    torch.cuda.synchronize()
    rows = _rows(N, W, 1)
    ro, _ = oracle.swa_attention(to64(q), to64(k), to64(v), W, rows=rows)
    check(to64(o)[:, :, rows], ro[:, :, rows], "bf16", "swa", rel_axes=(3,))
    rk, rv = oracle.global_kv_proj(to64(x), to64(wk), to64(wv), Hkv, d, rows=rows)
    check(to64(kc)[:, :, rows], rk[:, :, rows], "bf16", "K", rel_axes=(3,))
    check(to64(vc)[:, :, rows], rv[:, :, rows], "bf16", "V", rel_axes=(3,))
    rc, _ = oracle.cross_prefill_attention(to64(qc), to64(kc), to64(vc), rows=rows)
    check(to64(oc)[:, :, rows], rc[:, :, rows], "bf16", "cross", rel_axes=(3,))


def test_decode_32k_full_size_sampled():
    wl = WORKLOADS["decode_32k_bf16"]
    B, ctx, Hq, Hkv, d = wl.batch, wl.seq, wl.n_heads, wl.n_kv_heads, wl.head_dim
    print(f"full-size decode B={B} ctx={ctx}", flush=True)
    kc = randn((B, Hkv, ctx, d), seed_for(wl.wid, 0), device=DEV)
    vc = randn((B, Hkv, ctx, d), seed_for(wl.wid, 1), device=DEV)
    q = randn((B, Hq, d), seed_for(wl.wid, 2), device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    o = yk.yoco_cross_attn_decode(q, kc, vc, ctx, lse=lse)
    torch.cuda.synchronize()
    g = Hq // Hkv
    for b, kvh in [(0, 0), (7, 3), (15, 7)]:
        heads = list(range(kvh * g, kvh * g + g))
        ro, rl = oracle.decode_attention(to64(q[b:b + 1, heads]), to64(kc[b:b + 1, kvh:kvh + 1]),
                                         to64(vc[b:b + 1, kvh:kvh + 1]), [ctx])
        check(to64(o[b:b + 1, heads]), ro, "bf16", f"decode b={b} kvh={kvh}", rel_axes=(2,))
        assert np.abs(to64(lse[b:b + 1, heads]) - rl).max() <= 1e-3


def test_early_exit_1m_full_size_sampled():
    """1M-token early-exit flow: SWA layer, projection of all tokens, then the
    last position through a cross layer as a decode call over the 1M cache."""
    wl = WORKLOADS["early_exit_1m_bf16"]
    B, N, D, Hq, Hkv, d, W = wl.batch, wl.seq, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.window
    print(f"full-size early exit N={N}", flush=True)
    q = randn((B, Hq, N, d), seed_for(wl.wid, 10), device=DEV)
    k = randn((B, Hkv, N, d), seed_for(wl.wid, 11), device=DEV)
    v = randn((B, Hkv, N, d), seed_for(wl.wid, 12), device=DEV)
    o = yk.yoco_swa_attn(q, k, v, W)
    torch.cuda.synchronize()
    rows = _rows(N, W, 2)
    # the oracle only needs the window of keys of each sampled row: query t
    # is the last of the window's positions lo..t
    for t in rows:
        lo = max(0, t - W + 1)
        n = t - lo + 1
        ro, _ = oracle.cross_prefill_attention(to64(q[:, :, t:t + 1]), to64(k[:, :, lo:t + 1]),
                                               to64(v[:, :, lo:t + 1]), n_kv=n, q_offset=n - 1)
        check(to64(o[:, :, t:t + 1]), ro, "bf16", f"swa row {t}", rel_axes=(3,))
    del q, k, v, o
    x = randn((B, N, D), seed_for(wl.wid, 0), device=DEV)
    wk = randn((Hkv * d, D), seed_for(wl.wid, 1), std=wl.weight_std, device=DEV)
    wv = randn((Hkv * d, D), seed_for(wl.wid, 2), std=wl.weight_std, device=DEV)
    kc = torch.empty(B, Hkv, N, d, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    yk.yoco_global_kv_proj(x, wk, wv, kc, vc)
    torch.cuda.synchronize()
    rk, rv = oracle.global_kv_proj(to64(x[:, rows]), to64(wk), to64(wv), Hkv, d)
    check(to64(kc[:, :, rows]), rk, "bf16", "K", rel_axes=(3,))
    check(to64(vc[:, :, rows]), rv, "bf16", "V", rel_axes=(3,))
    del x
    ql = randn((B, Hq, d), seed_for(wl.wid, 300), device=DEV)
    od = yk.yoco_cross_attn_decode(ql, kc, vc, N)
    torch.cuda.synchronize()
    g = Hq // Hkv
    for kvh in (0, Hkv - 1):
        heads = list(range(kvh * g, kvh * g + g))
        ro, _ = oracle.decode_attention(to64(ql[:, heads]), to64(kc[:, kvh:kvh + 1]), to64(vc[:, kvh:kvh + 1]), [N])
        check(to64(od[:, heads]), ro, "bf16", f"1M decode kvh={kvh}", rel_axes=(2,))


def test_decode_512k_fp8_full_size_sampled():
    wl = WORKLOADS["decode_512k_fp8"]
    B, ctx, Hq, Hkv, d = wl.batch, wl.seq, wl.n_heads, wl.n_kv_heads, wl.head_dim
    print(f"full-size fp8 decode B={B} ctx={ctx}", flush=True)
    caches, scales = [], []
    for idx in (0, 1):
        kf = randn((B, Hkv, ctx, d), seed_for(wl.wid, idx), dtype="f32", device=DEV)
        codes, sc = yk.yoco_kv_quantize_fp8(kf)
        torch.cuda.synchronize()
        # scales: oracle amax over each head, streamed head by head
        for h in (0, Hkv - 1):
            slab = kf[:, h].cpu().numpy()
            amax = np.float32(np.abs(slab).max())
            assert sc[h].item() == np.float32(amax / np.float32(448.0))
            # codes of sampled rows, bit-exact (encoded with the whole head's scale)
            y = slab[:, [0, 1, ctx // 2, ctx - 1]] / np.float32(sc[h].item())
            assert np.array_equal(codes[:, h, [0, 1, ctx // 2, ctx - 1]].cpu().numpy(), oracle.e4m3_encode(y))
        caches.append(codes)
        scales.append(sc)
        del kf
    q = randn((B, Hq, d), seed_for(wl.wid, 2), device=DEV)
    o = yk.yoco_cross_attn_decode(q, caches[0], caches[1], ctx, k_scale=scales[0], v_scale=scales[1])
    torch.cuda.synchronize()
    g = Hq // Hkv
    for b, kvh in [(0, 0), (B - 1, Hkv - 1)]:
        heads = list(range(kvh * g, kvh * g + g))
        kd = oracle.dequantize_kv_fp8(caches[0][b:b + 1, kvh:kvh + 1].cpu().numpy(), scales[0][kvh:kvh + 1].cpu().numpy())
        vd = oracle.dequantize_kv_fp8(caches[1][b:b + 1, kvh:kvh + 1].cpu().numpy(), scales[1][kvh:kvh + 1].cpu().numpy())
        ro, _ = oracle.decode_attention(to64(q[b:b + 1, heads]), kd, vd, [ctx])
        check(to64(o[b:b + 1, heads]), ro, "bf16", f"fp8 decode b={b} kvh={kvh}", rel_axes=(2,))
