"""The tiny float32 YOCO block with every attention call and the global KV
projection on the GPU (host glue -- RMSNorm of the self-decoder inputs,
per-layer projections, residual adds -- in float64 numpy), against the
float64 oracle block; and early exit on the GPU: the cross-decoder run on the
last position only (decode calls) equals the full cross prefill's last row."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.block import BlockParams
import shared_kv_attention_amd as yk
from shared_kv_attention_amd.synth import WORKLOADS, randn, seed_for

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _params(wl):
    D, Hq, Hkv, d = wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim
    idx = iter(range(1, 1000))
    r = lambda *shape: randn(shape, seed_for(wl.wid, next(idx)), std=wl.weight_std, dtype="f32").double().numpy()  # noqa: E731
    return BlockParams(
        n_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=wl.window,
        swa_wq=[r(Hq * d, D) for _ in range(wl.n_self_layers)],
        swa_wk=[r(Hkv * d, D) for _ in range(wl.n_self_layers)],
        swa_wv=[r(Hkv * d, D) for _ in range(wl.n_self_layers)],
        swa_wo=[r(D, Hq * d) for _ in range(wl.n_self_layers)],
        glob_wk=r(Hkv * d, D), glob_wv=r(Hkv * d, D),
        cross_wq=[r(Hq * d, D) for _ in range(wl.n_cross_layers)],
        cross_wo=[r(D, Hq * d) for _ in range(wl.n_cross_layers)])


def _norm(x, eps=1e-6):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _g(a):
    return torch.from_numpy(np.ascontiguousarray(a)).float().to(DEV)


def _heads(t, H, d):
    B, N, _ = t.shape
    return t.reshape(B, N, H, d).transpose(0, 2, 1, 3)


def _merge(t):
    B, H, N, d = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, N, H * d)


def _gpu_block(x, p, early_exit):
    Hq, Hkv, d, W = p.n_heads, p.n_kv_heads, p.head_dim, p.window
    B, N, D = x.shape
    for wq, wk, wv, wo in zip(p.swa_wq, p.swa_wk, p.swa_wv, p.swa_wo):
        n = _norm(x)
        q, k, v = (_heads(n @ w.T, h, d) for w, h in ((wq, Hq), (wk, Hkv), (wv, Hkv)))
        o = yk.yoco_swa_attn(_g(q), _g(k), _g(v), W)
        x = x + _merge(o.double().cpu().numpy()) @ wo.T
    kc = torch.empty(B, Hkv, N, d, dtype=torch.float32, device=DEV)
    vc = torch.empty_like(kc)
    yk.yoco_global_kv_proj(_g(x), _g(p.glob_wk), _g(p.glob_wv), kc, vc)
    if early_exit:
        last = x[:, -1]
        for wq, wo in zip(p.cross_wq, p.cross_wo):
            q = (_norm(last) @ wq.T).reshape(B, Hq, d)
            o = yk.yoco_cross_attn_decode(_g(q), kc, vc, N)
            last = last + o.double().cpu().numpy().reshape(B, Hq * d) @ wo.T
        return last
    for wq, wo in zip(p.cross_wq, p.cross_wo):
        q = _heads(_norm(x) @ wq.T, Hq, d)
        o = yk.yoco_cross_attn_prefill(_g(q), kc, vc)
        x = x + _merge(o.double().cpu().numpy()) @ wo.T
    return x


def test_tiny_block_matches_oracle_and_early_exit():
    wl = WORKLOADS["tiny_block_f32"]
    p = _params(wl)
    x = randn((wl.batch, wl.seq, wl.hidden), seed_for(wl.wid, 0), dtype="f32").double().numpy()
    ref, _ = oracle.yoco_block(x, p)
    out = _gpu_block(x, p, early_exit=False)
    err = np.abs(out - ref).max()
    print("tiny block max-abs error vs oracle:", err)
    assert err <= 1e-5
    last = _gpu_block(x, p, early_exit=True)
    ref_last, _ = oracle.yoco_block_early_exit(x, p)
    assert np.array_equal(ref_last, ref[:, -1])          # exact inside the oracle
    assert np.abs(last - ref_last).max() <= 1e-5
    assert np.abs(last - out[:, -1]).max() <= 1e-5       # early exit on the GPU
