"""GPU parity of yoco_swa_attn and yoco_cross_attn_prefill against the oracle,
and the method's invariants on the kernels (causality, window locality,
sharing, constant values, determinism)."""
import math

import numpy as np
import pytest
import torch

import oracle
import shared_kv_attention_amd as yk
from shared_kv_attention_amd.synth import randn
from tests._tol import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed):
    q = randn((B, Hq, Nq, d), seed, dtype=dt, device=DEV)
    k = randn((B, Hkv, Nk, d), seed + 1, dtype=dt, device=DEV)
    v = randn((B, Hkv, Nk, d), seed + 2, dtype=dt, device=DEV)
    return q, k, v


SWA_CASES = [
    # B, Hq, Hkv, N, d, W, dtype
    (1, 4, 1, 256, 64, 32, "f32"),       # tiny-block shapes
    (2, 6, 2, 300, 128, 70, "bf16"),     # ragged tail, several tiles
    (1, 8, 2, 200, 64, 1, "bf16"),       # window 1
    (1, 3, 1, 130, 128, 1000, "bf16"),   # window >= N: causal
    (2, 4, 4, 333, 128, 129, "f32"),
    (1, 24, 8, 517, 128, 256, "bf16"),   # 3B head grouping
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,W,dt", SWA_CASES)
def test_swa_parity(B, Hq, Hkv, N, d, W, dt):
    print(f"swa parity B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} W={W} {dt}", flush=True)
    q, k, v = _inputs(B, Hq, Hkv, N, N, d, dt, 100)
    lse = torch.empty(B, Hq, N, dtype=torch.float32, device=DEV)
    o = yk.yoco_swa_attn(q, k, v, W, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_attention(to64(q), to64(k), to64(v), W)
    check(to64(o), ro, dt, "swa O", rel_axes=(2, 3))
    tol = 1e-5 if dt == "f32" else 1e-3
    assert np.abs(to64(lse) - rl).max() <= tol


PREFILL_CASES = [
    # B, Hq, Hkv, Nq, n_kv, n_cap, q_offset, d, dtype
    (1, 4, 1, 256, 256, 256, 0, 64, "f32"),
    (2, 6, 2, 190, 190, 256, 0, 128, "bf16"),
    (1, 8, 2, 70, 300, 320, 230, 128, "bf16"),   # chunk of queries at an offset
    (2, 4, 2, 1, 257, 300, 256, 64, "bf16"),     # a single (last) position
    (1, 24, 8, 400, 400, 400, 0, 128, "bf16"),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,n_kv,n_cap,off,d,dt", PREFILL_CASES)
def test_cross_prefill_parity(B, Hq, Hkv, Nq, n_kv, n_cap, off, d, dt):
    print(f"prefill parity B={B} Hq={Hq} Nq={Nq} n_kv={n_kv} n_cap={n_cap} off={off} d={d} {dt}", flush=True)
    q, k, v = _inputs(B, Hq, Hkv, Nq, n_cap, d, dt, 200)
    if n_cap > n_kv:   # rows past the valid ones hold garbage that must never be read
        k[:, :, n_kv:] = float("nan")
        v[:, :, n_kv:] = float("nan")
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=DEV)
    o = yk.yoco_cross_attn_prefill(q, k, v, n_kv=n_kv, q_offset=off, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.cross_prefill_attention(to64(q), to64(k)[:, :, :n_kv], to64(v)[:, :, :n_kv], n_kv=n_kv,
                                            q_offset=off)
    check(to64(o), ro, dt, "prefill O", rel_axes=(2, 3))
    tol = 1e-5 if dt == "f32" else 1e-3
    assert np.abs(to64(lse) - rl).max() <= tol


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_causality_bitwise_on_gpu(dt):
    B, Hq, Hkv, N, d = 1, 4, 2, 300, 128
    q, k, v = _inputs(B, Hq, Hkv, N, N, d, dt, 300)
    t_star = 150
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for t in (q2, k2, v2):
        t[:, :, t_star + 1:] = 1e4 * torch.sign(randn(t[:, :, t_star + 1:].shape, 7, dtype=dt, device=DEV))
    for fn in (lambda a, b_, c: yk.yoco_swa_attn(a, b_, c, 64),
               lambda a, b_, c: yk.yoco_cross_attn_prefill(a, b_, c)):
        o1, o2 = fn(q, k, v), fn(q2, k2, v2)
        torch.cuda.synchronize()
        assert torch.equal(o1[:, :, :t_star + 1], o2[:, :, :t_star + 1])


def test_window_locality_bitwise_on_gpu():
    B, Hq, Hkv, N, d, W = 1, 4, 1, 400, 128, 100
    q, k, v = _inputs(B, Hq, Hkv, N, N, d, "bf16", 400)
    t0 = 250
    k2, v2 = k.clone(), v.clone()
    k2[:, :, :t0 - W + 1] = 1e4
    v2[:, :, :t0 - W + 1] = -1e4
    o1 = yk.yoco_swa_attn(q, k, v, W)
    o2 = yk.yoco_swa_attn(q, k2, v2, W)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, t0:], o2[:, :, t0:])


def test_sharing_shared_cache_equals_copies_bitwise():
    """Several cross layers reading one cache == each reading its own copy."""
    B, Hq, Hkv, N, d = 1, 8, 2, 260, 128
    _, k, v = _inputs(B, Hq, Hkv, N, N, d, "bf16", 500)
    outs_shared, outs_copy = [], []
    for layer in range(3):
        q = randn((B, Hq, N, d), 510 + layer, device=DEV)
        outs_shared.append(yk.yoco_cross_attn_prefill(q, k, v))
        outs_copy.append(yk.yoco_cross_attn_prefill(q, k.clone(), v.clone()))
    torch.cuda.synchronize()
    for a, b in zip(outs_shared, outs_copy):
        assert torch.equal(a, b)


def test_constant_values_give_ones_and_rows_sum_to_one():
    B, Hq, Hkv, N, d = 1, 4, 2, 200, 128
    q, k, _ = _inputs(B, Hq, Hkv, N, N, d, "bf16", 600)
    v = torch.ones(B, Hkv, N, d, dtype=torch.bfloat16, device=DEV)
    for o in (yk.yoco_swa_attn(q * 4, k * 4, v, 37), yk.yoco_cross_attn_prefill(q * 4, k * 4, v)):
        torch.cuda.synchronize()
        assert (o.float() - 1).abs().max().item() <= 2e-2


def test_deterministic_rerun():
    q, k, v = _inputs(2, 6, 2, 300, 300, 128, "bf16", 700)
    a = yk.yoco_swa_attn(q, k, v, 50)
    b = yk.yoco_swa_attn(q, k, v, 50)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_planted_key_dominates_across_tiles():
    B, Hq, Hkv, N, d = 1, 4, 1, 512, 128
    q, k, v = _inputs(B, Hq, Hkv, N, N, d, "bf16", 800)
    # key 40 aligned with every query: dominates rows >= 40 in causal attention
    k[0, 0, 40] = (q[0, :, 300:].float().mean(dim=(0, 1)) * 40).to(torch.bfloat16)
    o = yk.yoco_cross_attn_prefill(q, k, v)
    torch.cuda.synchronize()
    ro, _ = oracle.cross_prefill_attention(to64(q), to64(k), to64(v), rows=list(range(300, 512)))
    check(to64(o)[:, :, 300:], ro[:, :, 300:], "bf16", "planted", rel_axes=(2, 3))


def test_cache_past_2_pow_31_bytes_reads_its_first_keys():
    """A cache of 2^24 rows of bf16 d = 128 (4 GiB per tensor): the first key
    tile's byte count is past 2^31.  One query at the last position, key 0
    planted to dominate every other (all zero) key: the output must be v[0]
    -- a tile that loaded as zeros would give the mean of V instead."""
    n, d = 1 << 24, 128
    print(f"prefill over {n} cache rows", flush=True)
    q = randn((1, 1, 1, d), 810, device=DEV)
    k = torch.zeros(1, 1, n, d, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(1, 1, n, d, dtype=torch.bfloat16, device=DEV)
    k[0, 0, 0] = (q[0, 0, 0].float() * 5).to(torch.bfloat16)    # score ~ 5 |q|^2 / sqrt(d) ~ 56 >> ln(2^24)
    v[0, 0, 0] = randn((d,), 811, device=DEV)
    v[0, 0, 1:4096] = randn((4095, d), 812, device=DEV)
    o = yk.yoco_cross_attn_prefill(q, k, v, q_offset=n - 1)
    torch.cuda.synchronize()
    ro, _ = oracle.decode_attention(to64(q)[:, :, 0], to64(k[:, :, :4096]), to64(v[:, :, :4096]), [4096])
    # the other 2^24 - 4096 keys have score 0 and value 0: they only add to the
    # denominator, which the planted key's weight e^56 makes negligible
    check(to64(o)[:, :, 0], ro, "bf16", "2^24-row cache", rel_axes=(2,))
    assert (o[0, 0, 0].float() - v[0, 0, 0].float()).abs().max().item() <= 2e-2
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["swa", "causal"])
def test_attention_writes_nothing_outside_its_outputs(kind, dt):
    """o and lse inside NaN-filled guard regions (ragged query count, several
    query tiles): every guard element is still NaN afterwards, every output
    element finite."""
    B, Hq, Hkv, N, d, G = 2, 6, 2, 333, 128, 8192
    q, k, v = _inputs(B, Hq, Hkv, N, N, d, dt, 820)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    obuf = torch.full((G + B * Hq * N * d + G,), float("nan"), dtype=tdt, device=DEV)
    lbuf = torch.full((G + B * Hq * N + G,), float("nan"), dtype=torch.float32, device=DEV)
    o = obuf[G:G + B * Hq * N * d].view(B, Hq, N, d)
    lse = lbuf[G:G + B * Hq * N].view(B, Hq, N)
    if kind == "swa":
        yk.yoco_swa_attn(q, k, v, 100, o=o, lse=lse)
    else:
        yk.yoco_cross_attn_prefill(q[:, :, 33:].contiguous(), k, v, q_offset=33, o=obuf[G:G + B * Hq * (N - 33) * d]
                                   .view(B, Hq, N - 33, d), lse=lbuf[G:G + B * Hq * (N - 33)].view(B, Hq, N - 33))
        o = obuf[G:G + B * Hq * (N - 33) * d]
        lse = lbuf[G:G + B * Hq * (N - 33)]
    torch.cuda.synchronize()
    for buf, m in ((obuf, o.numel()), (lbuf, lse.numel())):
        assert bool(torch.isnan(buf[:G]).all()) and bool(torch.isnan(buf[G + m:]).all())
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())


def test_prefill_step_graph_replays_match_eager():
    """The prefill step (window layers, the global projection, causal cross
    layers over the shared cache) captured as a HIP graph: every replay, with
    eager work and synchronisations between the replays, reproduces the eager
    step bitwise."""
    B, Hq, Hkv, N, d, D, W = 1, 8, 2, 640, 128, 512, 128
    swa = [_inputs(B, Hq, Hkv, N, N, d, "bf16", 1300 + 10 * i) for i in range(2)]
    x = randn((B, N, D), 1350, device=DEV)
    wk = randn((Hkv * d, D), 1351, std=0.05, device=DEV)
    wv = randn((Hkv * d, D), 1352, std=0.05, device=DEV)
    qc = [randn((B, Hq, N, d), 1360 + i, device=DEV) for i in range(2)]
    kc = torch.empty(B, Hkv, N, d, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    o_swa = [torch.empty(B, Hq, N, d, dtype=torch.bfloat16, device=DEV) for _ in swa]
    o_cross = [torch.empty(B, Hq, N, d, dtype=torch.bfloat16, device=DEV) for _ in qc]

    def step():
        for (q, k, v), o in zip(swa, o_swa):
            yk.yoco_swa_attn(q, k, v, W, o=o)
        yk.yoco_global_kv_proj(x, wk, wv, kc, vc)
        for q, o in zip(qc, o_cross):
            yk.yoco_cross_attn_prefill(q, kc, vc, o=o)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in o_swa + o_cross + [kc, vc]]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in o_swa + o_cross + [kc, vc]:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(o_swa + o_cross + [kc, vc], ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        step()   # eager work between replays
        torch.cuda.synchronize()
