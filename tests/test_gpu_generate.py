"""The one-token generation step on the GPU: the self-decoder's ring-cache
window decode (yoco_swa_decode, with its append of the current token), the
one-token append of the global KV projection (yoco_global_kv_proj at
N = 1, pos0 = t), and the cross-decoder decode calls -- each against the
oracle, and the whole tiny block generated token by token against the
oracle's full forward (causality: generation reproduces the prefill rows)."""
import numpy as np
import pytest
import torch

import oracle
import shared_kv_attention_amd as yk
from shared_kv_attention_amd.synth import WORKLOADS, randn
from _tol import check, to64
from test_gpu_block import _g, _norm, _params

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ring_from_sequence(k, v, pos, W):
    """GPU ring [B, Hkv, W, d] holding positions max(0, pos-W+1)..pos of the
    sequences k, v [B, Hkv, N, d] in slots t mod W; other slots hold 1e4
    (finite, far from any real value: a read of them would show)."""
    B, Hkv, _, d = k.shape
    kr = torch.full((B, Hkv, W, d), 1e4, dtype=k.dtype, device=DEV)
    vr = torch.full_like(kr, 1e4)
    for t in range(max(0, pos - W + 1), pos + 1):
        kr[:, :, t % W] = k[:, :, t]
        vr[:, :, t % W] = v[:, :, t]
    return kr, vr


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("W,pos", [(64, 0), (64, 10), (64, 63), (64, 64), (64, 201), (1024, 1023), (1024, 5000),
                                   (1, 9), (300, 299), (300, 1000)])
def test_swa_decode_matches_oracle(dt, d, W, pos):
    print(f"swa_decode dt={dt} d={d} W={W} pos={pos}", flush=True)
    B, Hq, Hkv = 2, 8, 2
    base = 7000 + 13 * W + pos % 97
    q = randn((B, Hq, d), base + 1, dtype=dt, device=DEV)
    kr = randn((B, Hkv, W, d), base + 2, dtype=dt, device=DEV)
    vr = randn((B, Hkv, W, d), base + 3, dtype=dt, device=DEV)
    kn = randn((B, Hkv, d), base + 4, dtype=dt, device=DEV)
    vn = randn((B, Hkv, d), base + 5, dtype=dt, device=DEV)
    before_k, before_v = kr.clone(), vr.clone()
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    o = yk.yoco_swa_decode(q, kr, vr, pos, k_new=kn, v_new=vn, lse=lse)
    torch.cuda.synchronize()
    # the append wrote exactly slot pos mod W, and nothing else
    s = pos % W
    assert torch.equal(kr[:, :, s], kn) and torch.equal(vr[:, :, s], vn)
    keep = [i for i in range(W) if i != s]
    assert torch.equal(kr[:, :, keep], before_k[:, :, keep]) and torch.equal(vr[:, :, keep], before_v[:, :, keep])
    ref_o, ref_lse = oracle.swa_ring_decode_attention(to64(q), to64(kr), to64(vr), pos)
    check(to64(o), ref_o, dt, f"swa_decode o (dt={dt} d={d} W={W} pos={pos})", rel_axes=(2,))
    tol = 1e-5 if dt == "f32" else 1e-3
    assert np.abs(to64(lse) - ref_lse).max() <= tol


@pytest.mark.parametrize("B,Hq,Hkv,W,pos,rows", [
    (2, 16, 2, 512, 700, None),          # 8 query heads per KV head: two head groups share each split
    (64, 8, 8, 8192, 10000, [0, 37, 63]),  # long splits: the whole-line K form (sampled sequences checked)
    (16, 32, 8, 1024, 1500, [0, 5, 15]),   # the generation shape: 16 splits of 64 slots
    (16, 64, 8, 1024, 700, [1, 9]),        # two head groups, 11 splits
])
def test_swa_decode_append_with_head_groups_and_long_splits(B, Hq, Hkv, W, pos, rows):
    """The append folded into the decode: the split holding slot pos mod W
    reads the token from k_new / v_new in every head group and in the
    whole-line K form; the ring ends up holding it."""
    d = 128
    print(f"swa_decode append B={B} Hq={Hq} Hkv={Hkv} W={W} pos={pos}", flush=True)
    q = randn((B, Hq, d), 7401 + B, device=DEV)
    kr = randn((B, Hkv, W, d), 7402 + B, device=DEV)
    vr = randn((B, Hkv, W, d), 7403 + B, device=DEV)
    kn = randn((B, Hkv, d), 7404 + B, device=DEV)
    vn = randn((B, Hkv, d), 7405 + B, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    o = yk.yoco_swa_decode(q, kr, vr, pos, k_new=kn, v_new=vn, lse=lse)
    torch.cuda.synchronize()
    s = pos % W
    assert torch.equal(kr[:, :, s], kn) and torch.equal(vr[:, :, s], vn)
    rows = list(range(B)) if rows is None else rows
    ref_o, ref_lse = oracle.swa_ring_decode_attention(to64(q[rows]), to64(kr[rows]), to64(vr[rows]), pos)
    check(to64(o[rows]), ref_o, "bf16", "swa_decode with append", rel_axes=(2,))
    assert np.abs(to64(lse[rows]) - ref_lse).max() <= 1e-3


def test_swa_decode_without_append_leaves_ring_untouched():
    B, Hq, Hkv, W, d = 1, 4, 1, 128, 64
    q = randn((B, Hq, d), 7101, device=DEV)
    kr = randn((B, Hkv, W, d), 7102, device=DEV)
    vr = randn((B, Hkv, W, d), 7103, device=DEV)
    kc, vc = kr.clone(), vr.clone()
    o = yk.yoco_swa_decode(q, kr, vr, 77)
    torch.cuda.synchronize()
    assert torch.equal(kr, kc) and torch.equal(vr, vc)
    ref, _ = oracle.swa_ring_decode_attention(to64(q), to64(kr), to64(vr), 77)
    check(to64(o), ref, "bf16", "swa_decode (no append)", rel_axes=(2,))


@pytest.mark.parametrize("W", [64, 100])
def test_swa_decode_equals_prefill_rows(W):
    """The window decode of position pos over a ring filled from a sequence
    equals row pos of the sliding-window prefill of that sequence."""
    B, Hq, Hkv, N, d = 2, 8, 2, 300, 128
    q = randn((B, Hq, N, d), 7201 + W, device=DEV)
    k = randn((B, Hkv, N, d), 7202 + W, device=DEV)
    v = randn((B, Hkv, N, d), 7203 + W, device=DEV)
    o_pre = yk.yoco_swa_attn(q, k, v, W)
    for pos in (0, 31, W - 1, W, 150, N - 1):
        print(f"swa_decode vs prefill W={W} pos={pos}", flush=True)
        kr, vr = _ring_from_sequence(k, v, pos, W)
        o_dec = yk.yoco_swa_decode(q[:, :, pos].contiguous(), kr, vr, pos)
        ref, _ = oracle.swa_attention(to64(q), to64(k), to64(v), W, rows=[pos])
        check(to64(o_dec), ref[:, :, pos], "bf16", f"decode pos {pos}", rel_axes=(2,))
        check(to64(o_dec), to64(o_pre[:, :, pos]), "bf16", f"decode vs prefill pos {pos}", rel_axes=(2,))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_projection_append_equals_prefill_rows_bitwise(dt):
    """Projecting one token per call into row pos0 = t gives, bitwise, the
    rows of the projection of the whole sequence (each row depends on its own
    token only, with the same arithmetic)."""
    B, N, D, Hkv, d = 2, 37, 256, 2, 64
    x = randn((B, N, D), 7301, dtype=dt, device=DEV)
    wk = randn((Hkv * d, D), 7302, std=0.05, dtype=dt, device=DEV)
    wv = randn((Hkv * d, D), 7303, std=0.05, dtype=dt, device=DEV)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    kp = torch.zeros(B, Hkv, N, d, dtype=tdt, device=DEV)
    vp = torch.zeros_like(kp)
    yk.yoco_global_kv_proj(x, wk, wv, kp, vp)
    ka = torch.zeros_like(kp)
    va = torch.zeros_like(kp)
    for t in range(N):
        yk.yoco_global_kv_proj(x[:, t:t + 1].contiguous(), wk, wv, ka, va, pos0=t)
    torch.cuda.synchronize()
    assert torch.equal(ka, kp) and torch.equal(va, vp)


def test_tiny_block_generation_matches_oracle():
    """The tiny float32 block generated token by token on the GPU -- ring
    decode with append for the self-decoder, one-row projection append, cross
    decode over rows 0..t -- equals the oracle's full forward rows."""
    wl = WORKLOADS["tiny_block_f32"]
    p = _params(wl)
    x = randn((wl.batch, wl.seq, wl.hidden), 1000 * wl.wid + 900, dtype="f32").double().numpy()
    ref, _ = oracle.yoco_block(x, p)
    Hq, Hkv, d, W = p.n_heads, p.n_kv_heads, p.head_dim, p.window
    B, N, D = x.shape
    rings = [(torch.zeros(B, Hkv, W, d, device=DEV), torch.zeros(B, Hkv, W, d, device=DEV)) for _ in p.swa_wq]
    kc = torch.zeros(B, Hkv, N, d, device=DEV)
    vc = torch.zeros_like(kc)
    out = np.empty_like(x)
    for t in range(N):
        h = x[:, t]
        for (wq, wk, wv, wo), (kr, vr) in zip(zip(p.swa_wq, p.swa_wk, p.swa_wv, p.swa_wo), rings):
            n = _norm(h)
            q = _g((n @ wq.T).reshape(B, Hq, d))
            kn = _g((n @ wk.T).reshape(B, Hkv, d))
            vn = _g((n @ wv.T).reshape(B, Hkv, d))
            o = yk.yoco_swa_decode(q, kr, vr, t, k_new=kn, v_new=vn)
            h = h + o.double().cpu().numpy().reshape(B, Hq * d) @ wo.T
        yk.yoco_global_kv_proj(_g(h[:, None, :]), _g(p.glob_wk), _g(p.glob_wv), kc, vc, pos0=t)
        for wq, wo in zip(p.cross_wq, p.cross_wo):
            q = _g((_norm(h) @ wq.T).reshape(B, Hq, d))
            o = yk.yoco_cross_attn_decode(q, kc, vc, t + 1)
            h = h + o.double().cpu().numpy().reshape(B, Hq * d) @ wo.T
        out[:, t] = h
    check(out, ref, "f32", "tiny block generated token by token")


def test_generation_step_graph_replays_match_eager():
    """One generation step (ring decode with its append, the projection append,
    cross decode) captured as a HIP graph: every replay, with eager work and
    synchronisations between the replays, reproduces the eager step bitwise.
    The cross cache is long enough for the whole-line K form of the decode."""
    B, Hq, Hkv, d, W, D, ctx = 32, 32, 8, 128, 256, 256, 16384
    pos = ctx - 1
    kr = randn((B, Hkv, W, d), 970, device=DEV)
    vr = randn((B, Hkv, W, d), 971, device=DEV)
    kc = randn((B, Hkv, ctx, d), 972, device=DEV)
    vc = randn((B, Hkv, ctx, d), 973, device=DEV)
    wk = randn((Hkv * d, D), 974, std=0.05, device=DEV)
    wv = randn((Hkv * d, D), 975, std=0.05, device=DEV)
    qs, qc = randn((B, Hq, d), 976, device=DEV), randn((B, Hq, d), 977, device=DEV)
    kn, vn = randn((B, Hkv, d), 978, device=DEV), randn((B, Hkv, d), 979, device=DEV)
    hid = randn((B, 1, D), 980, device=DEV)
    o_self = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=DEV)
    o_cross = torch.empty_like(o_self)
    ws_s = torch.empty(yk.yoco_swa_decode_workspace_bytes(B, Hq, Hkv, W, d), dtype=torch.uint8, device=DEV)
    ws_c = torch.empty(yk.yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d), dtype=torch.uint8, device=DEV)

    def step():
        yk.yoco_swa_decode(qs, kr, vr, pos, k_new=kn, v_new=vn, o=o_self, workspace=ws_s)
        yk.yoco_global_kv_proj(hid, wk, wv, kc, vc, pos0=pos)
        yk.yoco_cross_attn_decode(qc, kc, vc, ctx, o=o_cross, workspace=ws_c)

    step()
    torch.cuda.synchronize()
    ref = (o_self.clone(), o_cross.clone(), kr.clone(), kc[:, :, pos].clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        o_self.fill_(0)
        o_cross.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (o_self, o_cross, kr, kc[:, :, pos])
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        step()   # eager work between replays
        torch.cuda.synchronize()
