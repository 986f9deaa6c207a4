"""GPU parity of the block's position-wise layers (yoco_qkv_proj, yoco_swiglu,
yoco_linear_residual) against the float64 oracle, and the tiny float32 YOCO
block run wholly on the GPU (every norm, projection, attention, feed-forward
and residual add in libyoco) against the oracle block, full forward and early
exit.

Tolerances: float32 |out - ref| <= 1e-5 max(1, |ref|) (values O(1)).  bf16:
these outputs are unnormalised products (a SwiGLU activation reaches ~10), so
every element must satisfy |out - ref| <= 8e-3 |ref| + 2e-2 rms(ref) and every
row a relative L2 error <= 1e-2: the bf16 output rounding is at most
2^-8 |ref|; with a norm gain, x * gamma is rounded to bf16 before the product,
which perturbs each pre-activation by about 2^-8 / sqrt(3) of its rms, and
SwiGLU multiplies two pre-activations (so the perturbation is scaled by the
other factor, up to ~4); an indexing mistake gives errors of the order of the
values themselves."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.block import BlockParams
import shared_kv_attention_amd as yk
from shared_kv_attention_amd.synth import WORKLOADS, randn, seed_for
from _tol import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def glue_check(out, ref, dt, what):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.all(np.isfinite(out)), f"{what}: non-finite"
    err = np.abs(out - ref)
    if dt == "f32":
        bound = 1e-5 * np.maximum(1.0, np.abs(ref))
        worst = np.argmax(err - bound)
        assert np.all(err <= bound), f"{what}: err {err.flat[worst]:.3e} at |ref| {abs(ref.flat[worst]):.3e}"
        return
    rms = np.sqrt(np.mean(ref ** 2))
    bound = 8e-3 * np.abs(ref) + 2e-2 * rms
    worst = np.argmax(err - bound)
    assert np.all(err <= bound), f"{what}: err {err.flat[worst]:.3e} > {bound.flat[worst]:.3e}"
    rows = ref.reshape(-1, ref.shape[-1])
    rel = np.linalg.norm((out - ref).reshape(rows.shape), axis=1) / np.maximum(np.linalg.norm(rows, axis=1), 1e-30)
    assert rel.max() <= 1e-2, f"{what}: row relative L2 {rel.max():.3e}"


def _tdt(dt):
    return torch.float32 if dt == "f32" else torch.bfloat16


def _gain(D, seed, dt):
    return (1 + 0.5 * randn((D,), seed, dtype=dt, device=DEV).float()).to(_tdt(dt))


QKV_CASES = [
    # B, N, D, Hq, Hkv, d, gain, dtype
    (1, 77, 256, 4, 1, 64, False, "f32"),
    (2, 200, 384, 3, 1, 128, True, "bf16"),
    (1, 1, 128, 2, 0, 64, False, "bf16"),        # q only, one token
    (1, 300, 192, 6, 2, 64, True, "f32"),
    (3, 129, 512, 8, 0, 128, False, "bf16"),     # cross-layer query projection
    (3, 7, 384, 3, 1, 128, True, "bf16"),        # 21 tokens: the few-token form, two token groups
    (1, 64, 256, 2, 2, 64, False, "bf16"),       # 64 tokens, the largest few-token case
]


@pytest.mark.parametrize("B,N,D,Hq,Hkv,d,gain,dt", QKV_CASES)
def test_qkv_proj_matches_oracle(B, N, D, Hq, Hkv, d, gain, dt):
    print(f"qkv_proj B={B} N={N} D={D} Hq={Hq} Hkv={Hkv} d={d} gain={gain} {dt}", flush=True)
    s = 1.0 / math.sqrt(D)
    x = randn((B, N, D), 3000 + N, dtype=dt, device=DEV)
    wq = randn((Hq * d, D), 3001, std=s, dtype=dt, device=DEV)
    wk = randn((Hkv * d, D), 3002, std=s, dtype=dt, device=DEV) if Hkv else None
    wv = randn((Hkv * d, D), 3003, std=s, dtype=dt, device=DEV) if Hkv else None
    g = _gain(D, 3004, dt) if gain else None
    q, k, v = yk.yoco_qkv_proj(x, wq, d, wk, wv, norm_w=g)
    torch.cuda.synchronize()
    g64 = None if g is None else to64(g)
    rq, _ = oracle.global_kv_proj(to64(x), to64(wq), to64(wq), Hq, d, gamma=g64)
    glue_check(to64(q), rq, dt, "q")
    if Hkv:
        rk, rv = oracle.global_kv_proj(to64(x), to64(wk), to64(wv), Hkv, d, gamma=g64)
        glue_check(to64(k), rk, dt, "k")
        glue_check(to64(v), rv, dt, "v")
    else:
        assert k is None and v is None


SWIGLU_CASES = [
    # B, N, D, F, gain, dtype
    (1, 77, 256, 768, False, "f32"),
    (2, 130, 384, 344, True, "bf16"),     # F not a multiple of the 64-feature tile
    (1, 1, 128, 64, False, "bf16"),
    (1, 257, 192, 520, True, "f32"),
    (3, 11, 384, 344, True, "bf16"),      # 33 tokens: few-token form, F not a multiple of its 8-row groups
    (16, 1, 256, 8192, False, "bf16"),    # one token for each of 16 sequences
]


@pytest.mark.parametrize("B,N,D,F,gain,dt", SWIGLU_CASES)
def test_swiglu_matches_oracle(B, N, D, F, gain, dt):
    print(f"swiglu B={B} N={N} D={D} F={F} gain={gain} {dt}", flush=True)
    s = 1.0 / math.sqrt(D)
    x = randn((B, N, D), 3100 + N, dtype=dt, device=DEV)
    wg = randn((F, D), 3101, std=s, dtype=dt, device=DEV)
    wu = randn((F, D), 3102, std=s, dtype=dt, device=DEV)
    g = _gain(D, 3103, dt) if gain else None
    h = yk.yoco_swiglu(x, wg, wu, norm_w=g)
    torch.cuda.synchronize()
    xg, wg64, wu64 = to64(x), to64(wg), to64(wu)
    g64 = None if g is None else to64(g)
    ref = np.stack([np.stack([oracle.swiglu_hidden_row(xg[b, n], wg64, wu64, g64) for n in range(N)])
                    for b in range(B)])
    glue_check(to64(h), ref, dt, "swiglu h")


RES_CASES = [
    # B, N, K, F, a_heads, dtype
    (1, 77, 256, 256, 4, "f32"),      # W_o over a head-major attention output (4 heads of 64)
    (2, 130, 384, 192, 3, "bf16"),    # 3 heads of 128
    (1, 200, 768, 256, 0, "f32"),     # W_down over row-major activations
    (3, 1, 512, 128, 0, "bf16"),
    (1, 300, 1024, 520, 0, "bf16"),   # F not a multiple of the 128-feature tile
    (5, 8, 512, 200, 4, "bf16"),      # 40 tokens, head-major gather, few-token form
    (1, 1, 8192, 3072, 0, "bf16"),    # one token through W_down at the 3B shape
]


@pytest.mark.parametrize("B,N,K,F,a_heads,dt", RES_CASES)
def test_linear_residual_matches_oracle(B, N, K, F, a_heads, dt):
    print(f"linear_residual B={B} N={N} K={K} F={F} heads={a_heads} {dt}", flush=True)
    if a_heads:
        a = randn((B, a_heads, N, K // a_heads), 3200 + N, dtype=dt, device=DEV)
        rows = to64(a).transpose(0, 2, 1, 3).reshape(B, N, K)     # the concatenation over heads
    else:
        a = randn((B, N, K), 3200 + N, dtype=dt, device=DEV)
        rows = to64(a)
    w = randn((F, K), 3201, std=1.0 / math.sqrt(K), dtype=dt, device=DEV)
    y = randn((B, N, F), 3202, dtype=dt, device=DEV)
    y0 = to64(y)
    yk.yoco_linear_residual(a, w, y, a_heads=a_heads)
    torch.cuda.synchronize()
    ref = y0 + oracle.linear_rows(rows, to64(w))
    glue_check(to64(y), ref, dt, "y + a W^T")


def test_linear_residual_accumulates_in_place_twice():
    """Two residual products into the same stream add both terms."""
    B, N, K, F = 1, 65, 256, 128
    a1 = randn((B, N, K), 3301, dtype="f32", device=DEV)
    a2 = randn((B, N, K), 3302, dtype="f32", device=DEV)
    w = randn((F, K), 3303, std=1 / 16, dtype="f32", device=DEV)
    y = randn((B, N, F), 3304, dtype="f32", device=DEV)
    y0 = to64(y)
    yk.yoco_linear_residual(a1, w, y)
    yk.yoco_linear_residual(a2, w, y)
    torch.cuda.synchronize()
    ref = y0 + oracle.linear_rows(to64(a1), to64(w)) + oracle.linear_rows(to64(a2), to64(w))
    glue_check(to64(y), ref, "f32", "two residual products")


# ---------------------------------------------------------------- the whole block on the GPU
def _params(wl, with_ffn=True):
    D, Hq, Hkv, d, F = wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.ffn_dim
    idx = iter(range(1, 1000))
    dt = "f32" if wl.dtype == "f32" else "bf16"
    r = lambda *shape, std=wl.weight_std: randn(shape, seed_for(wl.wid, next(idx)), std=std, dtype=dt,  # noqa: E731
                                                device=DEV)
    ffn = lambda: (r(F, D), r(F, D), r(D, F, std=wl.weight_std * math.sqrt(D / F)))  # noqa: E731
    gp = dict(
        swa=[(r(Hq * d, D), r(Hkv * d, D), r(Hkv * d, D), r(D, Hq * d)) for _ in range(wl.n_self_layers)],
        glob=(r(Hkv * d, D), r(Hkv * d, D)),
        cross=[(r(Hq * d, D), r(D, Hq * d)) for _ in range(wl.n_cross_layers)])
    gp["swa_ffn"] = [ffn() for _ in range(wl.n_self_layers)] if with_ffn else []
    gp["cross_ffn"] = [ffn() for _ in range(wl.n_cross_layers)] if with_ffn else []
    c = lambda t: to64(t)  # noqa: E731
    p = BlockParams(
        n_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=wl.window,
        swa_wq=[c(w[0]) for w in gp["swa"]], swa_wk=[c(w[1]) for w in gp["swa"]],
        swa_wv=[c(w[2]) for w in gp["swa"]], swa_wo=[c(w[3]) for w in gp["swa"]],
        glob_wk=c(gp["glob"][0]), glob_wv=c(gp["glob"][1]),
        cross_wq=[c(w[0]) for w in gp["cross"]], cross_wo=[c(w[1]) for w in gp["cross"]],
        swa_ffn=[tuple(c(t) for t in f) for f in gp["swa_ffn"]],
        cross_ffn=[tuple(c(t) for t in f) for f in gp["cross_ffn"]])
    return gp, p


def _gpu_ffn(x, f):
    if f is not None:
        h = yk.yoco_swiglu(x, f[0], f[1])
        yk.yoco_linear_residual(h, f[2], x)


def gpu_block(x, gp, wl, early_exit=False, rope=0.0):
    """The block on the GPU, x [B, N, D] updated in place; returns (x or its
    last row after the cross layers, K, V)."""
    Hq, Hkv, d, W = wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.window
    B, N, D = x.shape
    for layer, (wq, wk, wv, wo) in enumerate(gp["swa"]):
        q, k, v = yk.yoco_qkv_proj(x, wq, d, wk, wv, rope_theta=rope)
        o = yk.yoco_swa_attn(q, k, v, W)
        yk.yoco_linear_residual(o, wo, x, a_heads=Hq)
        _gpu_ffn(x, gp["swa_ffn"][layer] if gp["swa_ffn"] else None)
    kc = torch.empty(B, Hkv, N, d, dtype=x.dtype, device=DEV)
    vc = torch.empty_like(kc)
    yk.yoco_global_kv_proj(x, gp["glob"][0], gp["glob"][1], kc, vc, rope_theta=rope)
    if early_exit:
        last = x[:, N - 1:N].contiguous()
        for layer, (wq, wo) in enumerate(gp["cross"]):
            q, _, _ = yk.yoco_qkv_proj(last, wq, d, rope_theta=rope, rope_pos0=N - 1)
            o = yk.yoco_cross_attn_decode(q.reshape(B, Hq, d).contiguous(), kc, vc, N)
            yk.yoco_linear_residual(o.reshape(B, Hq, 1, d), wo, last, a_heads=Hq)
            _gpu_ffn(last, gp["cross_ffn"][layer] if gp["cross_ffn"] else None)
        return last[:, 0], kc, vc
    for layer, (wq, wo) in enumerate(gp["cross"]):
        q, _, _ = yk.yoco_qkv_proj(x, wq, d, rope_theta=rope)
        o = yk.yoco_cross_attn_prefill(q, kc, vc)
        yk.yoco_linear_residual(o, wo, x, a_heads=Hq)
        _gpu_ffn(x, gp["cross_ffn"][layer] if gp["cross_ffn"] else None)
    return x, kc, vc


@pytest.mark.parametrize("with_ffn,rope", [(True, 0.0), (False, 0.0), (True, 640e3)])
def test_tiny_block_wholly_on_gpu_matches_oracle(with_ffn, rope):
    wl = WORKLOADS["tiny_block_f32"]
    print(f"tiny block on the GPU, ffn={with_ffn} rope={rope}", flush=True)
    gp, p = _params(wl, with_ffn)
    p.rope_theta = rope
    x = randn((wl.batch, wl.seq, wl.hidden), seed_for(wl.wid, 0), dtype="f32", device=DEV)
    x64 = to64(x)
    out, kc, vc = gpu_block(x.clone(), gp, wl, rope=rope)
    last, _, _ = gpu_block(x.clone(), gp, wl, early_exit=True, rope=rope)
    torch.cuda.synchronize()
    ref, (rk, rv) = oracle.yoco_block(x64, p)
    check(to64(kc), rk, "f32", "shared K")
    check(to64(vc), rv, "f32", "shared V")
    check(to64(out), ref, "f32", "block output")
    ref_last, _ = oracle.yoco_block_early_exit(x64, p)
    assert np.array_equal(ref_last, ref[:, -1])          # the oracle's own identity
    check(to64(last), ref_last, "f32", "early-exit last row")


def test_block_glue_at_the_3b_shape_sampled_rows():
    """The 3B-shaped layer glue in the launch configuration the benchmark times
    (D 3072, 24/8 heads of 128, N 4096, SwiGLU 8192), bf16, checked on
    sampled tokens."""
    wl = WORKLOADS["prefill_3b_bf16"]
    B, N, D, Hq, Hkv, d, F = wl.batch, wl.seq, wl.hidden, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.ffn_dim
    x = randn((B, N, D), 3400, device=DEV)
    wq = randn((Hq * d, D), 3401, std=wl.weight_std, device=DEV)
    wk = randn((Hkv * d, D), 3402, std=wl.weight_std, device=DEV)
    wv = randn((Hkv * d, D), 3403, std=wl.weight_std, device=DEV)
    wo = randn((D, Hq * d), 3404, std=wl.weight_std, device=DEV)
    wg = randn((F, D), 3405, std=wl.weight_std, device=DEV)
    wu = randn((F, D), 3406, std=wl.weight_std, device=DEV)
    wd = randn((D, F), 3407, std=wl.weight_std, device=DEV)
    q, k, v = yk.yoco_qkv_proj(x, wq, d, wk, wv)
    h = yk.yoco_swiglu(x, wg, wu)
    y1 = x.clone()
    yk.yoco_linear_residual(q, wo, y1, a_heads=Hq)
    y2 = x.clone()
    yk.yoco_linear_residual(h, wd, y2)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 2047, 3001, N - 1]
    x64 = to64(x)[:, rows]
    rq, _ = oracle.global_kv_proj(x64, to64(wq), to64(wq), Hq, d)
    rk, rv = oracle.global_kv_proj(x64, to64(wk), to64(wv), Hkv, d)
    glue_check(to64(q)[:, :, rows], rq, "bf16", "q (3B)")
    glue_check(to64(k)[:, :, rows], rk, "bf16", "k (3B)")
    glue_check(to64(v)[:, :, rows], rv, "bf16", "v (3B)")
    wg64, wu64 = to64(wg), to64(wu)
    rh = np.stack([oracle.swiglu_hidden_row(x64[0, i], wg64, wu64) for i in range(len(rows))])[None]
    glue_check(to64(h)[:, rows], rh, "bf16", "swiglu h (3B)")
    # the residual products, from the GPU's own q and h (bf16 inputs, exact in float64)
    q_rows = to64(q)[:, :, rows].transpose(0, 2, 1, 3).reshape(B, len(rows), Hq * d)
    glue_check(to64(y1)[:, rows], x64 + oracle.linear_rows(q_rows, to64(wo)), "bf16", "x + o W_o^T (3B)")
    glue_check(to64(y2)[:, rows], x64 + oracle.linear_rows(to64(h)[:, rows], to64(wd)), "bf16", "x + h W_down^T (3B)")


# ---------------------------------------------------------------- rotary embedding in the epilogues
ROPE_CASES = [
    # B, N, D, Hq, Hkv, d, theta, pos0, dtype   (token count picks the kernel form)
    (1, 77, 256, 4, 1, 64, 10000.0, 0, "f32"),          # 128 x 128 form
    (1, 300, 256, 4, 2, 128, 640e3, 5000, "bf16"),      # wide form
    (3, 5, 256, 2, 1, 128, 80e6, 1 << 20, "bf16"),      # few-token form at a 1M-token position
    (1, 64, 128, 2, 0, 64, 5e6, 123456, "bf16"),        # query only
]


@pytest.mark.parametrize("B,N,D,Hq,Hkv,d,theta,pos0,dt", ROPE_CASES)
def test_qkv_proj_rope_matches_oracle(B, N, D, Hq, Hkv, d, theta, pos0, dt):
    print(f"qkv_proj rope B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} theta={theta} pos0={pos0} {dt}", flush=True)
    s = 1.0 / math.sqrt(D)
    x = randn((B, N, D), 3500 + N, dtype=dt, device=DEV)
    wq = randn((Hq * d, D), 3501, std=s, dtype=dt, device=DEV)
    wk = randn((Hkv * d, D), 3502, std=s, dtype=dt, device=DEV) if Hkv else None
    wv = randn((Hkv * d, D), 3503, std=s, dtype=dt, device=DEV) if Hkv else None
    q, k, v = yk.yoco_qkv_proj(x, wq, d, wk, wv, rope_theta=theta, rope_pos0=pos0)
    torch.cuda.synchronize()
    rq, _ = oracle.global_kv_proj(to64(x), to64(wq), to64(wq), Hq, d)
    glue_check(to64(q), oracle.apply_rope(rq, pos0, theta), dt, "rotated q")
    if Hkv:
        rk, rv = oracle.global_kv_proj(to64(x), to64(wk), to64(wv), Hkv, d)
        glue_check(to64(k), oracle.apply_rope(rk, pos0, theta), dt, "rotated k")
        glue_check(to64(v), rv, dt, "v (never rotated)")


@pytest.mark.parametrize("B,N,dt", [(2, 300, "bf16"), (1, 77, "f32"), (16, 1, "bf16"), (2, 8200, "bf16")])
def test_global_kv_proj_rope_matches_oracle(B, N, dt):
    """Keys rotated at their cache positions pos0 + t (every kernel form),
    values untouched."""
    D, Hkv, d, theta, pos0 = 256, 2, 128, 80e6, 1000
    n_cap = pos0 + N + 3
    print(f"kv_proj rope B={B} N={N} {dt}", flush=True)
    x = randn((B, N, D), 3600 + N, dtype=dt, device=DEV)
    wk = randn((Hkv * d, D), 3601, std=0.06, dtype=dt, device=DEV)
    wv = randn((Hkv * d, D), 3602, std=0.06, dtype=dt, device=DEV)
    ko = torch.zeros(B, Hkv, n_cap, d, dtype=_tdt(dt), device=DEV)
    vo = torch.zeros_like(ko)
    yk.yoco_global_kv_proj(x, wk, wv, ko, vo, pos0=pos0, rope_theta=theta)
    torch.cuda.synchronize()
    rows = list(range(N)) if N <= 300 else [0, 1, 4095, 4096, N - 1]
    rk, rv = oracle.global_kv_proj(to64(x)[:, rows], to64(wk), to64(wv), Hkv, d)
    rk = np.stack([oracle.apply_rope(rk[:, :, i:i + 1], pos0 + r, theta)[:, :, 0] for i, r in enumerate(rows)], axis=2)
    idx = [pos0 + r for r in rows]
    glue_check(to64(ko)[:, :, idx], rk, dt, "rotated keys")
    glue_check(to64(vo)[:, :, idx], rv, dt, "values")


# ---------------------------------------------------------------- gated-retention self-decoder
def test_gret_block_on_gpu_matches_oracle_and_exits_early():
    """The block with gated-retention self-decoder layers ([S §3 Gated
    Retention], the YOCO-gRet layout): per layer the Q/K/V projection,
    yoco_gret_prefill, yoco_gret_group_norm_swish and the output projection
    (residual) with a SwiGLU feed-forward, then the global projection and the
    cross-decoder -- in bf16 on the GPU.  The gate logits and the swish gate's
    input are two small position-wise products the library has no call for;
    the test forms them with torch from the normalised layer input.
    Checked: the shared K/V and the block output against the float64 oracle,
    and the early exit (cross-decoder on the last position only, through
    decode calls) against the full forward's last row."""
    B, N, D, H, Hkv, d, F, Ls, Lc, tau = 1, 300, 256, 4, 1, 64, 512, 2, 2, 4.0
    print("gated-retention block on the GPU", flush=True)
    idx = iter(range(3500, 3600))
    # weights N(0, 0.02) as in the 3B-shaped configuration; gate logits of
    # standard deviation ~2.4 (decays from ~0.3 to ~1)
    r = lambda *shape, std=0.02: randn(shape, next(idx), std=std, device=DEV)  # noqa: E731
    gr = [dict(wq=r(H * d, D), wk=r(H * d, D), wv=r(H * d, D), wo=r(D, H * d), wz=r(H, D, std=0.15),
               wg=r(H * d, D), ffn=(r(F, D), r(F, D), r(D, F))) for _ in range(Ls)]
    glob = (r(Hkv * d, D), r(Hkv * d, D))
    cross = [dict(wq=r(H * d, D), wo=r(D, H * d), ffn=(r(F, D), r(F, D), r(D, F))) for _ in range(Lc)]
    x0 = randn((B, N, D), 3600, device=DEV)

    stages, sublayers = [], []

    def self_decoder(x):
        for L in gr:
            q, k, v = yk.yoco_qkv_proj(x, L["wq"], d, L["wk"], L["wv"])
            xf = x.float()
            n = xf * torch.rsqrt((xf * xf).mean(-1, keepdim=True) + 1e-6)
            z = (n @ L["wz"].float().t()).permute(0, 2, 1).contiguous()            # [B, H, N] float32
            g = (n @ L["wg"].float().t()).to(torch.bfloat16).contiguous()          # [B, N, H*d]
            y, _ = yk.yoco_gret_prefill(q, k, v, z, tau, state_out=False)
            gn = yk.yoco_gret_group_norm_swish(y, g)
            stages.append((q.clone(), k.clone(), v.clone(), z.clone(), g.clone(), y.clone(), gn.clone()))
            x_in = x.clone()
            yk.yoco_linear_residual(gn, L["wo"], x)
            x_mid = x.clone()
            _gpu_ffn(x, L["ffn"])
            sublayers.append((x_in, gn, L["wo"], x_mid, L["ffn"], x.clone()))
        kc = torch.empty(B, Hkv, N, d, dtype=torch.bfloat16, device=DEV)
        vc = torch.empty_like(kc)
        yk.yoco_global_kv_proj(x, glob[0], glob[1], kc, vc)
        return kc, vc

    x = x0.clone()
    kc, vc = self_decoder(x)
    last = x[:, N - 1:N].contiguous()
    cross_stages = []
    for L in cross:
        q, _, _ = yk.yoco_qkv_proj(x, L["wq"], d)
        o = yk.yoco_cross_attn_prefill(q, kc, vc)
        cross_stages.append((q.clone(), o.clone()))
        x_in = x.clone()
        yk.yoco_linear_residual(o, L["wo"], x, a_heads=H)
        x_mid = x.clone()
        _gpu_ffn(x, L["ffn"])
        merged = o.permute(0, 2, 1, 3).reshape(B, N, H * d)
        sublayers.append((x_in, merged, L["wo"], x_mid, L["ffn"], x.clone()))
    for L in cross:   # early exit: the last position alone, over the same cache
        q, _, _ = yk.yoco_qkv_proj(last, L["wq"], d)
        o = yk.yoco_cross_attn_decode(q.reshape(B, H, d).contiguous(), kc, vc, N)
        yk.yoco_linear_residual(o.reshape(B, H, 1, d), L["wo"], last, a_heads=H)
        _gpu_ffn(last, L["ffn"])
    torch.cuda.synchronize()

    c = lambda t: to64(t)  # noqa: E731
    # each gated-retention stage against the oracle fed the GPU's own inputs
    for q, k, v, z, g, y, gn in stages:
        ry, _ = oracle.gret_recurrent(c(q), c(k), c(v), c(z), tau)
        rg = oracle.gret_group_norm_swish(c(y), c(g))
        for got, want, what in ((c(y), ry, "retention"), (c(gn), rg, "group norm x swish")):
            rel = np.linalg.norm(got - want, axis=-1) / np.linalg.norm(want, axis=-1)
            assert rel.max() <= 1e-2, (what, rel.max())
    for q, o in cross_stages:
        ro, _ = oracle.cross_prefill_attention(c(q), c(kc), c(vc))
        rel = np.linalg.norm(c(o) - ro, axis=-1) / np.linalg.norm(ro, axis=-1)
        assert rel.max() <= 1e-2, ("cross attention", rel.max())
    # every residual step (output projection, then the feed-forward) of the 4
    # layers against the oracle applied to the GPU's own stream: per token
    # row, the error is at most 1e-2 of the sub-layer's own contribution plus
    # the bf16 rounding of the updated stream (2^-9 relative; 2^-8 allowed)
    for x_in, a, wo, x_mid, ffn, x_out in sublayers:
        want_mid = c(x_in) + oracle.linear_rows(c(a), c(wo))
        want_out = np.stack([oracle.swiglu_ffn_row(row, tuple(c(t) for t in ffn), 1e-6) for row in c(x_mid)[0]])[None]
        for got, want, base, what in ((c(x_mid), want_mid, c(x_in), "output projection"),
                                      (c(x_out), want_out, c(x_mid), "feed-forward")):
            nrm = lambda t: np.linalg.norm(t, axis=-1)  # noqa: E731
            excess = nrm(got - want) - (1e-2 * nrm(want - base) + 2.0 ** -8 * nrm(want))
            assert excess.max() <= 0, (what, excess.max())
    p = BlockParams(n_heads=H, n_kv_heads=Hkv, head_dim=d, window=1, self_kind="gret", gret_tau=tau,
                    swa_wq=[c(L["wq"]) for L in gr], swa_wk=[c(L["wk"]) for L in gr],
                    swa_wv=[c(L["wv"]) for L in gr], swa_wo=[c(L["wo"]) for L in gr],
                    gret_wz=[c(L["wz"]) for L in gr], gret_wg=[c(L["wg"]) for L in gr],
                    glob_wk=c(glob[0]), glob_wv=c(glob[1]),
                    cross_wq=[c(L["wq"]) for L in cross], cross_wo=[c(L["wo"]) for L in cross],
                    swa_ffn=[tuple(c(t) for t in L["ffn"]) for L in gr],
                    cross_ffn=[tuple(c(t) for t in L["ffn"]) for L in cross])
    ref, (rk, rv) = oracle.yoco_block(c(x0), p)
    ref_last, _ = oracle.yoco_block_early_exit(c(x0), p)
    assert np.array_equal(ref_last, ref[:, -1])                  # the oracle's own identity
    # The whole block end to end.  Each of its sub-layers is checked above on
    # the GPU's own inputs; end to end their bf16 rounding errors compound
    # through the residual stream (the oracle's output moves by 0.24 %
    # relative per row for a 2^-9 relative perturbation of the input alone;
    # measured on the GPU up to ~4 % on the worst token row), so this is a
    # sanity bound only: 0.15 max-abs and 5e-2 relative L2 per token row.
    for got, want, what in ((to64(kc), rk, "K"), (to64(vc), rv, "V"), (to64(x), ref, "output"),
                            (to64(last)[:, 0], ref_last, "early exit")):
        err = np.abs(got - want)
        rel = np.linalg.norm(got - want, axis=-1) / np.linalg.norm(want, axis=-1)
        assert err.max() <= 0.15 and rel.max() <= 5e-2, (what, err.max(), rel.max())
    # the early exit equals the full forward's last row to the decode-vs-prefill bf16 bound
    assert np.abs(to64(last)[:, 0] - to64(x)[:, -1]).max() <= 2e-2
