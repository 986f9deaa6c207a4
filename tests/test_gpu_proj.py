"""GPU parity of yoco_global_kv_proj against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import shared_kv_attention_amd as yk
from shared_kv_attention_amd.synth import randn
from tests._tol import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # B, N, D, Hkv, d, n_cap, pos0, gamma, dtype, wstd
    (1, 256, 256, 1, 64, 256, 0, False, "f32", 1 / 16),
    (2, 300, 256, 2, 128, 320, 5, False, "bf16", 0.06),
    (1, 129, 512, 8, 128, 200, 71, True, "bf16", 0.04),
    (3, 77, 192, 3, 64, 100, 0, True, "f32", 0.07),
    # bf16 with 16 feature tiles and >= 16 tiles of 256 tokens: the 256-token
    # form; a ragged last token tile, an odd number of k stages (5 and 3), a
    # token tile across the batch boundary (weights scaled so that outputs stay
    # O(1): the absolute bound assumes bf16 output ulps of at most 2^-6)
    (1, 4100, 320, 8, 128, 4200, 37, True, "bf16", 0.03),
    (2, 2100, 192, 8, 128, 2100, 0, False, "bf16", 0.04),
]


@pytest.mark.parametrize("B,N,D,Hkv,d,n_cap,pos0,gamma,dt,wstd", CASES)
def test_kv_proj_parity(B, N, D, Hkv, d, n_cap, pos0, gamma, dt, wstd):
    print(f"kv_proj parity B={B} N={N} D={D} Hkv={Hkv} d={d} pos0={pos0} gamma={gamma} {dt}", flush=True)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    x = randn((B, N, D), 1000, dtype=dt, device=DEV)
    wk = randn((Hkv * d, D), 1001, std=wstd, dtype=dt, device=DEV)
    wv = randn((Hkv * d, D), 1002, std=wstd, dtype=dt, device=DEV)
    g = (1 + 0.5 * randn((D,), 1003, dtype=dt, device=DEV).float()).to(tdt) if gamma else None
    ko = torch.full((B, Hkv, n_cap, d), 7.0, dtype=tdt, device=DEV)
    vo = torch.full((B, Hkv, n_cap, d), 7.0, dtype=tdt, device=DEV)
    yk.yoco_global_kv_proj(x, wk, wv, ko, vo, pos0=pos0, norm_w=g)
    torch.cuda.synchronize()
    xg = to64(x)
    rk, rv = oracle.global_kv_proj(xg, to64(wk), to64(wv), Hkv, d,
                                   gamma=None if g is None else to64(g))
    ok, ov = to64(ko), to64(vo)
    check(ok[:, :, pos0:pos0 + N], rk, dt, "K", rel_axes=(2, 3))
    check(ov[:, :, pos0:pos0 + N], rv, dt, "V", rel_axes=(2, 3))
    # rows outside [pos0, pos0 + N) are untouched
    assert np.all(ok[:, :, :pos0] == 7.0) and np.all(ok[:, :, pos0 + N:] == 7.0)
    assert np.all(ov[:, :, :pos0] == 7.0) and np.all(ov[:, :, pos0 + N:] == 7.0)


@pytest.mark.parametrize("gamma", [False, True])
def test_kv_proj_long_prompt_appended_chunk(gamma):
    """A long bf16 prompt chunk (16400 tokens: the wide-tile form) appended at
    pos0 = 50 of a larger cache: sampled rows against the oracle, every row
    outside [pos0, pos0 + N) untouched."""
    B, N, D, Hkv, d, n_cap, pos0 = 2, 8200, 256, 2, 128, 8300, 50
    print(f"kv_proj long chunk B={B} N={N} pos0={pos0} gamma={gamma}", flush=True)
    x = randn((B, N, D), 1010, device=DEV)
    wk = randn((Hkv * d, D), 1011, std=0.06, device=DEV)
    wv = randn((Hkv * d, D), 1012, std=0.06, device=DEV)
    g = (1 + 0.5 * randn((D,), 1013, device=DEV).float()).to(torch.bfloat16) if gamma else None
    ko = torch.full((B, Hkv, n_cap, d), 7.0, dtype=torch.bfloat16, device=DEV)
    vo = torch.full_like(ko, 7.0)
    yk.yoco_global_kv_proj(x, wk, wv, ko, vo, pos0=pos0, norm_w=g)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 4095, 8191, N - 1]
    rk, rv = oracle.global_kv_proj(to64(x)[:, rows], to64(wk), to64(wv), Hkv, d,
                                   gamma=None if g is None else to64(g))
    ok, ov = to64(ko), to64(vo)
    idx = [pos0 + r for r in rows]
    check(ok[:, :, idx], rk, "bf16", "K", rel_axes=(2, 3))
    check(ov[:, :, idx], rv, "bf16", "V", rel_axes=(2, 3))
    assert np.all(ok[:, :, :pos0] == 7.0) and np.all(ok[:, :, pos0 + N:] == 7.0)
    assert np.all(ov[:, :, :pos0] == 7.0) and np.all(ov[:, :, pos0 + N:] == 7.0)


# ---------------------------------------------------------------------------
# 8-bit (e4m3fn) cache written by the projection itself
# ---------------------------------------------------------------------------
def _proj_inputs(B, N, D, Hkv, d, gamma, dt, seed):
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    x = randn((B, N, D), seed, dtype=dt, device=DEV)
    wk = randn((Hkv * d, D), seed + 1, std=0.05, dtype=dt, device=DEV)
    wv = randn((Hkv * d, D), seed + 2, std=0.05, dtype=dt, device=DEV)
    g = (1 + 0.5 * randn((D,), seed + 3, dtype=dt, device=DEV).float()).to(tdt) if gamma else None
    return x, wk, wv, g, tdt


FP8_CASES = [
    # B, N, D, Hkv, d, n_cap, gamma, dtype, rope_theta, sampled rows (None: all)
    (2, 300, 256, 2, 128, 320, False, "bf16", 0.0, None),      # 128 x 128 kernel, maxima in its epilogue
    (1, 40, 256, 2, 64, 64, True, "bf16", 0.0, None),           # a few tokens: block GEMM form + maxima pass
    (3, 77, 192, 3, 64, 100, True, "f32", 1e4, None),
    (1, 1, 256, 2, 128, 8, False, "bf16", 1e4, None),            # one-token prompt
    (1, 16400, 256, 2, 128, 16500, False, "bf16", 1e4, [0, 1, 127, 128, 8191, 16399]),   # wide form
    (1, 4096, 3072, 8, 128, 4096, False, "bf16", 0.0, [0, 1, 2047, 4095]),              # the 3B shape
]


@pytest.mark.parametrize("B,N,D,Hkv,d,n_cap,gamma,dt,rope,rows", FP8_CASES)
def test_kv_proj_fp8_cache_sets_scales(B, N, D, Hkv, d, n_cap, gamma, dt, rope, rows):
    """Codes and scales equal, bit for bit, the oracle's quantiser applied to
    the activation-dtype projection of the same rows; rows past N untouched."""
    print(f"kv_proj fp8 B={B} N={N} D={D} Hkv={Hkv} d={d} gamma={gamma} {dt} rope={rope}", flush=True)
    x, wk, wv, g, tdt = _proj_inputs(B, N, D, Hkv, d, gamma, dt, 1020)
    kr = torch.full((B, Hkv, n_cap, d), 7.0, dtype=tdt, device=DEV)
    vr = torch.full_like(kr, 7.0)
    yk.yoco_global_kv_proj(x, wk, wv, kr, vr, norm_w=g, rope_theta=rope)
    kc = torch.full((B, Hkv, n_cap, d), 0x55, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0x55)
    ks = torch.full((Hkv,), float("nan"), device=DEV)
    vs = torch.full((Hkv,), float("nan"), device=DEV)
    yk.yoco_global_kv_proj(x, wk, wv, kc, vc, norm_w=g, rope_theta=rope, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    for name, ref, codes, sc in (("K", kr, kc, ks), ("V", vr, vc, vs)):
        ref64 = to64(ref)[:, :, :N]
        want_s = oracle.kv_fp8_scales(ref64)
        assert np.array_equal(sc.cpu().numpy(), want_s), name
        sel = slice(None) if rows is None else rows
        want = oracle.encode_kv_fp8(ref64[:, :, sel], want_s)
        assert np.array_equal(codes.cpu().numpy()[:, :, :N][:, :, sel], want), f"{name} codes"
        assert bool((codes[:, :, N:] == 0x55).all()), f"{name}: rows past N touched"
    # the decoded cache is the oracle's float64 projection up to the 8-bit
    # rounding (half a step: 2^-4 relative, 2^-10 s among the subnormals) and
    # the activation dtype's own max-abs tolerance
    if rows is None:
        rk, rv = oracle.global_kv_proj(to64(x), to64(wk), to64(wv), Hkv, d, gamma=None if g is None else to64(g))
        if rope:
            rk = oracle.apply_rope(rk, 0, rope)
        for ref, codes, sc in ((rk, kc, ks), (rv, vc, vs)):
            deq = oracle.dequantize_kv_fp8(codes.cpu().numpy()[:, :, :N], sc.cpu().numpy())
            step = np.abs(ref) * 2.0 ** -4 + sc.cpu().numpy()[None, :, None, None] * 2.0 ** -10
            assert np.all(np.abs(deq - ref) <= step + (1e-5 if dt == "f32" else 2e-2))


@pytest.mark.parametrize("N0,N1,dt,rope", [(200, 1, "bf16", 1e4), (200, 100, "bf16", 0.0), (90, 7, "f32", 1e4)])
def test_kv_proj_fp8_append_uses_the_set_scales(N0, N1, dt, rope):
    """A prompt of N0 rows sets the scales; N1 rows appended at pos0 = N0 are
    encoded with those scales (not changed), bit for bit as the oracle encodes
    the activation-dtype projection of the appended rows."""
    B, D, Hkv, d, n_cap = 2, 256, 2, 128, 320
    print(f"kv_proj fp8 append N0={N0} N1={N1} {dt} rope={rope}", flush=True)
    x, wk, wv, g, tdt = _proj_inputs(B, N0 + N1, D, Hkv, d, False, dt, 1030)
    x0, x1 = x[:, :N0].contiguous(), x[:, N0:].contiguous()
    kc = torch.full((B, Hkv, n_cap, d), 0x55, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0x55)
    _, _, ks, vs = yk.yoco_global_kv_proj(x0, wk, wv, kc, vc, rope_theta=rope)
    ks0, vs0 = ks.clone(), vs.clone()
    kr = torch.zeros((B, Hkv, n_cap, d), dtype=tdt, device=DEV)
    vr = torch.zeros_like(kr)
    yk.yoco_global_kv_proj(x1, wk, wv, kr, vr, pos0=N0, rope_theta=rope)
    yk.yoco_global_kv_proj(x1, wk, wv, kc, vc, pos0=N0, rope_theta=rope, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert torch.equal(ks, ks0) and torch.equal(vs, vs0)
    for ref, codes, sc in ((kr, kc, ks), (vr, vc, vs)):
        want = oracle.encode_kv_fp8(to64(ref)[:, :, N0:N0 + N1], sc.cpu().numpy())
        assert np.array_equal(codes.cpu().numpy()[:, :, N0:N0 + N1], want)
        assert bool((codes[:, :, N0 + N1:] == 0x55).all())


def test_decode_over_a_cache_the_projection_wrote_in_8_bits():
    """yoco_cross_attn_decode over the projection's 8-bit cache equals the
    oracle's decode over the dequantised values (bf16 tolerances)."""
    B, N, D, Hkv, Hq, d = 2, 3000, 512, 4, 16, 128
    x, wk, wv, _, _ = _proj_inputs(B, N, D, Hkv, d, False, "bf16", 1040)
    kc = torch.empty((B, Hkv, N, d), dtype=torch.uint8, device=DEV)
    vc = torch.empty_like(kc)
    _, _, ks, vs = yk.yoco_global_kv_proj(x, wk, wv, kc, vc)
    q = randn((B, Hq, d), 1045, device=DEV)
    o = yk.yoco_cross_attn_decode(q, kc, vc, N, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    kd = oracle.dequantize_kv_fp8(kc.cpu().numpy(), ks.cpu().numpy())
    vd = oracle.dequantize_kv_fp8(vc.cpu().numpy(), vs.cpu().numpy())
    ro, _ = oracle.decode_attention(to64(q), kd, vd, [N] * B)
    check(to64(o), ro, "bf16", "decode over the projected 8-bit cache", rel_axes=(2,))


@pytest.mark.parametrize("B,N,D,pos0,rope", [(1, 4096, 3072, 0, 0.0), (2, 2100, 192, 3, 1e4), (1, 4100, 256, 0, 0.0),
                                             (3, 1400, 320, 9, 1e4), (1, 4096, 64, 0, 0.0), (2, 2048, 128, 1, 1e4),
                                             (1, 10000, 256, 0, 0.0)])
def test_kv_proj_ring_form_equals_staging_form(B, N, D, pos0, rope):
    """bf16 without a norm gain runs the three-stage ring form when its grid (256 features x 128 tokens per
    workgroup) covers the chip; with a gain of ones the 128 x 128 staging form runs on the same values.  The two
    forms sum every product and every square in the same order: outputs bitwise equal.  D / 64 = 48, 3, 4, 5 k
    stages cover every remainder of the ring's three buffers; ragged token tiles and tiles across the batch
    boundary included; one and two k stages (D = 64, 128) and a grid of several rounds (10000 tokens)."""
    Hkv, d = 8, 128
    n_cap = pos0 + N + 5
    print(f"kv_proj ring vs staging B={B} N={N} D={D} pos0={pos0} rope={rope}", flush=True)
    x = randn((B, N, D), 1100 + D, device=DEV)
    wk = randn((Hkv * d, D), 1101 + D, std=D ** -0.5, device=DEV)
    wv = randn((Hkv * d, D), 1102 + D, std=D ** -0.5, device=DEV)
    ones = torch.ones(D, dtype=torch.bfloat16, device=DEV)
    outs = []
    for g in (None, ones):
        ko = torch.full((B, Hkv, n_cap, d), 7.0, dtype=torch.bfloat16, device=DEV)
        vo = torch.full_like(ko, 7.0)
        yk.yoco_global_kv_proj(x, wk, wv, ko, vo, pos0=pos0, norm_w=g, rope_theta=rope)
        outs.append((ko, vo))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    rows = [0, 1, 127, 128, N - 1]
    rk, rv = oracle.global_kv_proj(to64(x)[:, rows], to64(wk), to64(wv), Hkv, d)
    if rope:
        # keys rotated at their cache positions
        rk = np.concatenate([oracle.apply_rope(rk[:, :, i:i + 1], pos0 + r, rope) for i, r in enumerate(rows)], axis=2)
    idx = [pos0 + r for r in rows]
    check(to64(outs[0][0])[:, :, idx], rk, "bf16", "K", rel_axes=(2, 3))
    check(to64(outs[0][1])[:, :, idx], rv, "bf16", "V", rel_axes=(2, 3))
    assert torch.all(outs[0][0][:, :, :pos0] == 7.0) and torch.all(outs[0][0][:, :, pos0 + N:] == 7.0)
