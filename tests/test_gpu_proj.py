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
