"""C-ABI checks that need no GPU.

* libyoco.so loads and exports every function include/yoco.h declares;
* every status code is reachable: argument validation runs before any HIP
  call, so each single-fault call below returns its error without touching
  a device (no compute is launched here);
* workspace queries are consistent.
"""
import ctypes
import os
import re

import pytest

import shared_kv_attention_amd as yk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "yoco.h")

OK, NULL, SHAPE, DTYPE, UNSUP, ALIGN, WS, HIP = range(8)
P = 4096          # an aligned, never-dereferenced fake device address
MIS = 4096 + 4    # misaligned


@pytest.fixture(scope="module")
def L():
    return yk.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(yoco_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert yk.yoco_version() == 100
    seen = set()
    for s in range(8):
        msg = yk.yoco_status_string(s)
        assert msg and msg not in seen
        seen.add(msg)
    assert yk.yoco_status_string(99) == "unknown status"


def proj(L, **kw):
    a = dict(x=P, g=None, wk=P, wv=P, ko=P, vo=P, ks=None, vs=None, B=1, N=8, D=128, Hkv=2, d=64, n_cap=16, pos0=0,
             eps=1e-6, rope=0.0, dt=yk.BF16, kvdt=None, ws=None, ws_bytes=0)
    a.update(kw)
    kvdt = a["dt"] if a["kvdt"] is None else a["kvdt"]
    return L.yoco_global_kv_proj(a["x"], a["g"], a["wk"], a["wv"], a["ko"], a["vo"], a["ks"], a["vs"], a["B"], a["N"],
                                 a["D"], a["Hkv"], a["d"], a["n_cap"], a["pos0"], a["eps"], a["rope"], a["dt"], kvdt,
                                 a["ws"], a["ws_bytes"], None)


FP8 = dict(kvdt=yk.FP8_E4M3, ks=P, vs=P, ws=P, ws_bytes=1 << 20)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(wv=None), NULL), (dict(vo=None), NULL),
    (dict(dt=yk.FP8_E4M3, kvdt=yk.BF16), DTYPE), (dict(dt=7, kvdt=yk.BF16), DTYPE),
    # an 8-bit cache: scales required; its workspace only when the call sets the scales (pos0 == 0)
    (dict(FP8, ks=None), NULL), (dict(FP8, vs=None), NULL),
    (dict(FP8, ws=None), WS), (dict(FP8, ws_bytes=16), WS), (dict(FP8, ws=MIS), ALIGN), (dict(FP8, ks=P + 2), ALIGN),
    (dict(FP8, dt=yk.FP8_E4M3), DTYPE), (dict(kvdt=yk.F32), DTYPE), (dict(dt=yk.F32, kvdt=yk.BF16), DTYPE),
    (dict(FP8, N=0), SHAPE), (dict(FP8, d=96), UNSUP),
    (dict(N=0), SHAPE), (dict(pos0=-1), SHAPE), (dict(pos0=9), SHAPE), (dict(n_cap=7), SHAPE),
    (dict(eps=float("nan")), SHAPE), (dict(eps=-1.0), SHAPE), (dict(Hkv=0), SHAPE),
    (dict(rope=-1.0), SHAPE), (dict(rope=float("nan")), SHAPE), (dict(rope=float("inf")), SHAPE),
    (dict(d=96), UNSUP), (dict(D=100), UNSUP),
    (dict(x=MIS), ALIGN), (dict(g=MIS), ALIGN), (dict(ko=MIS), ALIGN),
])
def test_global_kv_proj_errors(L, kw, code):
    assert proj(L, **kw) == code


def test_global_kv_proj_workspace_query():
    B, N, Hkv, d = 2, 300, 4, 128
    assert yk.yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, yk.BF16, yk.BF16) == 0
    assert yk.yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, yk.F32, yk.F32) == 0
    # per-head maxima (2 Hkv words, one 16-byte line here), then K and V staged in the activation dtype
    assert yk.yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, yk.BF16, yk.FP8_E4M3) == 32 + 2 * B * Hkv * N * d * 2
    assert yk.yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, yk.F32, yk.FP8_E4M3) == 32 + 2 * B * Hkv * N * d * 4
    assert yk.yoco_global_kv_proj_workspace_bytes(B, N, Hkv, 96, yk.BF16, yk.FP8_E4M3) == 0
    assert yk.yoco_global_kv_proj_workspace_bytes(0, N, Hkv, d, yk.BF16, yk.FP8_E4M3) == 0


def swa(L, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=2, N=64, d=128, W=16, scale=0.0, dt=yk.BF16)
    a.update(kw)
    return L.yoco_swa_attn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"],
                           a["W"], a["scale"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(o=None), NULL),
    (dict(dt=yk.FP8_E4M3), DTYPE),
    (dict(Hq=6, Hkv=4), SHAPE), (dict(W=0), SHAPE), (dict(N=0), SHAPE), (dict(B=0), SHAPE),
    (dict(scale=float("inf")), SHAPE),
    (dict(d=32), UNSUP), (dict(d=256), UNSUP),
    (dict(v=MIS), ALIGN), (dict(lse=4096 + 2), ALIGN),
])
def test_swa_errors(L, kw, code):
    assert swa(L, **kw) == code


def prefill(L, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Nq=8, n_kv=32, n_cap=40, off=24, d=64, scale=0.0,
             dt=yk.F32)
    a.update(kw)
    return L.yoco_cross_attn_prefill(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                     a["Nq"], a["n_kv"], a["n_cap"], a["off"], a["d"], a["scale"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), NULL), (dict(dt=5), DTYPE),
    (dict(off=25), SHAPE), (dict(off=-1), SHAPE), (dict(n_kv=41), SHAPE), (dict(n_cap=0), SHAPE),
    (dict(Nq=0), SHAPE), (dict(d=100), UNSUP), (dict(q=MIS), ALIGN),
])
def test_cross_prefill_errors(L, kw, code):
    assert prefill(L, **kw) == code


def decode(L, **kw):
    a = dict(q=P, k=P, v=P, ks=None, vs=None, cl=None, ctx=100, o=P, lse=None, B=2, Hq=8, Hkv=2, n_cap=128, d=128,
             scale=0.0, qdt=yk.BF16, kvdt=yk.BF16, ws=P, wsb=1 << 30)
    a.update(kw)
    return L.yoco_cross_attn_decode(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["cl"], a["ctx"], a["o"], a["lse"],
                                    a["B"], a["Hq"], a["Hkv"], a["n_cap"], a["d"], a["scale"], a["qdt"], a["kvdt"],
                                    a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(v=None), NULL), (dict(kvdt=yk.FP8_E4M3), NULL),
    (dict(kvdt=yk.FP8_E4M3, ks=P), NULL),
    (dict(qdt=yk.F32), DTYPE), (dict(qdt=yk.FP8_E4M3, kvdt=yk.FP8_E4M3, ks=P, vs=P), DTYPE),
    (dict(qdt=yk.F32, kvdt=yk.FP8_E4M3, ks=P, vs=P), DTYPE),
    (dict(ctx=0), SHAPE), (dict(ctx=129), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(B=0), SHAPE),
    (dict(scale=float("nan")), SHAPE),
    (dict(d=80), UNSUP),
    (dict(o=MIS), ALIGN), (dict(cl=4096 + 2), ALIGN), (dict(ws=MIS), ALIGN),
    (dict(ws=None), WS), (dict(wsb=16), WS),
])
def test_decode_errors(L, kw, code):
    assert decode(L, **kw) == code


def test_decode_workspace_query():
    need = yk.yoco_cross_attn_decode_workspace_bytes(2, 8, 2, 100, 128)
    assert need > 0 and need % 16 == 0
    big = yk.yoco_cross_attn_decode_workspace_bytes(16, 32, 8, 32768, 128)
    assert big > need
    # at least one partial (d + 2 floats) per (b, q-head)
    assert big >= 16 * 32 * 130 * 4
    for bad in [(0, 8, 2, 100, 128), (2, 6, 4, 100, 128), (2, 8, 2, 0, 128), (2, 8, 2, 100, 96)]:
        assert yk.yoco_cross_attn_decode_workspace_bytes(*bad) == 0


def test_decode_exact_workspace_boundary(L):
    need = yk.yoco_cross_attn_decode_workspace_bytes(2, 8, 2, 100, 128)
    assert decode(L, wsb=need - 1) == WS


def swa_dec(L, **kw):
    a = dict(q=P, kn=P, vn=P, kr=P, vr=P, pos=300, o=P, lse=None, B=2, Hq=8, Hkv=2, W=256, d=128,
             scale=0.0, dt=yk.BF16, ws=P, wsb=1 << 30)
    a.update(kw)
    return L.yoco_swa_decode(a["q"], a["kn"], a["vn"], a["kr"], a["vr"], a["pos"], a["o"], a["lse"], a["B"],
                             a["Hq"], a["Hkv"], a["W"], a["d"], a["scale"], a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(kr=None), NULL), (dict(o=None), NULL), (dict(kn=None), NULL), (dict(vn=None), NULL),
    (dict(dt=yk.FP8_E4M3), DTYPE), (dict(dt=7), DTYPE),
    (dict(pos=-1), SHAPE), (dict(W=0), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(B=0), SHAPE),
    (dict(scale=float("inf")), SHAPE),
    (dict(d=32), UNSUP),
    (dict(kn=MIS), ALIGN), (dict(vr=MIS), ALIGN), (dict(lse=4096 + 2), ALIGN), (dict(ws=MIS), ALIGN),
    (dict(ws=None), WS), (dict(wsb=16), WS),
])
def test_swa_decode_errors(L, kw, code):
    assert swa_dec(L, **kw) == code


def test_swa_decode_workspace_covers_every_position(L):
    need = yk.yoco_swa_decode_workspace_bytes(2, 8, 2, 256, 128)
    assert need > 0 and need % 16 == 0
    # positions before the ring fills plan on fewer keys: never more than the bound
    for pos in range(0, 600, 7):
        assert yk.yoco_cross_attn_decode_workspace_bytes(2, 8, 2, min(pos + 1, 256), 128) <= need
    for bad in [(0, 8, 2, 256, 128), (2, 8, 2, 0, 128), (2, 8, 2, 256, 100)]:
        assert yk.yoco_swa_decode_workspace_bytes(*bad) == 0


def gret(L, **kw):
    a = dict(q=P, k=P, v=P, z=P, tau=4.0, s_in=None, o=P, s_out=None, B=1, H=2, N=300, d=128, chunk=256,
             dt=yk.BF16, ws=P, wsb=1 << 30)
    a.update(kw)
    return L.yoco_gret_prefill(a["q"], a["k"], a["v"], a["z"], a["tau"], a["s_in"], a["o"], a["s_out"], a["B"], a["H"],
                               a["N"], a["d"], a["chunk"], a["dt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(z=None), NULL), (dict(o=None), NULL),
    (dict(dt=yk.F32), DTYPE), (dict(dt=yk.FP8_E4M3), DTYPE),
    (dict(N=0), SHAPE), (dict(tau=0.0), SHAPE), (dict(tau=-1.0), SHAPE), (dict(tau=float("nan")), SHAPE),
    (dict(d=96), UNSUP), (dict(chunk=64), UNSUP), (dict(chunk=512), UNSUP),
    (dict(k=MIS), ALIGN), (dict(s_out=4096 + 2), ALIGN), (dict(ws=MIS), ALIGN),
    (dict(ws=None), WS), (dict(wsb=16), WS),
])
def test_gret_prefill_errors(L, kw, code):
    assert gret(L, **kw) == code


def test_gret_workspace_query(L):
    need = yk.yoco_gret_prefill_workspace_bytes(1, 2, 300, 128, 256)
    assert need >= 2 * 300 * 4 + 2 * 2 * 128 * 128 * 6 and need % 16 == 0
    assert gret(L, wsb=need - 1) == WS
    for bad in [(0, 2, 300, 128, 256), (1, 2, 0, 128, 256), (1, 2, 300, 32, 256), (1, 2, 300, 128, 100)]:
        assert yk.yoco_gret_prefill_workspace_bytes(*bad) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(state=None), NULL), (dict(dt=yk.FP8_E4M3), DTYPE), (dict(B=0), SHAPE),
    (dict(tau=0.0), SHAPE), (dict(d=32), UNSUP), (dict(state=4096 + 2), ALIGN),
])
def test_gret_decode_errors(L, kw, code):
    a = dict(q=P, k=P, v=P, z=P, tau=4.0, state=P, o=P, B=2, H=3, d=128, dt=yk.BF16)
    a.update(kw)
    assert L.yoco_gret_decode(a["q"], a["k"], a["v"], a["z"], a["tau"], a["state"], a["o"], a["B"], a["H"], a["d"],
                              a["dt"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(y=None), NULL), (dict(dt=yk.FP8_E4M3), DTYPE), (dict(N=0), SHAPE), (dict(eps=-1.0), SHAPE),
    (dict(d=100), UNSUP), (dict(out=4096 + 1), ALIGN),
])
def test_gret_norm_errors(L, kw, code):
    a = dict(y=P, g=P, out=P, B=2, H=3, N=5, d=64, eps=1e-6, dt=yk.F32)
    a.update(kw)
    assert L.yoco_gret_group_norm_swish(a["y"], a["g"], a["out"], a["B"], a["H"], a["N"], a["d"], a["eps"], a["dt"],
                                        None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(wq=None), NULL), (dict(qo=None), NULL), (dict(wk=None), NULL), (dict(vo=None), NULL),
    (dict(dt=yk.FP8_E4M3), DTYPE), (dict(B=0), SHAPE), (dict(N=0), SHAPE), (dict(Hq=0), SHAPE), (dict(Hkv=-1), SHAPE),
    (dict(eps=float("inf")), SHAPE), (dict(rope=-2.0), SHAPE), (dict(rpos=-1), SHAPE),
    (dict(rpos=2 ** 31 - 5), SHAPE), (dict(d=32), UNSUP), (dict(D=96), UNSUP), (dict(D=65600), UNSUP),
    (dict(x=MIS), ALIGN), (dict(g=MIS), ALIGN), (dict(ko=MIS), ALIGN),
    # a q-only (cross layer) call ignores the k/v pointers
    (dict(Hkv=0, wk=None, wv=None, ko=None, vo=None, x=MIS), ALIGN),
])
def test_qkv_proj_errors(L, kw, code):
    a = dict(x=P, g=None, wq=P, wk=P, wv=P, qo=P, ko=P, vo=P, B=1, N=8, D=128, Hq=4, Hkv=2, d=64, eps=1e-6,
             rope=0.0, rpos=0, dt=yk.BF16)
    a.update(kw)
    assert L.yoco_qkv_proj(a["x"], a["g"], a["wq"], a["wk"], a["wv"], a["qo"], a["ko"], a["vo"], a["B"], a["N"],
                           a["D"], a["Hq"], a["Hkv"], a["d"], a["eps"], a["rope"], a["rpos"], a["dt"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(wu=None), NULL), (dict(h=None), NULL), (dict(dt=yk.FP8_E4M3), DTYPE),
    (dict(N=0), SHAPE), (dict(F=0), SHAPE), (dict(F=66), SHAPE), (dict(eps=-1.0), SHAPE),
    (dict(D=100), UNSUP), (dict(h=MIS), ALIGN), (dict(wg=MIS), ALIGN),
])
def test_swiglu_errors(L, kw, code):
    a = dict(x=P, g=None, wg=P, wu=P, h=P, B=2, N=8, D=128, F=344, eps=1e-6, dt=yk.F32)
    a.update(kw)
    assert L.yoco_swiglu(a["x"], a["g"], a["wg"], a["wu"], a["h"], a["B"], a["N"], a["D"], a["F"], a["eps"], a["dt"],
                         None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(a=None), NULL), (dict(y=None), NULL), (dict(dt=7), DTYPE), (dict(B=0), SHAPE), (dict(F=6), SHAPE),
    (dict(heads=-1), SHAPE), (dict(heads=3), SHAPE), (dict(K=96), UNSUP), (dict(heads=8), UNSUP),
    (dict(y=MIS), ALIGN), (dict(w=MIS), ALIGN),
])
def test_linear_residual_errors(L, kw, code):
    a = dict(a=P, heads=2, w=P, y=P, B=1, N=16, K=256, F=128, dt=yk.BF16)
    a.update(kw)
    assert L.yoco_linear_residual(a["a"], a["heads"], a["w"], a["y"], a["B"], a["N"], a["K"], a["F"], a["dt"],
                                  None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(dt=yk.FP8_E4M3), DTYPE), (dict(Nq=0), SHAPE), (dict(Nq=301), SHAPE),
    (dict(W=0), SHAPE), (dict(d=32), UNSUP), (dict(k=MIS), ALIGN),
])
def test_swa_attn_halo_errors(L, kw, code):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=8, Hkv=2, Nq=200, Nkv=300, d=128, W=64, dt=yk.BF16)
    a.update(kw)
    assert L.yoco_swa_attn_halo(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                                a["Nkv"], a["d"], a["W"], 0.0, a["dt"], None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(op=None), NULL), (dict(lp=None), NULL), (dict(o=None), NULL), (dict(dt=yk.FP8_E4M3), DTYPE),
    (dict(S=0), SHAPE), (dict(rows=0), SHAPE), (dict(d=96), UNSUP), (dict(o=MIS), ALIGN), (dict(lse=4096 + 2), ALIGN),
])
def test_attn_merge_errors(L, kw, code):
    a = dict(op=P, lp=P, o=P, lse=None, S=4, rows=64, d=128, dt=yk.BF16)
    a.update(kw)
    assert L.yoco_attn_merge(a["op"], a["lp"], a["o"], a["lse"], a["S"], a["rows"], a["d"], a["dt"], None) == code


def test_peak_microbenchmark_errors(L):
    assert L.yoco_peak_hbm_read(None, 1024, P, 8, None) == NULL
    assert L.yoco_peak_hbm_read(P, 1000, P, 8, None) == SHAPE
    assert L.yoco_peak_hbm_read(P, 1024, P, 0, None) == SHAPE
    assert L.yoco_peak_hbm_read(MIS, 1024, P, 8, None) == ALIGN
    assert L.yoco_peak_mfma_bf16(10, None, 8, None) == NULL
    assert L.yoco_peak_mfma_bf16(0, P, 8, None) == SHAPE
    assert L.yoco_peak_mfma_bf16((1 << 20) + 1, P, 8, None) == SHAPE
    assert L.yoco_peak_mfma_bf16(10, P, 70000, None) == SHAPE
    assert L.yoco_peak_mfma_bf16_toggling(16, None, 8, None) == NULL
    assert L.yoco_peak_mfma_bf16_toggling(12, P, 8, None) == SHAPE
    assert L.yoco_peak_mfma_bf16_toggling(0, P, 8, None) == SHAPE
    assert L.yoco_peak_mfma_bf16_toggling(1 << 21, P, 8, None) == SHAPE
    assert L.yoco_peak_mfma_bf16_toggling(16, P, 0, None) == SHAPE
    assert L.yoco_peak_mfma_bf16_toggling(16, P + 1, 8, None) == ALIGN


def quant(L, **kw):
    a = dict(kv=P, dt=yk.F32, codes=P, scale=P, B=2, Hkv=4, n=10, d=64, ws=P, wsb=64)
    a.update(kw)
    return L.yoco_kv_quantize_fp8(a["kv"], a["dt"], a["codes"], a["scale"], a["B"], a["Hkv"], a["n"], a["d"],
                                  a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kv=None), NULL), (dict(scale=None), NULL), (dict(dt=yk.FP8_E4M3), DTYPE),
    (dict(n=0), SHAPE), (dict(Hkv=0), SHAPE), (dict(d=48), UNSUP), (dict(codes=MIS), ALIGN),
    (dict(ws=None), WS), (dict(wsb=15), WS),
])
def test_quantize_errors(L, kw, code):
    assert quant(L, **kw) == code


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(yk, "library_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(yk, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        yk.lib()
