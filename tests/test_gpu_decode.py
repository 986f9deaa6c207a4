"""GPU parity of yoco_cross_attn_decode (bf16, f32, fp8-e4m3 caches) and of the
fp8 cache writer yoco_kv_quantize_fp8 against the oracle."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import shared_kv_attention_amd as yk
from shared_kv_attention_amd.synth import randn
from tests._tol import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


DECODE_CASES = [
    # B, Hq, Hkv, n_cap, ctx, ctx_lens, d, dtype
    (1, 4, 1, 256, 256, None, 64, "f32"),
    (3, 8, 2, 1000, 1000, [1000, 1, 517], 128, "bf16"),
    (2, 24, 8, 4096, 4096, None, 128, "bf16"),
    (2, 6, 2, 700, 650, [650, 333], 64, "bf16"),
    (2, 12, 2, 300, 300, None, 128, "bf16"),      # 6 query heads per KV head: two head groups
    (1, 4, 4, 5000, 4999, None, 128, "f32"),
    # splits of 1024 keys: the whole-line K form, with ragged lengths (rows past
    # each length hold NaN and must never be read)
    (32, 32, 8, 16384, 16384, [16384, 1, 16383, 1024, 1025, 2047, 5000, 16000] * 4, 128, "bf16"),
    # 64-key splits over many (sequence, KV head) pairs with ragged lengths that
    # leave some splits empty; two head groups at head dim 64; 256-key splits
    (16, 32, 8, 1024, 1024, [1024, 1, 63, 64, 65, 1000, 512, 1023] * 2, 128, "bf16"),
    (8, 64, 8, 300, 300, None, 64, "bf16"),
    (64, 32, 8, 2048, 2048, None, 128, "bf16"),
]


@pytest.mark.parametrize("B,Hq,Hkv,n_cap,ctx,ctx_lens,d,dt", DECODE_CASES)
def test_decode_parity(B, Hq, Hkv, n_cap, ctx, ctx_lens, d, dt):
    print(f"decode parity B={B} Hq={Hq} Hkv={Hkv} n_cap={n_cap} ctx={ctx} lens={ctx_lens} d={d} {dt}", flush=True)
    q = randn((B, Hq, d), 900, dtype=dt, device=DEV)
    k = randn((B, Hkv, n_cap, d), 901, dtype=dt, device=DEV)
    v = randn((B, Hkv, n_cap, d), 902, dtype=dt, device=DEV)
    lens = [ctx] * B if ctx_lens is None else ctx_lens
    for b in range(B):   # rows >= ctx_b must never be read
        k[b, :, lens[b]:] = float("nan")
        v[b, :, lens[b]:] = float("nan")
    cl = None if ctx_lens is None else torch.tensor(ctx_lens, dtype=torch.int32, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    o = yk.yoco_cross_attn_decode(q, k, v, ctx, ctx_lens=cl, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_attention(to64(q), to64(k), to64(v), lens)
    check(to64(o), ro, dt, "decode O", rel_axes=(2,))
    assert np.abs(to64(lse) - rl).max() <= (1e-5 if dt == "f32" else 1e-3)


def test_decode_planted_key_at_split_boundaries():
    B, Hq, Hkv, n, d = 1, 4, 1, 20000, 128
    q = randn((B, Hq, d), 910, device=DEV)
    k = randn((B, Hkv, n, d), 911, device=DEV)
    v = randn((B, Hkv, n, d), 912, device=DEV)
    for s in (0, 255, 256, 10000, n - 1):
        k2 = k.clone()
        k2[0, 0, s] = (q[0].float().mean(0) * 30).to(torch.bfloat16)
        o = yk.yoco_cross_attn_decode(q, k2, v, n)
        torch.cuda.synchronize()
        ro, _ = oracle.decode_attention(to64(q), to64(k2), to64(v), [n])
        check(to64(o), ro, "bf16", f"planted key at {s}", rel_axes=(2,))


def test_decode_matches_prefill_last_row():
    """Early exit: the last prompt position through decode == through prefill."""
    B, Hq, Hkv, N, d = 2, 8, 2, 777, 128
    q = randn((B, Hq, N, d), 920, device=DEV)
    k = randn((B, Hkv, N, d), 921, device=DEV)
    v = randn((B, Hkv, N, d), 922, device=DEV)
    op = yk.yoco_cross_attn_prefill(q, k, v)
    od = yk.yoco_cross_attn_decode(q[:, :, -1].contiguous(), k, v, N)
    torch.cuda.synchronize()
    ro, _ = oracle.decode_attention(to64(q)[:, :, -1], to64(k), to64(v), [N] * B)
    check(to64(od), ro, "bf16", "decode last row", rel_axes=(2,))
    check(to64(op)[:, :, -1], ro, "bf16", "prefill last row", rel_axes=(2,))


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quantize_fp8_bit_exact(src):
    B, Hkv, n, d = 2, 4, 333, 128
    kv = randn((B, Hkv, n, d), 930, dtype=src, device=DEV)
    kv[:, 1] *= 37.0
    kv[:, 2] = 0
    kv[:, 3] *= 1e-3
    codes, scale = yk.yoco_kv_quantize_fp8(kv)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_kv_fp8(kv.float().cpu().numpy())
    assert np.array_equal(scale.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("B,Hq,Hkv,n,lens,d", [
    (2, 8, 2, 3000, [3000, 1234], 128),
    # 32 sequences of ragged length over a 16384-row cache (splits of 1024 keys)
    (32, 32, 8, 16384, [16384, 1, 16383, 1024, 1025, 2047, 5000, 16000] * 4, 128),
    # head dim 64 (one code byte per lane and key in P V) and 1, 3, 6 query heads per KV head
    (2, 8, 2, 3000, [3000, 777], 64),
    (3, 4, 4, 2500, [2500, 1, 1999], 64),        # 1 query head per KV head
    (2, 6, 2, 4100, [4100, 4099], 128),          # 3 per KV head
    (2, 12, 2, 1500, [1500, 65], 64),            # 6 per KV head: two head groups, the second of 2
    # 16 splits of 64 keys over 128 (sequence, KV head) pairs, some empty
    (16, 32, 8, 1024, [1024, 3, 64, 65, 1000, 1, 512, 1023] * 2, 128),
])
def test_decode_fp8_parity(B, Hq, Hkv, n, lens, d):
    print(f"fp8 decode parity B={B} Hq={Hq} Hkv={Hkv} n={n} d={d}", flush=True)
    q = randn((B, Hq, d), 940, device=DEV)
    kf = randn((B, Hkv, n, d), 941, dtype="f32", device=DEV)
    vf = randn((B, Hkv, n, d), 942, dtype="f32", device=DEV)
    kc, ks = yk.yoco_kv_quantize_fp8(kf)
    vc, vs = yk.yoco_kv_quantize_fp8(vf)
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = yk.yoco_cross_attn_decode(q, kc, vc, n, ctx_lens=cl, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    kd = oracle.dequantize_kv_fp8(kc.cpu().numpy(), ks.cpu().numpy())
    vd = oracle.dequantize_kv_fp8(vc.cpu().numpy(), vs.cpu().numpy())
    ro, _ = oracle.decode_attention(to64(q), kd, vd, lens)
    check(to64(o), ro, "bf16", "fp8 decode", rel_axes=(2,))
    # quantisation error against the unquantised cache is reported, not gated
    ru, _ = oracle.decode_attention(to64(q), to64(kf), to64(vf), lens)
    print("fp8 cache: max |O - O_unquantised| =", np.abs(to64(o) - ru).max())


def test_decode_constant_values():
    B, Hq, Hkv, n, d = 2, 8, 2, 2000, 128
    q = randn((B, Hq, d), 950, device=DEV) * 5
    k = randn((B, Hkv, n, d), 951, device=DEV) * 5
    v = torch.ones(B, Hkv, n, d, dtype=torch.bfloat16, device=DEV)
    o = yk.yoco_cross_attn_decode(q, k, v, n)
    torch.cuda.synchronize()
    assert (o.float() - 1).abs().max().item() <= 2e-2


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("B,Hq,Hkv,n", [(3, 8, 2, 5000), (16, 32, 8, 1024)])
def test_decode_writes_nothing_outside_its_outputs(kv, B, Hq, Hkv, n):
    """o and lse live inside NaN-filled guard regions of a larger allocation:
    every guard element is still NaN (bitwise) after the call."""
    d, G = 128, 4096
    q = randn((B, Hq, d), 960, device=DEV)
    if kv == "fp8":
        kc, ks = yk.yoco_kv_quantize_fp8(randn((B, Hkv, n, d), 961, dtype="f32", device=DEV))
        vc, vs = yk.yoco_kv_quantize_fp8(randn((B, Hkv, n, d), 962, dtype="f32", device=DEV))
    else:
        kc, vc = randn((B, Hkv, n, d), 961, device=DEV), randn((B, Hkv, n, d), 962, device=DEV)
        ks = vs = None
    obuf = torch.full((G + B * Hq * d + G,), float("nan"), dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((G + B * Hq + G,), float("nan"), dtype=torch.float32, device=DEV)
    o = obuf[G:G + B * Hq * d].view(B, Hq, d)
    lse = lbuf[G:G + B * Hq].view(B, Hq)
    yk.yoco_cross_attn_decode(q, kc, vc, n, k_scale=ks, v_scale=vs, o=o, lse=lse)
    torch.cuda.synchronize()
    for buf, m in ((obuf, B * Hq * d), (lbuf, B * Hq)):
        assert bool(torch.isnan(buf[:G]).all()) and bool(torch.isnan(buf[G + m:]).all())
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())


# ---------------------------------------------------------------------------
# The two K-load forms of the bf16 d = 128 split kernel over one split plan
# ---------------------------------------------------------------------------
_FORMS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_lib", "libyoco_decode_forms.so")


@pytest.mark.parametrize("B,Hq,Hkv,ctx,lens,n_splits", [
    (16, 32, 8, 32768, None, 32),                                  # 1024-key splits (libyoco's 4096-workgroup plan)
    (4, 24, 8, 20000, [20000, 1, 12345, 19999], 7),                # ragged, 2880-key splits
    (2, 8, 2, 3000, [3000, 64], 47),                               # 64-key splits (short: operand-layout territory)
])
def test_decode_k_load_forms_are_bitwise_equal(B, Hq, Hkv, ctx, lens, n_splits):
    """The whole-line form (8 keys x one 128-byte line per load, a DPP row
    rotate into the operand layout) and the operand-layout form run over the
    same split plan give identical o and lse."""
    print(f"decode K-load forms B={B} Hq={Hq} ctx={ctx} splits={n_splits}", flush=True)
    L = ctypes.CDLL(_FORMS)
    vp, i_, f_ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.yoco_test_decode_form.argtypes = [vp] * 4 + [i_] + [vp] * 3 + [i_] * 7 + [f_, vp]
    d = 128
    chunk = -(-ctx // n_splits)
    chunk = -(-chunk // 64) * 64
    n_splits = -(-ctx // chunk)
    q = randn((B, Hq, d), 970, device=DEV)
    k = randn((B, Hkv, ctx, d), 971, device=DEV)
    v = randn((B, Hkv, ctx, d), 972, device=DEV)
    cl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    ws = torch.empty(B * Hq * n_splits * (d + 2), dtype=torch.float32, device=DEV)
    outs = []
    for full in (0, 1):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
        p = lambda t: None if t is None else vp(t.data_ptr())  # noqa: E731
        st = L.yoco_test_decode_form(p(q), p(k), p(v), p(cl), ctx, p(o), p(lse), p(ws), B, Hq, Hkv, ctx, n_splits,
                                     chunk, full, f_(d ** -0.5 * 1.4426950408889634),
                                     vp(torch.cuda.current_stream().cuda_stream))
        assert st == 0
        torch.cuda.synchronize()
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    ro, _ = oracle.decode_attention(to64(q), to64(k), to64(v), [ctx] * B if lens is None else lens)
    check(to64(outs[1][0]), ro, "bf16", "whole-line form", rel_axes=(2,))
