"""The allocation-free decode entry point, called through the C ABI.

yoco_cross_attn_decode_noalloc runs the kernels of yoco_cross_attn_decode with
the library's fixed per-device array as the workspace.  Two calls in a row,
the second on a smaller input, must each give exactly the output (and
log-sum-exp) of the workspace form on the same inputs, and both must match
the float64 oracle to the bf16 / f32 tolerances.  Sizes beyond the array are
rejected before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import shared_kv_attention_amd as yk
from shared_kv_attention_amd.synth import randn
from tests._tol import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc(q, k, v, ctx, o, lse, ctx_lens=None, k_scale=None, v_scale=None):
    """Direct ctypes call of the C entry point (no binding logic in between)."""
    L = yk.lib()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    B, Hq, d = q.shape
    Hkv, n_cap = k.shape[1], k.shape[2]
    qdt = yk.BF16 if q.dtype == torch.bfloat16 else yk.F32
    kdt = {torch.bfloat16: yk.BF16, torch.float32: yk.F32, torch.uint8: yk.FP8_E4M3}[k.dtype]
    return L.yoco_cross_attn_decode_noalloc(p(q), p(k), p(v), p(k_scale), p(v_scale), p(ctx_lens), ctx, p(o), p(lse),
                                            B, Hq, Hkv, n_cap, d, 0.0, qdt, kdt,
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


CASES = [
    # (B, Hq, Hkv, n_cap, ctx, ctx_lens, d, dtype): a large call, then a smaller one
    ((4, 32, 8, 32768, 32768, None, 128, "bf16"), (2, 8, 2, 3000, 2999, [2999, 17], 64, "bf16")),
    ((2, 24, 8, 8192, 8000, [8000, 4097], 128, "f32"), (1, 4, 1, 300, 300, None, 128, "f32")),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_form(first, second):
    for i, (B, Hq, Hkv, n_cap, ctx, ctx_lens, d, dt) in enumerate((first, second)):
        print(f"noalloc call {i}: B={B} Hq={Hq} Hkv={Hkv} n_cap={n_cap} ctx={ctx} d={d} {dt}", flush=True)
        assert yk.yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d) <= \
            yk.yoco_cross_attn_decode_noalloc_max_bytes()
        q = randn((B, Hq, d), 1300 + i, dtype=dt, device=DEV)
        k = randn((B, Hkv, n_cap, d), 1310 + i, dtype=dt, device=DEV)
        v = randn((B, Hkv, n_cap, d), 1320 + i, dtype=dt, device=DEV)
        lens = [ctx] * B if ctx_lens is None else ctx_lens
        cl = None if ctx_lens is None else torch.tensor(ctx_lens, dtype=torch.int32, device=DEV)
        o_ref = torch.empty_like(q)
        lse_ref = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
        yk.yoco_cross_attn_decode(q, k, v, ctx, ctx_lens=cl, o=o_ref, lse=lse_ref)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
        assert _noalloc(q, k, v, ctx, o, lse, ctx_lens=cl) == 0
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "no-alloc output differs from the workspace form"
        assert torch.equal(lse, lse_ref)
        ro, rl = oracle.decode_attention(to64(q), to64(k), to64(v), lens)
        check(to64(o), ro, dt, "no-alloc decode O", rel_axes=(2,))
        assert np.abs(to64(lse) - rl).max() <= (1e-5 if dt == "f32" else 1e-3)


def test_noalloc_fp8_cache_then_smaller():
    for i, (B, n) in enumerate(((8, 65536), (1, 1000))):
        Hq, Hkv, d = 32, 8, 128
        print(f"noalloc fp8 call {i}: B={B} n={n}", flush=True)
        q = randn((B, Hq, d), 1330 + i, device=DEV)
        kc, ks = yk.yoco_kv_quantize_fp8(randn((B, Hkv, n, d), 1340 + i, dtype="f32", device=DEV))
        vc, vs = yk.yoco_kv_quantize_fp8(randn((B, Hkv, n, d), 1350 + i, dtype="f32", device=DEV))
        o_ref = yk.yoco_cross_attn_decode(q, kc, vc, n, k_scale=ks, v_scale=vs)
        o = torch.full_like(q, float("nan"))
        assert _noalloc(q, kc, vc, n, o, None, k_scale=ks, v_scale=vs) == 0
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)


def test_noalloc_rejects_sizes_beyond_its_array():
    # 1024 sequences x 64 query heads at d = 128 (one split each: 65536 partial
    # rows, 32 MiB) need more than the array holds: rejected before anything
    # is launched (the pointers are never read)
    B, Hq, Hkv, ctx, d = 1024, 64, 8, 1000, 128
    assert yk.yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d) > yk.yoco_cross_attn_decode_noalloc_max_bytes()
    L = yk.lib()
    P = ctypes.c_void_p(4096)
    st = L.yoco_cross_attn_decode_noalloc(P, P, P, None, None, None, ctx, P, None, B, Hq, Hkv, ctx, d, 0.0, yk.BF16,
                                          yk.BF16, None)
    assert st == 6   # YOCO_ERR_WORKSPACE
