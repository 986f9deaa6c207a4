"""Python binding of libyoco.so: the MI355X YOCO shared-KV attention hot path.

Thin argument marshalling over the C ABI declared in include/yoco.h: every
function takes torch tensors that already live on the GPU, checks dtypes and
contiguity, and passes raw device pointers plus torch's current HIP stream to
the library.  All computation happens in the library's HIP kernels; there is
no fallback of any kind -- if libyoco.so is missing the first call raises.

Entry points (same names as the C functions):
    yoco_global_kv_proj        RMSNorm + one-time K/V projection into the cache
    yoco_swa_attn              self-decoder sliding-window attention
    yoco_cross_attn_prefill    causal cross-attention over the shared cache
    yoco_cross_attn_decode     one-token split-K decode over the shared cache
    yoco_kv_quantize_fp8       8-bit (e4m3fn) cache writer with per-head scales
"""

import ctypes
import os

__all__ = [
    "YocoError",
    "lib",
    "library_path",
    "yoco_global_kv_proj",
    "yoco_global_kv_proj_workspace_bytes",
    "yoco_swa_attn",
    "yoco_swa_attn_halo",
    "yoco_peak_hbm_read",
    "yoco_peak_mfma_bf16",
    "yoco_peak_mfma_bf16_toggling",
    "yoco_attn_merge",
    "yoco_cross_attn_prefill",
    "yoco_cross_attn_decode",
    "yoco_cross_attn_decode_workspace_bytes",
    "yoco_cross_attn_decode_noalloc",
    "yoco_cross_attn_decode_noalloc_max_bytes",
    "yoco_swa_decode",
    "yoco_swa_decode_workspace_bytes",
    "yoco_gret_prefill",
    "yoco_gret_prefill_workspace_bytes",
    "yoco_gret_decode",
    "yoco_gret_group_norm_swish",
    "yoco_qkv_proj",
    "yoco_swiglu",
    "yoco_linear_residual",
    "yoco_kv_quantize_fp8",
    "yoco_kv_quantize_fp8_workspace_bytes",
    "yoco_status_string",
    "yoco_version",
    "F32",
    "BF16",
    "FP8_E4M3",
]

F32, BF16, FP8_E4M3 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libyoco.so")
_lib = None

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "yoco_global_kv_proj": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _f, _i, _i,
                                 _vp, _sz, _vp]),
    "yoco_global_kv_proj_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "yoco_swa_attn": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "yoco_swa_attn_halo": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "yoco_attn_merge": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "yoco_cross_attn_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "yoco_cross_attn_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i,
                                    _vp, _sz, _vp]),
    "yoco_cross_attn_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "yoco_cross_attn_decode_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                                            _i, _vp]),
    "yoco_cross_attn_decode_noalloc_max_bytes": (_sz, []),
    "yoco_swa_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "yoco_swa_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "yoco_gret_prefill": (_i, [_vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "yoco_gret_prefill_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "yoco_gret_decode": (_i, [_vp, _vp, _vp, _vp, _f, _vp, _vp, _i, _i, _i, _i, _vp]),
    "yoco_gret_group_norm_swish": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]),
    "yoco_qkv_proj": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _f, _i, _i, _vp]),
    "yoco_swiglu": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]),
    "yoco_linear_residual": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "yoco_kv_quantize_fp8": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "yoco_kv_quantize_fp8_workspace_bytes": (_sz, [_i]),
    "yoco_peak_hbm_read": (_i, [_vp, _sz, _vp, _i, _vp]),
    "yoco_peak_mfma_bf16": (_i, [_i, _vp, _i, _vp]),
    "yoco_peak_mfma_bf16_toggling": (_i, [_i, _vp, _i, _vp]),
    "yoco_status_string": (ctypes.c_char_p, [_i]),
    "yoco_version": (_i, []),
}


def lib():
    """Load libyoco.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is missing: build it with `python -m shared_kv_attention_amd.build` "
                "(there is no fallback path)")
        handle = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class YocoError(RuntimeError):
    def __init__(self, status, fn):
        self.status = status
        super().__init__(f"{fn}: status {status} ({yoco_status_string(status)})")


def yoco_status_string(status):
    return lib().yoco_status_string(int(status)).decode()


def yoco_version():
    return lib().yoco_version()


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.uint8:
        return FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(status, fn):
    if status != 0:
        raise YocoError(status, fn)


def yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, act_dtype, kv_dtype):
    return lib().yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, act_dtype, kv_dtype)


def yoco_global_kv_proj(x, w_k, w_v, k_out, v_out, pos0=0, norm_w=None, eps=1e-6, rope_theta=0.0, k_scale=None,
                        v_scale=None, workspace=None, stream=None):
    """K/V cache rows [pos0, pos0+N) = RMSNorm(x) @ W^T, split into KV heads.

    x [B, N, D]; w_k, w_v [Hkv*d, D]; k_out, v_out [B, Hkv, n_cap, d] in x's dtype, or uint8 for an 8-bit
    (e4m3fn) cache: then k_scale, v_scale [Hkv] float32 are written (pos0 == 0; allocated if not given) or read
    (pos0 > 0).  rope_theta > 0 rotates the keys at their cache positions.
    Returns (k_out, v_out), or (k_out, v_out, k_scale, v_scale) for an 8-bit cache.
    """
    torch = _torch()
    B, N, D = x.shape
    _, Hkv, n_cap, d = k_out.shape
    act, kvd = _dtype_code(x), _dtype_code(k_out)
    fp8 = kvd == FP8_E4M3
    if fp8 and k_scale is None:
        k_scale = torch.empty(Hkv, dtype=torch.float32, device=x.device)
    if fp8 and v_scale is None:
        v_scale = torch.empty(Hkv, dtype=torch.float32, device=x.device)
    if fp8 and workspace is None:
        need = yoco_global_kv_proj_workspace_bytes(B, N, Hkv, d, act, kvd)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().yoco_global_kv_proj(_ptr(x), _ptr(norm_w), _ptr(w_k), _ptr(w_v), _ptr(k_out), _ptr(v_out),
                                   _ptr(k_scale if fp8 else None), _ptr(v_scale if fp8 else None),
                                   B, N, D, Hkv, d, n_cap, pos0, eps, float(rope_theta), act, kvd,
                                   _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "yoco_global_kv_proj")
    if fp8:
        return k_out, v_out, k_scale, v_scale
    return k_out, v_out


def yoco_qkv_proj(x, w_q, head_dim, w_k=None, w_v=None, q_out=None, k_out=None, v_out=None, norm_w=None,
                  eps=1e-6, rope_theta=0.0, rope_pos0=0, stream=None):
    """Pre-norm Q/K/V projection: q [B, Hq, N, d] = heads(RMSNorm(x) @ W_q^T), k and v likewise
    ([B, Hkv, N, d]); w_k = w_v = None projects q only.  rope_theta > 0 rotates q and k of token n
    at position rope_pos0 + n.  Returns (q, k, v) (k, v None for q only)."""
    torch = _torch()
    B, N, D = x.shape
    d = int(head_dim)
    Hq = w_q.shape[0] // d
    Hkv = 0 if w_k is None else w_k.shape[0] // d
    if q_out is None:
        q_out = torch.empty(B, Hq, N, d, dtype=x.dtype, device=x.device)
    if Hkv > 0:
        if k_out is None:
            k_out = torch.empty(B, Hkv, N, d, dtype=x.dtype, device=x.device)
        if v_out is None:
            v_out = torch.empty(B, Hkv, N, d, dtype=x.dtype, device=x.device)
    st = lib().yoco_qkv_proj(_ptr(x), _ptr(norm_w), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(q_out),
                             _ptr(k_out if Hkv else None), _ptr(v_out if Hkv else None), B, N, D, Hq, Hkv, d,
                             float(eps), float(rope_theta), int(rope_pos0), _dtype_code(x), _stream(stream))
    _check(st, "yoco_qkv_proj")
    return q_out, (k_out if Hkv else None), (v_out if Hkv else None)


def yoco_swiglu(x, w_gate, w_up, h=None, norm_w=None, eps=1e-6, stream=None):
    """h [B, N, F] = silu(RMSNorm(x) @ W_gate^T) * (RMSNorm(x) @ W_up^T)."""
    torch = _torch()
    B, N, D = x.shape
    F = w_gate.shape[0]
    if h is None:
        h = torch.empty(B, N, F, dtype=x.dtype, device=x.device)
    st = lib().yoco_swiglu(_ptr(x), _ptr(norm_w), _ptr(w_gate), _ptr(w_up), _ptr(h), B, N, D, F, float(eps),
                           _dtype_code(x), _stream(stream))
    _check(st, "yoco_swiglu")
    return h


def yoco_linear_residual(a, w, y, a_heads=0, stream=None):
    """y [B, N, F] += rows(a) @ W^T in place; a [B, N, K], or head-major [B, H, N, K/H] with a_heads = H."""
    B, N, F = y.shape
    K = w.shape[1]
    st = lib().yoco_linear_residual(_ptr(a), int(a_heads), _ptr(w), _ptr(y), B, N, K, F, _dtype_code(y),
                                    _stream(stream))
    _check(st, "yoco_linear_residual")
    return y


def yoco_swa_attn(q, k, v, window, o=None, lse=None, softmax_scale=0.0, stream=None):
    """Sliding-window attention; q [B, Hq, N, d], k/v [B, Hkv, N, d]. Returns o."""
    torch = _torch()
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if o is None:
        o = torch.empty_like(q)
    st = lib().yoco_swa_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, int(window),
                             float(softmax_scale), _dtype_code(q), _stream(stream))
    _check(st, "yoco_swa_attn")
    return o


def yoco_peak_hbm_read(buf, blocks=2048, partial=None, stream=None):
    """Stream `buf` (a device tensor, size a multiple of 16 bytes) once; returns the per-workgroup uint32 sums
    (as int32)."""
    torch = _torch()
    if partial is None:
        partial = torch.empty(blocks, dtype=torch.int32, device=buf.device)
    st = lib().yoco_peak_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(partial), int(blocks),
                                  _stream(stream))
    _check(st, "yoco_peak_hbm_read")
    return partial


def yoco_peak_mfma_bf16(iters, blocks=1024, out=None, device=None, stream=None):
    """Matrix-core loop: blocks x 4 waves x iters x 8 MFMAs of 32x32x16 bf16; returns out [4 * blocks]."""
    torch = _torch()
    if out is None:
        out = torch.empty(4 * blocks, dtype=torch.float32, device=device or "cuda")
    st = lib().yoco_peak_mfma_bf16(int(iters), _ptr(out), int(blocks), _stream(stream))
    _check(st, "yoco_peak_mfma_bf16")
    return out


def yoco_peak_mfma_bf16_toggling(iters, blocks=1024, out=None, device=None, stream=None):
    """The matrix-core loop on operands that change every instruction (iters a multiple of 8); returns
    out [4 * blocks], exactly 0."""
    torch = _torch()
    if out is None:
        out = torch.empty(4 * blocks, dtype=torch.float32, device=device or "cuda")
    st = lib().yoco_peak_mfma_bf16_toggling(int(iters), _ptr(out), int(blocks), _stream(stream))
    _check(st, "yoco_peak_mfma_bf16_toggling")
    return out


def yoco_swa_attn_halo(q, k, v, window, o=None, lse=None, softmax_scale=0.0, stream=None):
    """One shard's sliding-window attention: k/v [B, Hkv, Nkv, d] are a halo of earlier rows followed by the
    shard's rows, q [B, Hq, Nq, d] the shard's own (last Nq) rows.  Returns o."""
    torch = _torch()
    B, Hq, Nq, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if o is None:
        o = torch.empty_like(q)
    st = lib().yoco_swa_attn_halo(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nkv, d, int(window),
                                  float(softmax_scale), _dtype_code(q), _stream(stream))
    _check(st, "yoco_swa_attn_halo")
    return o


def yoco_attn_merge(o_parts, lse_parts, o=None, lse=None, stream=None):
    """Merge per-shard attention results: o_parts [S, ..., d], lse_parts [S, ...] float32.  Returns o [..., d]."""
    torch = _torch()
    S, d = o_parts.shape[0], o_parts.shape[-1]
    rows = o_parts[0].numel() // d
    if o is None:
        o = torch.empty(o_parts.shape[1:], dtype=o_parts.dtype, device=o_parts.device)
    st = lib().yoco_attn_merge(_ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse), S, rows, d, _dtype_code(o_parts),
                               _stream(stream))
    _check(st, "yoco_attn_merge")
    return o


def yoco_cross_attn_prefill(q, k, v, n_kv=None, q_offset=0, o=None, lse=None, softmax_scale=0.0, stream=None):
    """Causal cross-attention; q [B, Hq, Nq, d] at positions q_offset.., cache k/v [B, Hkv, n_cap, d]."""
    torch = _torch()
    B, Hq, Nq, d = q.shape
    Hkv, n_cap = k.shape[1], k.shape[2]
    if n_kv is None:
        n_kv = n_cap
    if o is None:
        o = torch.empty_like(q)
    st = lib().yoco_cross_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, n_kv, n_cap,
                                       q_offset, d, float(softmax_scale), _dtype_code(q), _stream(stream))
    _check(st, "yoco_cross_attn_prefill")
    return o


def yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d):
    return lib().yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d)


def yoco_cross_attn_decode(q, k_cache, v_cache, ctx, ctx_lens=None, k_scale=None, v_scale=None, o=None, lse=None,
                           workspace=None, softmax_scale=0.0, stream=None):
    """One decode step; q [B, Hq, d], caches [B, Hkv, n_cap, d] (bf16/f32, or uint8 e4m3fn codes)."""
    torch = _torch()
    B, Hq, d = q.shape
    Hkv, n_cap = k_cache.shape[1], k_cache.shape[2]
    need = yoco_cross_attn_decode_workspace_bytes(B, Hq, Hkv, ctx, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    st = lib().yoco_cross_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(ctx_lens), int(ctx), _ptr(o),
        _ptr(lse), B, Hq, Hkv, n_cap, d, float(softmax_scale), _dtype_code(q), _dtype_code(k_cache),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "yoco_cross_attn_decode")
    return o


def yoco_cross_attn_decode_noalloc_max_bytes():
    return lib().yoco_cross_attn_decode_noalloc_max_bytes()


def yoco_cross_attn_decode_noalloc(q, k_cache, v_cache, ctx, o, ctx_lens=None, k_scale=None, v_scale=None, lse=None,
                                   softmax_scale=0.0, stream=None):
    """yoco_cross_attn_decode with the library's fixed device array as its workspace (nothing is allocated;
    the caller passes the output o).  Calls that overlap on one GPU race."""
    B, Hq, d = q.shape
    Hkv, n_cap = k_cache.shape[1], k_cache.shape[2]
    st = lib().yoco_cross_attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(ctx_lens), int(ctx), _ptr(o),
        _ptr(lse), B, Hq, Hkv, n_cap, d, float(softmax_scale), _dtype_code(q), _dtype_code(k_cache),
        _stream(stream))
    _check(st, "yoco_cross_attn_decode_noalloc")
    return o


def yoco_swa_decode_workspace_bytes(B, Hq, Hkv, W, d):
    return lib().yoco_swa_decode_workspace_bytes(B, Hq, Hkv, W, d)


def yoco_swa_decode(q, k_ring, v_ring, pos, k_new=None, v_new=None, o=None, lse=None, workspace=None,
                    softmax_scale=0.0, stream=None):
    """Self-decoder window decode of the token at position pos; q [B, Hq, d], rings [B, Hkv, W, d]
    (position t in slot t mod W).  k_new/v_new [B, Hkv, d], if given, are written to slot pos mod W first."""
    torch = _torch()
    B, Hq, d = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    need = yoco_swa_decode_workspace_bytes(B, Hq, Hkv, W, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    st = lib().yoco_swa_decode(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_ring), _ptr(v_ring), int(pos), _ptr(o), _ptr(lse),
        B, Hq, Hkv, W, d, float(softmax_scale), _dtype_code(q), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "yoco_swa_decode")
    return o


def yoco_gret_prefill_workspace_bytes(B, H, N, d, chunk=256):
    return lib().yoco_gret_prefill_workspace_bytes(B, H, N, d, chunk)


def yoco_gret_prefill(q, k, v, gate_logit, tau, state_in=None, o=None, state_out=None, chunk=256, workspace=None,
                      stream=None):
    """Gated retention, chunkwise: q, k, v [B, H, N, d] bf16, gate_logit [B, H, N] f32; returns (o, state_out).
    state_out is allocated ([B, H, d, d] f32) unless given; pass state_out=False to skip it."""
    torch = _torch()
    B, H, N, d = q.shape
    need = yoco_gret_prefill_workspace_bytes(B, H, N, d, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(q)
    if state_out is None:
        state_out = torch.empty(B, H, d, d, dtype=torch.float32, device=q.device)
    elif state_out is False:
        state_out = None
    st = lib().yoco_gret_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate_logit), float(tau), _ptr(state_in), _ptr(o), _ptr(state_out),
        B, H, N, d, int(chunk), _dtype_code(q), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "yoco_gret_prefill")
    return o, state_out


def yoco_gret_decode(q, k, v, gate_logit, tau, state, o=None, stream=None):
    """Gated retention, one recurrent step: q, k, v [B, H, d]; gate_logit [B, H] f32; state [B, H, d, d] f32
    (updated in place).  Returns o."""
    B, H, d = q.shape
    if o is None:
        o = _torch().empty_like(q)
    st = lib().yoco_gret_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(gate_logit), float(tau), _ptr(state), _ptr(o),
                                B, H, d, _dtype_code(q), _stream(stream))
    _check(st, "yoco_gret_decode")
    return o


def yoco_gret_group_norm_swish(y, g, out=None, eps=1e-6, stream=None):
    """Per-head GroupNorm of y [B, H, N, d] times swish(g) ([B, N, H*d]); returns out [B, N, H*d]."""
    B, H, N, d = y.shape
    if out is None:
        out = _torch().empty_like(g)
    st = lib().yoco_gret_group_norm_swish(_ptr(y), _ptr(g), _ptr(out), B, H, N, d, float(eps), _dtype_code(y),
                                          _stream(stream))
    _check(st, "yoco_gret_group_norm_swish")
    return out


def yoco_kv_quantize_fp8_workspace_bytes(Hkv):
    return lib().yoco_kv_quantize_fp8_workspace_bytes(Hkv)


def yoco_kv_quantize_fp8(kv, codes=None, scale=None, workspace=None, stream=None):
    """Quantise kv [B, Hkv, n, d] (f32/bf16) to e4m3fn codes + per-head float32 scales."""
    torch = _torch()
    B, Hkv, n, d = kv.shape
    if codes is None:
        codes = torch.empty(kv.shape, dtype=torch.uint8, device=kv.device)
    if scale is None:
        scale = torch.empty(Hkv, dtype=torch.float32, device=kv.device)
    if workspace is None:
        workspace = torch.empty(max(yoco_kv_quantize_fp8_workspace_bytes(Hkv), 16), dtype=torch.uint8,
                                device=kv.device)
    st = lib().yoco_kv_quantize_fp8(_ptr(kv), _dtype_code(kv), _ptr(codes), _ptr(scale), B, Hkv, n, d,
                                    _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "yoco_kv_quantize_fp8")
    return codes, scale
