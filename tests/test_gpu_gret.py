"""Gated retention on the GPU against the float64 oracle: the chunkwise
prefill (outputs and final state), the recurrent decode step, the state
hand-over from prefill to decode, and the per-head GroupNorm with swish gate.

Retention outputs are not normalised (their scale grows with the decay
horizon: with a gate near 1 a row sums O(N) terms, and single outputs reach
~10x the slice's RMS), so their parity is relative, per (b, h) slice:
||out - ref||_2 <= 1e-2 ||ref||_2, and per element
|out - ref| <= 8e-3 |ref| + 2e-2 rms(ref) -- bf16 output rounding alone is up
to 2^-9 |ref|, the bf16 weights and state add about as much, and an indexing
mistake shows up as errors of the order of the value itself.  The GroupNorm
output is O(1) and uses the usual absolute bf16 / f32 bounds."""
import numpy as np
import pytest
import torch

import oracle
import shared_kv_attention_amd as yk
from shared_kv_attention_amd.synth import randn
from _tol import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def rel_check(out, ref, what, rel=1e-2, elem=8e-3, floor=2e-2):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape
    assert np.all(np.isfinite(out)), f"{what}: non-finite"
    B, H = ref.shape[:2]
    for b in range(B):
        for h in range(H):
            e = out[b, h] - ref[b, h]
            rms = np.sqrt(np.mean(ref[b, h] ** 2))
            r = np.linalg.norm(e) / max(np.linalg.norm(ref[b, h]), 1e-300)
            assert r <= rel, f"{what} (b={b}, h={h}): relative L2 {r:.3e}"
            bound = elem * np.abs(ref[b, h]) + floor * rms
            worst = np.argmax(np.abs(e) - bound)
            assert np.all(np.abs(e) <= bound), \
                f"{what} (b={b}, h={h}): err {np.abs(e).flat[worst]:.3e} > bound {bound.flat[worst]:.3e}"


def _inputs(B, H, N, d, seed, zshift, zscale):
    s = d ** -0.25    # q . k ~ N(0, 1)
    q = randn((B, H, N, d), seed, std=s, device=DEV)
    k = randn((B, H, N, d), seed + 1, std=s, device=DEV)
    v = randn((B, H, N, d), seed + 2, device=DEV)
    z = randn((B, H, N), seed + 3, std=zscale, dtype="f32", device=DEV) + zshift
    return q, k, v, z


CASES = [
    # B, H, N, d, chunk, tau, z shift, z scale, initial state
    (1, 2, 300, 128, 256, 4.0, 2.0, 1.0, False),     # ragged last chunk, decay near 1
    (2, 3, 512, 64, 128, 1.0, 0.0, 2.0, True),       # moderate decay, given state
    (1, 1, 77, 128, 128, 16.0, 1.0, 1.0, True),      # one short chunk
    (1, 2, 1, 64, 256, 4.0, 0.0, 1.0, False),        # a single position
    (1, 2, 600, 128, 256, 0.5, -4.0, 2.0, False),    # strong decay (tiny gates: no overflow allowed)
    (2, 2, 1000, 64, 256, 16.0, 6.0, 1.0, True),     # gate ~1: nearly linear attention
]


@pytest.mark.parametrize("B,H,N,d,chunk,tau,zs,zc,with_state", CASES)
def test_gret_prefill_matches_oracle(B, H, N, d, chunk, tau, zs, zc, with_state):
    print(f"gret prefill B={B} H={H} N={N} d={d} chunk={chunk} tau={tau} z~{zs}+{zc}N state={with_state}", flush=True)
    q, k, v, z = _inputs(B, H, N, d, 8000 + N + d, zs, zc)
    s0 = randn((B, H, d, d), 8100 + N, std=0.1, dtype="f32", device=DEV) if with_state else None
    o, st = yk.yoco_gret_prefill(q, k, v, z, tau, state_in=s0, chunk=chunk)
    torch.cuda.synchronize()
    ref_o, ref_st = oracle.gret_chunkwise(to64(q), to64(k), to64(v), to64(z), tau, chunk,
                                          None if s0 is None else to64(s0))
    rel_check(to64(o), ref_o, "gret prefill o")
    rel_check(to64(st), ref_st, "gret prefill state")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_gret_decode_matches_oracle(dt, d):
    B, H = 3, 4
    q = randn((B, H, d), 8201 + d, dtype=dt, device=DEV)
    k = randn((B, H, d), 8202 + d, dtype=dt, device=DEV)
    v = randn((B, H, d), 8203 + d, dtype=dt, device=DEV)
    z = randn((B, H), 8204 + d, std=2.0, dtype="f32", device=DEV)
    st = randn((B, H, d, d), 8205 + d, std=0.3, dtype="f32", device=DEV)
    st0 = to64(st)
    o = yk.yoco_gret_decode(q, k, v, z, 4.0, st)
    torch.cuda.synchronize()
    ref_o, ref_st = oracle.gret_recurrent(to64(q)[:, :, None], to64(k)[:, :, None], to64(v)[:, :, None],
                                          to64(z)[:, :, None], 4.0, st0)
    if dt == "f32":
        rel_check(to64(o), ref_o[:, :, 0], "gret decode o", rel=1e-5, elem=1e-5, floor=1e-5)
    else:
        rel_check(to64(o), ref_o[:, :, 0], "gret decode o")
    rel_check(to64(st), ref_st, "gret decode state", rel=1e-6, elem=1e-6, floor=1e-6)


@pytest.mark.parametrize("N1", [200, 256])
def test_prefill_then_decode_continues_the_sequence(N1):
    """Prefill of N1 positions hands its state to decode steps for the next
    positions; every output equals the oracle's run over the whole sequence."""
    B, H, d, extra, tau = 1, 3, 128, 6, 4.0
    q, k, v, z = _inputs(B, H, N1 + extra, d, 8300 + N1, 1.0, 1.5)
    o_pre, st = yk.yoco_gret_prefill(q[:, :, :N1].contiguous(), k[:, :, :N1].contiguous(),
                                     v[:, :, :N1].contiguous(), z[:, :, :N1].contiguous(), tau)
    outs = [to64(o_pre)]
    for t in range(N1, N1 + extra):
        o_t = yk.yoco_gret_decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                                  z[:, :, t].contiguous(), tau, st)
        outs.append(to64(o_t)[:, :, None])
    torch.cuda.synchronize()
    ref, _ = oracle.gret_recurrent(to64(q), to64(k), to64(v), to64(z), tau)
    rel_check(np.concatenate(outs, axis=2), ref, "prefill + decode")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_group_norm_swish_matches_oracle(dt, d):
    B, H, N = 2, 3, 37
    y = randn((B, H, N, d), 8401 + d, std=3.0, dtype=dt, device=DEV) + 0.5
    g = randn((B, N, H * d), 8402 + d, dtype=dt, device=DEV)
    out = yk.yoco_gret_group_norm_swish(y.contiguous(), g)
    torch.cuda.synchronize()
    ref = oracle.gret_group_norm_swish(to64(y), to64(g))
    check(to64(out), ref, dt, f"group norm swish ({dt}, d={d})")


def test_gret_prefill_full_size_sampled_heads():
    """The 3B-shaped self-decoder layer (B1, N4096, 24 heads, d128, chunk 256)
    in the launch configuration the benchmark times; two heads checked
    against the oracle in full."""
    B, H, N, d = 1, 24, 4096, 128
    q, k, v, z = _inputs(B, H, N, d, 8500, 3.0, 1.0)
    o, st = yk.yoco_gret_prefill(q, k, v, z, 16.0)
    torch.cuda.synchronize()
    for h in (0, 17):
        ref_o, ref_st = oracle.gret_chunkwise(to64(q[:, h:h + 1]), to64(k[:, h:h + 1]), to64(v[:, h:h + 1]),
                                              to64(z[:, h:h + 1]), 16.0, 256)
        rel_check(to64(o[:, h:h + 1]), ref_o, f"full-size head {h}")
        rel_check(to64(st[:, h:h + 1]), ref_st, f"full-size state head {h}")


def test_gret_graph_replays_match_eager():
    """Gated-retention prefill (three kernels, workspace) and decode (state
    updated in place) captured as one HIP graph: every replay, with eager work
    between the replays, reproduces the eager calls bitwise."""
    B, H, N, d = 1, 4, 700, 128
    s = d ** -0.25
    q = randn((B, H, N, d), 990, std=s, device=DEV)
    k = randn((B, H, N, d), 991, std=s, device=DEV)
    v = randn((B, H, N, d), 992, device=DEV)
    z = randn((B, H, N), 993, dtype="f32", device=DEV) + 3.0
    o = torch.empty_like(q)
    st = torch.empty(B, H, d, d, dtype=torch.float32, device=DEV)
    ws = torch.empty(yk.yoco_gret_prefill_workspace_bytes(B, H, N, d, 256), dtype=torch.uint8, device=DEV)
    qd, kd, vd = (randn((B, H, d), 994 + i, std=s, device=DEV) for i in range(3))
    zd = randn((B, H), 997, dtype="f32", device=DEV) + 3.0
    od = torch.empty(B, H, d, dtype=torch.bfloat16, device=DEV)
    st_dec = torch.empty_like(st)

    def calls():
        yk.yoco_gret_prefill(q, k, v, z, 16.0, o=o, state_out=st, workspace=ws)
        st_dec.copy_(st)
        yk.yoco_gret_decode(qd, kd, vd, zd, 16.0, st_dec, o=od)

    calls()
    torch.cuda.synchronize()
    ref = (o.clone(), st.clone(), od.clone(), st_dec.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        for t in (o, st, od, st_dec):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((o, st, od, st_dec), ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager calls"
        calls()
        torch.cuda.synchronize()
