"""Tolerances of the parity tests and the helpers that apply them.

bf16 inputs with float32 accumulation: max-abs <= 2e-2 and mean-abs <= 2e-3
against the float64 oracle; because attention outputs shrink like
sqrt(e/|A|) at long context (so absolute bounds alone would accept an
all-zero output) every compared (b, h) slice must also satisfy
||out - ref||_2 <= 1e-2 * ||ref||_2.  float32 inputs: max-abs <= 1e-5.
Log-sum-exp: 1e-3 (bf16), 1e-5 (f32).
"""
import numpy as np

BF16_MAX, BF16_MEAN, BF16_REL = 2e-2, 2e-3, 1e-2
F32_MAX = 1e-5


def to64(t):
    return t.detach().to("cpu").double().numpy()


def check(out, ref, dtype, what="", rel_axes=None, rel_tol=BF16_REL):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - ref)
    if dtype == "f32":
        assert err.max() <= F32_MAX, f"{what}: max-abs {err.max():.3e} > {F32_MAX}"
        return err.max()
    assert err.max() <= BF16_MAX, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= BF16_MEAN, f"{what}: mean-abs {err.mean():.3e}"
    if rel_axes is not None:
        num = np.sqrt(np.sum((out - ref) ** 2, axis=rel_axes))
        den = np.sqrt(np.sum(ref ** 2, axis=rel_axes))
        rel = num / np.maximum(den, 1e-30)
        assert rel.max() <= rel_tol, f"{what}: relative L2 error {rel.max():.3e}"
    return err.max()
