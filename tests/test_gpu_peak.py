"""The achievable-peak microbenchmarks compute checkable results: the read's
per-workgroup sums add up (modulo 2^32) to the sum of every 32-bit word of
the buffer, and the matrix-core loops' outputs equal 128 * iters (operands
of ones) and 0 (operands that cancel over every 8 rounds) exactly."""
import pytest
import torch

import shared_kv_attention_amd as yk

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("n_words,blocks", [(4, 1), (1 << 20, 64), ((1 << 24) + 12, 2048)])
def test_peak_read_reads_every_word(n_words, blocks):
    g = torch.Generator(device=DEV)
    g.manual_seed(n_words)
    buf = torch.randint(-(1 << 31), (1 << 31) - 1, (n_words,), dtype=torch.int32, device=DEV, generator=g)
    part = yk.yoco_peak_hbm_read(buf, blocks=blocks)
    torch.cuda.synchronize()
    got = int(part.to(torch.int64).sum().item()) % (1 << 32)
    ref = int(buf.to(torch.int64).sum().item()) % (1 << 32)
    assert got == ref


@pytest.mark.parametrize("iters,blocks", [(1, 1), (1000, 256), (1 << 20, 8)])
def test_peak_mfma_exact(iters, blocks):
    out = yk.yoco_peak_mfma_bf16(iters, blocks=blocks)
    torch.cuda.synchronize()
    assert torch.all(out == 128.0 * iters)


@pytest.mark.parametrize("iters,blocks", [(8, 1), (1000, 256), (1 << 20, 8)])
def test_peak_mfma_toggling_exact(iters, blocks):
    out = yk.yoco_peak_mfma_bf16_toggling(iters, blocks=blocks)
    torch.cuda.synchronize()
    assert torch.all(out == 0.0)
