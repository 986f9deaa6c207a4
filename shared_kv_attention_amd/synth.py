"""Seeded synthetic inputs and the workload shapes they are drawn for.

This module holds no arithmetic of the attention method: it only names the
workloads (shapes, dtypes, value distributions) and draws seeded tensors.
Both the GPU tests and the float64 oracle checks take their inputs from here.

Recipe: every tensor is drawn as float32 N(0, 1) from a torch generator seeded
with ``1000 * workload_id + tensor_index``, multiplied by its standard
deviation, and rounded to the workload's dtype (round-to-nearest-even for
bfloat16).  Large tensors are drawn directly on the GPU; the oracle is then
given the exact drawn values (copied back), never a re-draw.

Value distributions follow the workloads: activations, queries and cached
keys/values N(0, 1); projection weights N(0, 0.02) for the 3B-shaped
workloads and N(0, 1/16) (= 1/sqrt(256)) for the tiny block.
"""

from dataclasses import dataclass
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "seed_for", "randn"]


@dataclass(frozen=True)
class Workload:
    wid: int                 # used in seeds
    name: str
    dtype: str               # "f32" | "bf16" | "fp8-kv"
    batch: int
    seq: int                 # prompt length, or decode context
    hidden: int              # model width D (0 when unused)
    n_heads: int
    n_kv_heads: int
    head_dim: int
    n_self_layers: int
    n_cross_layers: int
    window: int              # sliding window (0 when unused)
    weight_std: float
    decode_steps: int = 0
    ffn_dim: int = 0         # SwiGLU hidden size of the block layers (0: no feed-forward)


WORKLOADS = {
    "tiny_block_f32": Workload(1, "tiny_block_f32", "f32", 1, 256, 256, 4, 1, 64,
                               2, 2, 32, 1.0 / 16.0, ffn_dim=768),
    "prefill_3b_bf16": Workload(2, "prefill_3b_bf16", "bf16", 1, 4096, 3072, 24, 8, 128,
                                8, 8, 1024, 0.02, ffn_dim=8192),
    "decode_32k_bf16": Workload(3, "decode_32k_bf16", "bf16", 16, 32768, 0, 32, 8, 128,
                                0, 16, 0, 0.0, decode_steps=128),
    "early_exit_1m_bf16": Workload(4, "early_exit_1m_bf16", "bf16", 1, 1 << 20, 4096, 32, 8,
                                   128, 4, 8, 1024, 0.02),
    "decode_512k_fp8": Workload(5, "decode_512k_fp8", "fp8-kv", 8, 1 << 19, 0, 32, 8, 128,
                                0, 16, 0, 0.0, decode_steps=8),
    # one generated token per sequence at the decode shape: 16 self-decoder
    # layers (window 1024, ring caches), the one-row global KV projection
    # (hidden = 32 heads x 128), 16 cross-decoder layers over 32768 rows
    "generation_32k_bf16": Workload(6, "generation_32k_bf16", "bf16", 16, 32768, 4096, 32, 8, 128,
                                    16, 16, 1024, 0.02, decode_steps=16),
    # gated-retention self-decoder layer at the 3B shape (24 heads of 128,
    # chunk 256), and its recurrent decode step for 16 sequences
    "gret_3b_bf16": Workload(7, "gret_3b_bf16", "bf16", 1, 4096, 3072, 24, 24, 128,
                             8, 0, 0, 0.0, decode_steps=64),
}


def seed_for(workload_id: int, tensor_index: int) -> int:
    return 1000 * workload_id + tensor_index


_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def randn(shape, seed: int, std: float = 1.0, dtype: str = "bf16",
          device: Optional[str] = None) -> torch.Tensor:
    """Seeded N(0, std) tensor rounded to ``dtype`` ("f32" or "bf16")."""
    device = device or "cpu"
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(_DTYPES[dtype])
