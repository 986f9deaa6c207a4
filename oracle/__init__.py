"""Plain float64 CPU oracle for the YOCO shared-KV attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library under
``shared_kv_attention_amd/`` and its Python binding) imports, calls or links
anything here.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this package.

The oracle shares no code with the GPU path: no kernels, headers, helpers,
tables or constants.  It is numpy in float64, written row by row so that each
output row depends only on that row's own inputs; row-sampled comparisons are
therefore exact, and the method's invariants (causality, sharing, early exit)
hold bitwise inside the oracle.

Pages cited in this package (the method's only description here):
  [S] paperlayer.ai source-linked summary of "You Only Cache Once:
      Decoder-Decoder Architectures for Language Models" (arXiv 2405.05254v2),
      cited by its section (e.g. [S §2], [S §3 Sliding-Window Attention]).
  [P] podcast transcript "YOCO: caching once for decoder-decoder long-context
      language models" (do-not-panic.com episode of 2026-09-25), cited by
      subtitle segment (e.g. [P seg. 12]).
  [A] pith.science record of arXiv 2405.05254 (the paper's abstract).

Modules:
  attention   softmax attention over an explicit allowed-key set per row:
              sliding-window, causal cross prefill, single-query decode.
  projection  RMSNorm and the one-time global K/V projection.
  fp8         OCP fp8-e4m3fn codec and per-head KV quantisation.
  block       the tiny YOCO block (self-decoder, projection, cross-decoder)
              and its early-exit variant.
  retention   gated retention (recurrent, parallel, chunkwise) and its
              per-head GroupNorm with swish gate.
  memory      closed-form KV-cache sizes the pages reason with.
"""

from .attention import (  # noqa: F401
    attend_row,
    attention_rows,
    swa_attention,
    cross_prefill_attention,
    decode_attention,
    swa_allowed,
    causal_allowed,
    ring_window,
    swa_ring_decode_attention,
    merge_partial_attention,
)
from .projection import rmsnorm_row, rmsnorm, global_kv_proj  # noqa: F401
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    kv_fp8_scales,
    quantize_kv_fp8,
    encode_kv_fp8,
    dequantize_kv_fp8,
)
from .block import BlockParams, linear_rows, silu, swiglu_hidden_row, swiglu_ffn_row, yoco_block, yoco_block_early_exit, yoco_block_generate  # noqa: F401
from .memory import yoco_kv_cache_bytes, transformer_kv_cache_bytes  # noqa: F401
from .retention import (  # noqa: F401
    gret_log_decay,
    gret_recurrent,
    gret_parallel,
    gret_chunkwise,
    gret_group_norm_swish,
)
from .rope import rope_inv_freq, apply_rope  # noqa: F401,E402
