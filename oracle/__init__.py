"""Plain fp64 CPU oracle for nanochat's attention hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the package
``transformer_attention_06_amd`` and its HIP library) imports, calls, links or
executes anything in this directory. The only callers are ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``.

The oracle is numpy float64 throughout and imports neither torch nor the GPU
binding. Every function computes the plain mathematical definition of its
step (dense masked score matrices, explicit softmax, explicit chain rule);
the tiled / online-softmax / split-K / recompute-from-LSE schemes of the GPU
path reach the same result up to rounding and are not reproduced here.

Sources (titles and sections of the pages this follows):
  * "nanochat Admin & Developer Guide", section 3 "The GPT Model (Internals)":
    RoPE with base 100000, weightless QK RMSNorm, grouped-query attention,
    the SSSL sliding-window pattern; section 6 "Attention: FA3 with SDPA
    Fallback" (GQA via repeat-interleave of KV heads, single-token decode
    slicing the key window); section 7 "The Inference Engine & Tool Use",
    "KV cache" (cache layout (B, T, H, D) per layer, int32 per-row lengths,
    in-place cache update, batch-1 prefill replicated to the sample rows).
  * "nanochat (Fucina port)", "Architecture": no-weight RMSNorm, half-split
    RoPE built from an inverse-frequency table, grouped causal attention.
  * "nanochat Admin & Developer Guide", section 5 "Precision: Explicit dtype
    & FP8" (float8 e4m3 operands with tensorwise dynamic scaling) for the
    fp8 forward in fp8.py.

Parity pins for every function live in tests/test_oracle.py (closed forms,
invariants, brute force, finite differences and torch fp64 library
cross-checks). No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    visible_mask,
    kv_head_of,
    attn_probs,
    attn_fwd,
    attn_bwd,
    decode,
)
from .prologue import (  # noqa: F401
    inv_freq,
    rope_angles,
    rms_norm,
    rope_rotate,
    positions_from_offsets,
    qk_prologue_fwd,
    qk_prologue_bwd,
)
from .engine import (  # noqa: F401
    round_to,
    decode_step,
    kv_cache_replicate,
    cache_append,
    prefill_chunk,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_value,
    e4m3_decode,
    e4m3_encode,
    tensorwise_descale,
    quantize_tensorwise,
    attn_fwd_fp8,
)
