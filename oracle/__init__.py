"""CPU fp64 oracle for paged MLA decode -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the bench may
import or call anything in this package.  The product path (the HIP library
and its Python binding) never does, and shares no code with it.
"""

from .mla_oracle import (  # noqa: F401
    bf16_to_f64,
    visible_tokens,
    gather_latents,
    attend_f64,
    decode_ref,
    decode_ref_rows,
    decode_bruteforce,
    softmax_weights,
    explicit_heads,
    absorb_query,
    absorb_output,
    absorb_ref,
    attend_chunks_and_merge,
    merge_partials,
    kv_append_ref,
)
from . import fp8_cache  # noqa: F401
from . import prefill  # noqa: F401  (MLA prefill, per-head form)  (FP8 latent cache: format, quantize, dequantize)
