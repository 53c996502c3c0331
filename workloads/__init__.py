"""Seeded synthetic inputs for paged MLA decode.

This package only draws and lays out inputs: sequence lengths, the physical
page pool and its permutation, the block table, and bf16 query / latent-cache
bits.  It holds none of the attention arithmetic, so both the CPU oracle and
the HIP path may take their inputs from it.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    DecodeCase,
    CaseSpec,
    bf16_bits_from_f32,
    make_case,
    make_config_case,
    HEAD_DIM,
    V_DIM,
    PAGE,
    AbsorbCase,
    make_absorb_case,
    NOPE_DIM,
    ROPE_DIM,
    AppendCase,
    make_append_case,
    PrefillCase,
    make_prefill_case,
)
