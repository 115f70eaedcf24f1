"""Seeded synthetic inputs for paged attention.

This package only draws and lays out inputs: sequence lengths, block tables,
slot mappings, and the raw bits of q/k/v.  It holds none of the attention
arithmetic, so both the CPU oracle and the HIP path can consume its output
without sharing any of the method's code.
"""

from .configs import (  # noqa: F401
    BLOCK_SIZE,
    CONFIG_NAMES,
    FP8_K_SCALE,
    FP8_POISON,
    FP8_V_SCALE,
    DecodeWorkload,
    PrefillWorkload,
    SpecVerifyWorkload,
    bf16_bits_from_f32,
    make_decode,
    make_mixed,
    make_prefill,
    make_spec_verify,
    make_tiny_decode,
    make_tiny_prefill,
    make_tiny_shared,
    poison_bits,
)
