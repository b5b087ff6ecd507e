"""Seeded synthetic inputs for the ISD verify/propose step.

This package only draws random inputs (logits, proposals, uniforms, hidden
states and head weights) and encodes them as bf16/fp32 bytes.  It holds none
of the step's own arithmetic, so both the CPU oracle and the HIP path can
consume exactly the same bytes.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    gen_hidden,
    gen_head_weights,
    gen_sequence,
    gen_step,
    gen_uniforms,
    host_bytes_per_step,
)
from .lora import LORA_CONFIGS, extend_mask, gen_exact_head, gen_lora  # noqa: F401
