"""Seeded synthetic inputs for the DiT denoiser hot path.

This package is shared by the CPU oracle (``oracle/``) and by the HIP path
(``diffusion_transformer_denoising_dit_amd``).  It holds workload shapes and
random-number draws only: no step of the method's arithmetic lives here.

Every tensor is produced as bfloat16 bit patterns (``numpy.uint16``) so that
both sides consume identical bits; the oracle widens them exactly to fp64, the
GPU side views them as ``torch.bfloat16``.
"""

from .configs import CONFIGS, BlockShape, AttnShape, LoopShape, get_config
from .gen import (
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    block_inputs,
    attention_inputs,
    loop_inputs,
    seed_sequence,
    normal_bf16,
)

__all__ = [
    "CONFIGS",
    "BlockShape",
    "AttnShape",
    "LoopShape",
    "get_config",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "block_inputs",
    "attention_inputs",
    "loop_inputs",
    "seed_sequence",
    "normal_bf16",
]
