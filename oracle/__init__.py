"""CPU oracle for the DiT denoiser hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy statement of what one denoising step computes:
adaLN modulation, QKV projection, Q/K RMSNorm over the full hidden width,
axial RoPE, joint attention over [visual; valid text] keys with a materialised
softmax, output projection with a gated residual, a GELU MLP with a gated
residual, classifier-free guidance and the flow-matching Euler update; split
attention with a statistic merge; and step caching (``stepcache``: the skip
controller, the relative L1 change score, the output estimator and the
block-0 probe); and the MM-DiT double-stream and single-stream blocks
(``mmdit``); a Wan-style block with text cross-attention (``wan``).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It shares no code with the HIP path and never
imports it; the HIP path never imports it either.  The only module the two
have in common is ``synthetic`` (seeded input draws, no arithmetic of the
method).

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (closed forms, invariants, brute force on tiny inputs or an
independent library routine).  Nothing here is "parity unpinned".
"""

from .numerics import bf16_decode, round_bf16
from .dit import (
    adaln_modulate,
    linear,
    rms_norm_full,
    token_positions,
    rope_axial,
    attention_probs,
    joint_attention,
    attention_partial,
    merge_partials,
    gelu_erf,
    block_forward,
    cfg_combine,
    euler_update,
    sigma_schedule,
    timestep_features,
    silu,
    denoise_step,
    step_tokens,
    arithmetic,
)
from . import mmdit, stepcache, wan

__all__ = [
    "bf16_decode", "round_bf16", "adaln_modulate", "linear", "rms_norm_full",
    "token_positions", "rope_axial", "attention_probs", "attention_partial", "merge_partials", "joint_attention",
    "gelu_erf", "block_forward", "cfg_combine", "euler_update", "sigma_schedule",
    "timestep_features", "silu", "denoise_step", "arithmetic",
]
