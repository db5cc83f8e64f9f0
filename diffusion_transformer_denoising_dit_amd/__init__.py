"""MI355X-native (gfx950) DiT denoiser hot path.

The compute lives in ``libdit.so`` (hand-written HIP kernels behind the C ABI
of ``include/dit.h``); this package only loads it and marshals arguments.
"""

from ._lib import (  # noqa: F401
    DIT_MAX_BATCH,
    EPI_BF16,
    EPI_F32,
    EPI_GATED_RES_F32,
    EPI_GELU_BF16,
    EPI_SILU_BF16,
    EXPORTED,
    LIB_PATH,
    AttnDesc,
    BlockDesc,
    BlockWeights,
    DitError,
    LinearArgs,
    attn_desc,
    block_desc,
    block_weights,
    dit_adaln_modulate,
    dit_block_forward,
    dit_block_workspace_bytes,
    dit_cast_bf16_f32,
    dit_cast_f32_bf16,
    dit_debug_positions,
    dit_euler_step,
    dit_joint_attention,
    dit_linear,
    dit_qk_rmsnorm_rope,
    dit_timestep_features,
    dit_version,
    lib,
    ModelDesc,
    ModelWeights,
    model_desc,
    model_weights,
    dit_denoise_step,
    dit_denoise_workspace_bytes,
)
