"""Workload shapes for the DiT denoiser hot path.

Shapes follow the image and video workloads the pages describe: FLUX-like
1024x1024 images (4.1k visual tokens) and Wan-like 81-frame videos at 480p and
720p (32.8k and 75.6k visual tokens), each joined by a fixed-capacity text
sequence whose tail is padding ("Difflet", section 4.2 Representing Attention
Mask; "ChunkFlow", Appendix C Table 2).  The latent grid is the VAE latent
(8x spatial, 4x temporal downsampling, 16 channels) after patchification.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class AttnShape:
    """Joint attention over [visual; text] tokens for every batch row."""

    name: str
    batch: int
    n_vis: int
    n_txt: int
    heads: int
    head_dim: int
    # ("fixed", (L_0, L_1, ...)) or ("uniform", lo, hi) inclusive, drawn per row
    txt_valid: tuple = ("fixed", ())
    seed: int = 0

    @property
    def n_tok(self) -> int:
        return self.n_vis + self.n_txt

    @property
    def hidden(self) -> int:
        return self.heads * self.head_dim


@dataclass(frozen=True)
class BlockShape:
    """One DiT block: adaLN, QKV, Q/K RMSNorm + RoPE, joint attention,
    output projection, gated residual, GELU MLP, gated residual."""

    name: str
    batch: int
    grid: Tuple[int, int, int]  # latent grid (t, h, w) after patchify
    n_txt: int
    heads: int
    head_dim: int
    mlp: int
    rope: Tuple[int, int, int]  # dims given to the (t, h, w) axes, sum == head_dim
    txt_valid: tuple = ("fixed", ())
    rope_theta: float = 10000.0
    ln_eps: float = 1e-6
    rms_eps: float = 1e-6
    seed: int = 0

    @property
    def n_vis(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def n_tok(self) -> int:
        return self.n_vis + self.n_txt

    @property
    def hidden(self) -> int:
        return self.heads * self.head_dim

    def attn(self) -> AttnShape:
        return AttnShape(self.name, self.batch, self.n_vis, self.n_txt, self.heads,
                         self.head_dim, self.txt_valid, self.seed)


@dataclass(frozen=True)
class LoopShape:
    """A stack of DiT blocks driven by a flow-matching Euler sampler with
    classifier-free guidance (conditional and unconditional rows stacked as
    batch 2)."""

    name: str
    block: BlockShape
    depth: int
    steps: int
    guidance: float
    latent_channels: int  # per visual token after patchify (16 ch x 2 x 2)
    freq_dim: int = 256  # sinusoidal timestep features
    seed: int = 0
    cfg: bool = True  # batch rows (conditional, unconditional) share one latent


C1 = BlockShape("c1_tiny", batch=1, grid=(1, 16, 16), n_txt=32, heads=4, head_dim=64,
                mlp=1024, rope=(0, 32, 32), txt_valid=("fixed", (20,)), seed=1)
C2 = BlockShape("c2_image", batch=2, grid=(1, 64, 64), n_txt=512, heads=24, head_dim=128,
                mlp=12288, rope=(0, 64, 64), txt_valid=("uniform", 77, 512), seed=2)
C3 = BlockShape("c3_video480", batch=1, grid=(21, 30, 52), n_txt=512, heads=40,
                head_dim=128, mlp=13824, rope=(44, 42, 42), txt_valid=("fixed", (226,)),
                seed=3)
C4 = AttnShape("c4_video720_attn", batch=1, n_vis=21 * 45 * 80, n_txt=512, heads=40,
               head_dim=128, txt_valid=("fixed", (300,)), seed=4)
C5 = LoopShape("c5_image_loop", block=BlockShape(
    "c5_block", batch=2, grid=(1, 64, 64), n_txt=512, heads=24, head_dim=128, mlp=12288,
    rope=(0, 64, 64), txt_valid=("uniform", 77, 512), seed=5),
    depth=24, steps=30, guidance=5.0, latent_channels=64, seed=5)

# One denoising step of a single-block video DiT at the c3 shape (no guidance):
# the step the benchmark times.
C3_STEP = LoopShape("c3_step", block=C3, depth=1, steps=30, guidance=1.0, latent_channels=64,
                    seed=3, cfg=False)
# c5 with a single block: row subsets stay exact, so the full-size step can be
# checked on sampled visual rows.
C5_DEPTH1 = LoopShape("c5_depth1", block=C5.block, depth=1, steps=30, guidance=5.0,
                      latent_channels=64, seed=5)
# A small stack the oracle can run through all 30 steps.
TINY_LOOP = LoopShape("tiny_loop", block=BlockShape(
    "tiny_loop_block", batch=2, grid=(1, 8, 8), n_txt=24, heads=2, head_dim=64, mlp=256,
    rope=(0, 32, 32), txt_valid=("fixed", (10, 3)), seed=6),
    depth=2, steps=30, guidance=5.0, latent_channels=64, seed=6)

CONFIGS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}


def get_config(key: str):
    return CONFIGS[key]
