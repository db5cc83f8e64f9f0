"""Pins of the oracle's denoising step (CPU only): brute force on tiny
shapes, closed forms of the sampler and properties that hold at any size."""

import numpy as np
import pytest

import oracle as O
from synthetic import configs as C
from synthetic import gen as G
from tests import brute


def _tiny(cfg, depth=2, seed=91):
    blk = C.BlockShape("tiny_step", batch=2, grid=(1, 2, 2), n_txt=3, heads=2, head_dim=4, mlp=8,
                       rope=(0, 2, 2), txt_valid=("fixed", (1, 3)), seed=seed)
    return C.LoopShape("tiny_step_loop", block=blk, depth=depth, steps=3, guidance=3.0,
                       latent_channels=4, freq_dim=8, seed=seed, cfg=cfg)


class _Model:
    """Oracle-facing view of LoopInputs with optional overrides."""

    def __init__(self, shape, **over):
        self.inputs = G.loop_inputs(shape)
        self.shape = shape
        self.over = over
        for n in ("t_w1", "t_b1", "t_w2", "t_b2", "in_w", "in_b", "fin_mod_w", "fin_mod_b",
                  "out_w", "out_b", "text", "txt_valid"):
            setattr(self, n, over.get(n, getattr(self.inputs, n)))

    def layer(self, l):
        w = self.inputs.layer(l)
        if self.over.get("zero_gates"):
            D = self.shape.block.hidden
            for k in ("mod_w", "mod_b"):
                w[k] = w[k].copy()
                w[k][2 * D:3 * D] = 0
                w[k][5 * D:6 * D] = 0
        return w


def _to_lists(m):
    dec = lambda a: O.bf16_decode(a).tolist()
    M = {n: dec(getattr(m, n)) for n in ("t_w1", "t_b1", "t_w2", "t_b2", "in_w", "in_b",
                                         "fin_mod_w", "fin_mod_b", "out_w", "out_b", "text")}
    M["layers"] = [{k: dec(v) for k, v in m.layer(l).items()} for l in range(m.shape.depth)]
    M["txt_valid"] = [int(v) for v in m.txt_valid]
    M["shape"] = m.shape
    return M


@pytest.mark.parametrize("cfg", [True, False])
def test_step_brute_force_tiny(cfg):
    shape = _tiny(cfg)
    m = _Model(shape)
    Bl = 1 if cfg else shape.block.batch
    lat = O.bf16_decode(G.normal_bf16(5, (Bl, shape.block.n_vis, 4)))
    sig, nxt = 0.75, 0.5  # exact in fp32
    got, _ = O.denoise_step(m, lat, sig, nxt, 3.0, round_points=False)
    want = np.array(brute.step(_to_lists(m), lat.tolist(), sig, nxt, 3.0))
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_step_constant_velocity_and_guidance_independence():
    shape = _tiny(True)
    C_ = shape.latent_channels
    const = G.normal_bf16(7, (C_,))
    m = _Model(shape, out_w=np.zeros((C_, shape.block.hidden), np.uint16), out_b=const)
    lat = O.bf16_decode(G.normal_bf16(6, (1, shape.block.n_vis, C_)))
    a, v = O.denoise_step(m, lat, 0.5, 0.25, 3.0)
    b, _ = O.denoise_step(m, lat, 0.5, 0.25, 9.0)
    np.testing.assert_array_equal(a, b)  # equal branches: guidance has no effect
    np.testing.assert_allclose(a, lat - 0.25 * O.bf16_decode(const), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(v, np.broadcast_to(O.bf16_decode(const), v.shape))


def test_step_zero_gates_make_blocks_identity():
    shape = _tiny(True, depth=3)
    m = _Model(shape, zero_gates=True)
    m0 = _Model(C.LoopShape("glue_only", block=shape.block, depth=0, steps=3, guidance=3.0,
                            latent_channels=4, freq_dim=8, seed=shape.seed, cfg=True))
    lat = O.bf16_decode(G.normal_bf16(8, (1, shape.block.n_vis, 4)))
    a, _ = O.denoise_step(m, lat, 0.9, 0.8, 3.0)
    b, _ = O.denoise_step(m0, lat, 0.9, 0.8, 3.0)
    np.testing.assert_array_equal(a, b)


def test_step_row_subset_exact_for_one_block():
    shape = C.LoopShape("sub", block=C.C1.__class__(**{**C.C1.__dict__, "batch": 2,
                                                          "txt_valid": ("fixed", (20, 9))}),
                        depth=1, steps=30, guidance=5.0, latent_channels=64, seed=12)
    m = _Model(shape)
    lat = O.bf16_decode(G.normal_bf16(9, (1, shape.block.n_vis, 64)))
    full, _ = O.denoise_step(m, lat, 0.6, 0.6 - 1 / 30, 5.0)
    rows = np.array([0, 3, 100, 200, 255, 256, 270])
    sub, _ = O.denoise_step(m, lat, 0.6, 0.6 - 1 / 30, 5.0, rows=rows)
    np.testing.assert_array_equal(sub, full[:, rows[rows < 256]])
