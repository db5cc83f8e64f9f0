"""Write the oracle's first denoising step of the full c5 model (expected
values for a GPU parity test).  Calls only ``oracle`` and ``synthetic``.

The model: 24 live DiT blocks at the FLUX-like image shape (hidden 3072,
24 heads x 128, MLP 12288, 4096 visual + 512 text tokens, valid text lengths
drawn per CFG row), random N(0, 0.02) weights, classifier-free guidance with
g = 5 over the stacked (conditional, unconditional) rows, the flow-matching
Euler step from sigma_0 = 1 to sigma_1 = 29/30 ("Difflet", section 3 Model
Pipelines; "19. Diffusion, Image, Video, and World Models", Follow the
diffusion pipeline).  The initial latent is the seeded N(0, 1) bf16 draw of
the loop inputs.

Three oracle evaluations of the same step are stored (velocity per CFG row,
[2, 4096, 64]):

* ``v_ref``   fp64 between bf16 rounding points at every place the GPU path
              stores bf16 (the reference; its values are bf16, kept as bits);
* ``v_exact`` fp64 without rounding (float32 storage, for the spread);
* ``v_twin``  fp32 between the same rounding points (bf16 bits), the second
              correct evaluation the composite tolerance is derived from.

The new latent is not stored: the test recomputes it from the stored
velocities with the oracle's guidance and Euler formulas.

    python tests/golden/make_c5_step0.py      (about 15 CPU-minutes)
"""

from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from synthetic import configs as C  # noqa: E402
from synthetic import gen as G  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c5_step0.npz")


def bf16_bits(a):
    """Exact bf16 values (fp64) -> their bit patterns."""
    f = np.asarray(a, np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(a, np.float64)), "not bf16 values"
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def main():
    shape = C.C5
    model = G.loop_inputs(shape)  # exposes shape, glue weights, text, txt_valid, layer(l)
    lat0 = O.bf16_decode(model.latent)[None]  # [1, n_vis, C]
    sig = O.sigma_schedule(shape.steps)
    out = {}
    for mode, round_points, arith in (("ref", True, np.float64), ("exact", False, np.float64),
                                      ("twin", True, np.float32)):
        t0 = time.time()
        with O.arithmetic(arith):
            _, v = O.denoise_step(model, lat0, sig[0], sig[1], shape.guidance,
                                  round_points=round_points)
        v = np.asarray(v, np.float64)
        out["v_" + mode] = v.astype(np.float32) if mode == "exact" else bf16_bits(v)
        print(f"{mode}: {time.time() - t0:.0f} s, max|v| {np.abs(v).max():.3f}", flush=True)
    np.savez_compressed(OUT, sigma=sig[0], sigma_next=sig[1], guidance=shape.guidance,
                        txt_valid=np.asarray(model.txt_valid), **out)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
