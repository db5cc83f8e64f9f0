"""How far apart two correct bf16-storing evaluations of a full-size DiT
block land: the fp64 oracle against the same formulas in fp32 between the
same bf16 rounding points (oracle.arithmetic).  This is the measurement the
composite tolerance of the GPU parity tests is built on (tests/gpu_util.py,
assert_composite).

At the c2 image shape and the c3 video shape, on the seeded row subsets the
GPU block tests compare, the two evaluations:

* agree to well inside the rel-L2 bar of 5e-3 (about 1.1e-3 measured);
* differ by more than 2e-2 in max-abs (0.053 at c2 over 113 rows, 0.078 at
  c3 over 75 rows, measured on this container): single one-ulp bf16 flips of
  the MLP hidden values, multiplied through W_dn and by gates up to |4|, on
  outputs that reach |x| ~ 30-40 where a bf16 ulp is already 0.125-0.25;
* are closer to each other than bf16 storage puts the oracle from its own
  unrounded evaluation (0.089 at c2).

The pages see the same effect between two correct bf16 parallelisations of
one DiT ("Difflet", section 7.4 Parallel Execution: max abs 7.8e-2 on
outputs up to 3.3).  BLAS in fp32 is not bit-reproducible across machines,
so the spread is asserted within a band, not to a fixed value.
"""

import numpy as np

import oracle as O
from synthetic import configs as C
from synthetic import gen as G
from tests.sampling import sample_rows


def _spread(shape, n_random, with_exact):
    inp = G.block_inputs(shape)
    rows = sample_rows(shape.n_vis, shape.n_txt, inp["txt_valid"], n_random=n_random,
                       seed=shape.seed)
    ref = O.block_forward(inp, shape, rows=rows)
    with O.arithmetic(np.float32):
        twin = O.block_forward(inp, shape, rows=rows)
    assert twin.dtype == np.float32
    twin = twin.astype(np.float64)
    d = np.abs(twin - ref)
    out = {"rows": len(rows), "max_abs": float(d.max()),
           "rel_l2": float(np.linalg.norm(twin - ref) / np.linalg.norm(ref)),
           "over": float((d > 2e-2).mean()), "max_ref": float(np.abs(ref).max())}
    if with_exact:
        exact = O.block_forward(inp, shape, rows=rows, round_points=False)
        out["exact_spread"] = float(np.abs(exact - ref).max())
    print(shape.name, out, flush=True)
    return out


def test_fp32_twin_spread_c2_block():
    s = _spread(C.C2, 64, with_exact=True)
    assert s["rows"] == 113
    assert s["rel_l2"] < 2e-3
    assert 0.03 < s["max_abs"] < 0.08
    assert s["over"] < 0.01
    assert s["max_abs"] < s["exact_spread"]


def test_fp32_twin_spread_c3_block():
    s = _spread(C.C3, 32, with_exact=False)
    assert s["rows"] == 75
    assert s["rel_l2"] < 2e-3
    assert 0.04 < s["max_abs"] < 0.12
    assert s["over"] < 0.02


def test_fp32_twin_is_a_second_evaluation_not_a_copy():
    """The twin really computes in fp32 (so it is a distinct evaluation) and
    is identical to the reference where no arithmetic happens between
    rounding points (gates zero: the block is the identity)."""
    inp = G.block_inputs(C.C1)
    with O.arithmetic(np.float32):
        twin = O.block_forward(inp, C.C1)
    ref = O.block_forward(inp, C.C1)
    assert twin.dtype == np.float32 and ref.dtype == np.float64
    assert 0 < np.abs(twin - ref).max() < 2e-2
    inp0 = dict(inp)
    inp0["mod"] = inp["mod"].copy()
    inp0["mod"][:, 2] = 0
    inp0["mod"][:, 5] = 0
    with O.arithmetic(np.float32):
        twin0 = O.block_forward(inp0, C.C1)
    np.testing.assert_array_equal(twin0.astype(np.float64), O.bf16_decode(inp["x"]))
