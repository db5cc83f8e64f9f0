"""Pins of the oracle's Wan-style block ("ChunkFlow" Appendix B, equations
(7)-(12): self-attention, text cross-attention, MLP) against independent
statements: a pure-Python token-by-token loop on tiny shapes; reduction to
the (separately pinned) DiT block on the video tokens alone when the
cross-attention adds nothing (zero output projection, or no valid context
token and zero bias); invariance to the padded context tokens' content;
identity under zero gates and zero cross projection; exact row subsets."""

import numpy as np
import pytest

import oracle as O
from oracle import wan as W
from synthetic import configs as C
from synthetic import gen as G
from tests import brute

TINY = C.BlockShape("wan_tiny", batch=2, grid=(1, 2, 3), n_txt=4, heads=2, head_dim=4, mlp=8,
                    rope=(0, 2, 2), txt_valid=("fixed", (1, 4)), seed=81)
SMALL = C.BlockShape("wan_small", batch=2, grid=(2, 3, 4), n_txt=9, heads=2, head_dim=8, mlp=24,
                     rope=(2, 2, 4), txt_valid=("fixed", (6, 9)), seed=82)

SELF_AND_MLP = ("w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "w_up", "b_up", "w_dn", "b_dn")


def _f(a):
    return O.bf16_decode(a)


def _dit_block_on_video(inp, s):
    """The DiT block of dit.block_forward on the video tokens alone."""
    vs = C.BlockShape(s.name + "_video_only", batch=s.batch, grid=s.grid, n_txt=0, heads=s.heads,
                      head_dim=s.head_dim, mlp=s.mlp, rope=s.rope, txt_valid=("fixed", (0,) * s.batch))
    blk = {k: inp[k] for k in SELF_AND_MLP}
    blk["x"], blk["mod"], blk["txt_valid"] = inp["x"], inp["mod"], np.zeros(s.batch, np.int32)
    return O.block_forward(blk, vs, round_points=False)


def test_wan_block_brute_force_tiny():
    s = TINY
    inp = G.wan_block_inputs(s)
    got = W.wan_block_forward(inp, s, round_points=False)
    Wl = {k: _f(v).tolist() for k, v in inp.items() if k.startswith(("w_", "b_", "g_"))}
    want = brute.wan_block(_f(inp["x"]).tolist(), _f(inp["ctx"]).tolist(), _f(inp["mod"]).tolist(),
                           Wl, s, inp["txt_valid"])
    np.testing.assert_allclose(got, np.array(want), rtol=1e-10, atol=1e-12)


def test_zero_cross_projection_is_the_dit_block_on_video_tokens():
    s = SMALL
    inp = G.wan_block_inputs(s)
    inp["w_co"] = np.zeros_like(_f(inp["w_co"]))
    inp["b_co"] = np.zeros_like(_f(inp["b_co"]))
    np.testing.assert_allclose(W.wan_block_forward(inp, s, round_points=False),
                               _dit_block_on_video(inp, s), rtol=1e-11, atol=1e-12)


def test_empty_context_row_adds_only_the_bias():
    """txt_valid[b] = 0: the cross-attention output is the empty sum, so with
    b_co = 0 batch row b equals the DiT block on its video tokens, while the
    other row (valid context) differs."""
    s = SMALL
    inp = G.wan_block_inputs(s)
    inp["txt_valid"] = np.array([0, 9], dtype=np.int32)
    inp["b_co"] = np.zeros_like(_f(inp["b_co"]))
    got = W.wan_block_forward(inp, s, round_points=False)
    ref = _dit_block_on_video(inp, s)
    np.testing.assert_allclose(got[0], ref[0], rtol=1e-11, atol=1e-12)
    assert np.abs(got[1] - ref[1]).max() > 1e-3


def test_padded_context_is_ignored():
    s = SMALL
    inp = G.wan_block_inputs(s)
    inp["txt_valid"] = np.array([3, 7], dtype=np.int32)
    base = W.wan_block_forward(inp, s)
    ctx = _f(inp["ctx"]).copy()
    rng = np.random.default_rng(9)
    for b, L in enumerate(inp["txt_valid"]):
        ctx[b, L:] = rng.standard_normal(ctx[b, L:].shape) * 100
    inp["ctx"] = ctx
    np.testing.assert_array_equal(W.wan_block_forward(inp, s), base)


def test_zero_gates_and_cross_projection_are_identity():
    s = SMALL
    inp = G.wan_block_inputs(s)
    m = _f(inp["mod"]).copy()
    m[:, 2] = 0
    m[:, 5] = 0
    inp["mod"] = m
    inp["w_co"] = np.zeros_like(_f(inp["w_co"]))
    inp["b_co"] = np.zeros_like(_f(inp["b_co"]))
    np.testing.assert_array_equal(W.wan_block_forward(inp, s), _f(inp["x"]))


def test_row_subsets_are_exact():
    s = SMALL
    inp = G.wan_block_inputs(s)
    rows = np.array([0, 7, 11, 12, 23])
    np.testing.assert_allclose(W.wan_block_forward(inp, s, rows=rows),
                               W.wan_block_forward(inp, s)[:, rows], rtol=1e-12, atol=1e-13)
