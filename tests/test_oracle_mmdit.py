"""Pins of the oracle's MM-DiT blocks ("ChunkFlow" Appendix B: double-stream
and single-stream blocks) against independent statements of them: pure-Python
token-by-token loops on tiny shapes, reduction to the (separately pinned) DiT
block when the two streams share weights and modulation, reduction of the
single-stream block's fused linears to the DiT block's attention and MLP
halves, zero gates, exact row subsets, and invariance to the padded text
tokens' content."""

import numpy as np
import pytest

import oracle as O
from oracle import mmdit as M
from synthetic import configs as C
from synthetic import gen as G
from tests import brute

TINY = C.BlockShape("mmdit_tiny", batch=2, grid=(1, 2, 2), n_txt=3, heads=2, head_dim=4, mlp=8,
                    rope=(0, 2, 2), txt_valid=("fixed", (1, 3)), seed=61)
SMALL = C.BlockShape("mmdit_small", batch=2, grid=(2, 3, 4), n_txt=7, heads=2, head_dim=8,
                     mlp=24, rope=(2, 2, 4), txt_valid=("fixed", (0, 5)), seed=62)


def _f(a):
    return O.bf16_decode(a)


def _lists(a):
    return _f(a).tolist()


def _wl(w):
    return {k: _lists(v) for k, v in w.items()}


def test_double_block_brute_force_tiny():
    s = TINY
    inp = G.double_block_inputs(s)
    gi, gt = M.double_block_forward(inp, s, round_points=False)
    bi, bt = brute.double_block(_lists(inp["x_img"]), _lists(inp["x_txt"]), _lists(inp["mod_img"]),
                                _lists(inp["mod_txt"]), _wl(inp["w_img"]), _wl(inp["w_txt"]), s,
                                inp["txt_valid"])
    np.testing.assert_allclose(gi, np.array(bi), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(gt, np.array(bt), rtol=1e-10, atol=1e-12)


def test_single_block_brute_force_tiny():
    s = TINY
    inp = G.single_block_inputs(s)
    got = M.single_block_forward(inp, s, round_points=False)
    want = brute.single_block(_lists(inp["x"]), _lists(inp["mod"]),
                              {k: _lists(inp[k]) for k in ("w1", "b1", "g_q", "g_k", "w2", "b2")}, s,
                              inp["txt_valid"])
    np.testing.assert_allclose(got, np.array(want), rtol=1e-10, atol=1e-12)


def test_double_block_with_shared_weights_is_the_dit_block():
    """Equal weights and modulation on both streams: the double-stream block
    is the joint DiT block on the concatenated sequence."""
    s = SMALL
    inp = G.double_block_inputs(s)
    inp["w_txt"] = inp["w_img"]
    inp["mod_txt"] = inp["mod_img"]
    gi, gt = M.double_block_forward(inp, s, round_points=False)
    blk = dict(inp["w_img"])
    blk["x"] = np.concatenate([_f(inp["x_img"]), _f(inp["x_txt"])], axis=1)
    blk["mod"] = _f(inp["mod_img"])
    blk["txt_valid"] = inp["txt_valid"]
    want = O.block_forward(blk, s, round_points=False)
    np.testing.assert_allclose(np.concatenate([gi, gt], axis=1), want, rtol=1e-11, atol=1e-12)


def test_single_block_halves_are_the_dit_block_halves():
    """linear2 = [W_o | 0]: the block is the DiT block with gate2 = 0 (its
    attention half); linear2 = [0 | W_dn]: the DiT block with gate1 = 0 and
    the second adaLN on the unchanged stream (its MLP half).  Pins the column
    split of linear1 and the concatenation order of linear2."""
    s = SMALL
    D, F = s.hidden, s.mlp
    inp = G.single_block_inputs(s)
    w1, b1, w2 = _f(inp["w1"]), _f(inp["b1"]), _f(inp["w2"])
    mod3 = _f(inp["mod"])
    blk = {"w_qkv": w1[:3 * D], "b_qkv": b1[:3 * D], "g_q": _f(inp["g_q"]), "g_k": _f(inp["g_k"]),
           "w_o": w2[:, :D], "b_o": _f(inp["b2"]), "w_up": w1[3 * D:], "b_up": b1[3 * D:],
           "w_dn": w2[:, D:], "b_dn": _f(inp["b2"]), "x": _f(inp["x"]),
           "txt_valid": inp["txt_valid"]}
    z = np.zeros_like(mod3[:, 0])
    sh, sc, g = mod3[:, 0], mod3[:, 1], mod3[:, 2]
    # attention half
    a = dict(inp)
    a["w2"] = np.concatenate([w2[:, :D], np.zeros((D, F))], axis=1)
    blk["mod"] = np.stack([sh, sc, g, z, z, z], axis=1)
    np.testing.assert_allclose(M.single_block_forward(a, s, round_points=False),
                               O.block_forward(blk, s, round_points=False), rtol=1e-11, atol=1e-12)
    # MLP half
    m = dict(inp)
    m["w2"] = np.concatenate([np.zeros((D, D)), w2[:, D:]], axis=1)
    blk["mod"] = np.stack([z, z, z, sh, sc, g], axis=1)
    np.testing.assert_allclose(M.single_block_forward(m, s, round_points=False),
                               O.block_forward(blk, s, round_points=False), rtol=1e-11, atol=1e-12)


def test_zero_gates_are_identity():
    s = SMALL
    inp = G.double_block_inputs(s)
    for k in ("mod_img", "mod_txt"):
        m = _f(inp[k]).copy()
        m[:, 2] = 0
        m[:, 5] = 0
        inp[k] = m
    gi, gt = M.double_block_forward(inp, s)
    np.testing.assert_array_equal(gi, _f(inp["x_img"]))
    np.testing.assert_array_equal(gt, _f(inp["x_txt"]))
    sinp = G.single_block_inputs(s)
    m = _f(sinp["mod"]).copy()
    m[:, 2] = 0
    sinp["mod"] = m
    np.testing.assert_array_equal(M.single_block_forward(sinp, s), _f(sinp["x"]))


@pytest.mark.parametrize("kind", ["double", "single"])
def test_row_subsets_are_exact(kind):
    s = SMALL
    rows = np.array([0, 5, 23, 24, 26, 30])  # image rows, the seam, text rows
    if kind == "double":
        inp = G.double_block_inputs(s)
        fi, ft = M.double_block_forward(inp, s)
        ri, rt = M.double_block_forward(inp, s, rows=rows)
        np.testing.assert_allclose(ri, fi[:, rows[rows < s.n_vis]], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(rt, ft[:, rows[rows >= s.n_vis] - s.n_vis], rtol=1e-12, atol=1e-13)
    else:
        inp = G.single_block_inputs(s)
        full = M.single_block_forward(inp, s)
        np.testing.assert_allclose(M.single_block_forward(inp, s, rows=rows), full[:, rows],
                                   rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kind", ["double", "single"])
def test_padded_text_content_is_ignored_by_image_rows(kind):
    """Padded text tokens are never keys: any content there leaves every
    image row and every valid text row unchanged."""
    s = SMALL
    rng = np.random.default_rng(5)
    if kind == "double":
        inp = G.double_block_inputs(s)
        gi, gt = M.double_block_forward(inp, s)
        x = _f(inp["x_txt"]).copy()
        for b, L in enumerate(inp["txt_valid"]):
            x[b, L:] = rng.standard_normal(x[b, L:].shape) * 50
        inp["x_txt"] = x
        hi, ht = M.double_block_forward(inp, s)
        np.testing.assert_array_equal(hi, gi)
        for b, L in enumerate(inp["txt_valid"]):
            np.testing.assert_array_equal(ht[b, :L], gt[b, :L])
    else:
        inp = G.single_block_inputs(s)
        full = M.single_block_forward(inp, s)
        x = _f(inp["x"]).copy()
        for b, L in enumerate(inp["txt_valid"]):
            x[b, s.n_vis + L:] = rng.standard_normal(x[b, s.n_vis + L:].shape) * 50
        inp["x"] = x
        new = M.single_block_forward(inp, s)
        for b, L in enumerate(inp["txt_valid"]):
            np.testing.assert_array_equal(new[b, :s.n_vis + L], full[b, :s.n_vis + L])
