"""Seeded generators of bfloat16 inputs (bit patterns) for the DiT hot path.

Recipe (identical for the oracle and the HIP path):

* one ``numpy.random.SeedSequence(0xD17 + shape.seed)`` per workload, spawned
  into one child stream per tensor in a fixed order;
* activations, Q/K/V, the modulation vector and the initial latent are
  N(0, 1); weights and biases are N(0, 0.02); RMSNorm gains are 1 + N(0, 0.02);
* every draw is made in float32 and rounded to bfloat16 (round to nearest,
  ties to even);
* text valid lengths are fixed per workload or drawn uniformly per batch row
  from an inclusive integer range.

Draws are made in chunks from one generator per tensor, which yields the same
stream as a single call, so the values do not depend on the chunk size.
"""

from __future__ import annotations

import numpy as np

from .configs import AttnShape, BlockShape, LoopShape

_ROOT = 0xD17
_CHUNK = 1 << 24


def seed_sequence(seed: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(_ROOT + int(seed))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (NaN kept quiet)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(ss: np.random.SeedSequence, shape, std: float = 1.0,
                 mean: float = 0.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(ss))
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        z = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            z *= np.float32(std)
        if mean != 0.0:
            z += np.float32(mean)
        out[s:e] = f32_to_bf16_bits(z)
    return out.reshape(shape)


def normal_bf16(seed: int, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """A seeded N(mean, std^2) tensor of bf16 bit patterns (one stream per seed)."""
    return _normal_bf16(seed_sequence(seed), shape, std, mean)


def _valid_lengths(ss: np.random.SeedSequence, spec: tuple, batch: int,
                   n_txt: int) -> np.ndarray:
    kind = spec[0]
    if kind == "fixed":
        vals = list(spec[1])
        if len(vals) == 1 and batch > 1:
            vals = vals * batch
        if len(vals) != batch:
            raise ValueError(f"fixed valid lengths {vals} do not match batch {batch}")
        out = np.asarray(vals, dtype=np.int32)
    elif kind == "uniform":
        lo, hi = int(spec[1]), int(spec[2])
        rng = np.random.Generator(np.random.PCG64(ss))
        out = rng.integers(lo, hi + 1, size=batch, dtype=np.int64).astype(np.int32)
    else:
        raise ValueError(f"unknown valid-length spec {spec!r}")
    if (out < 0).any() or (out > n_txt).any():
        raise ValueError(f"valid lengths {out} outside [0, {n_txt}]")
    return out


_BLOCK_ORDER = ("x", "mod", "w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o",
                "w_up", "b_up", "w_dn", "b_dn", "txt_valid")


def block_weights(children, D: int, F: int) -> dict:
    """Weights of one block from its per-tensor seed streams (weights are
    [out, in], the input dimension contiguous)."""
    c = dict(zip(_BLOCK_ORDER, children))
    return {
        "w_qkv": _normal_bf16(c["w_qkv"], (3 * D, D), 0.02),
        "b_qkv": _normal_bf16(c["b_qkv"], (3 * D,), 0.02),
        "g_q": _normal_bf16(c["g_q"], (D,), 0.02, 1.0),
        "g_k": _normal_bf16(c["g_k"], (D,), 0.02, 1.0),
        "w_o": _normal_bf16(c["w_o"], (D, D), 0.02),
        "b_o": _normal_bf16(c["b_o"], (D,), 0.02),
        "w_up": _normal_bf16(c["w_up"], (F, D), 0.02),
        "b_up": _normal_bf16(c["b_up"], (F,), 0.02),
        "w_dn": _normal_bf16(c["w_dn"], (D, F), 0.02),
        "b_dn": _normal_bf16(c["b_dn"], (D,), 0.02),
    }


def block_inputs(shape: BlockShape, weights: bool = True) -> dict:
    """x [B, N, D], mod [B, 6, D] (shift1, scale1, gate1, shift2, scale2,
    gate2), the block weights and txt_valid [B] (int32)."""
    B, N, D, F = shape.batch, shape.n_tok, shape.hidden, shape.mlp
    children = seed_sequence(shape.seed).spawn(len(_BLOCK_ORDER))
    c = dict(zip(_BLOCK_ORDER, children))
    out = {
        "x": _normal_bf16(c["x"], (B, N, D)),
        "mod": _normal_bf16(c["mod"], (B, 6, D)),
        "txt_valid": _valid_lengths(c["txt_valid"], shape.txt_valid, B, shape.n_txt),
    }
    if weights:
        out.update(block_weights(children, D, F))
    return out


def attention_inputs(shape: AttnShape, q_scale: float = 1.0) -> dict:
    """q, k, v as [B, N, H*d] bf16 (token-major, heads then head_dim), N(0, 1)
    (q optionally N(0, q_scale^2) for peaked softmax rows) and txt_valid [B]."""
    B, N, HD = shape.batch, shape.n_tok, shape.hidden
    cq, ck, cv, cl = seed_sequence(shape.seed).spawn(4)
    return {
        "q": _normal_bf16(cq, (B, N, HD), q_scale),
        "k": _normal_bf16(ck, (B, N, HD)),
        "v": _normal_bf16(cv, (B, N, HD)),
        "txt_valid": _valid_lengths(cl, shape.txt_valid, B, shape.n_txt),
    }


class LoopInputs:
    """Inputs of the denoising loop.  Per-layer weights are drawn on demand
    from a seed stream keyed by the layer index, so a caller can hold one
    layer at a time."""

    _ORDER = ("latent", "text", "t_w1", "t_b1", "t_w2", "t_b2", "in_w", "in_b",
              "fin_mod_w", "fin_mod_b", "out_w", "out_b", "txt_valid")

    def __init__(self, shape: LoopShape):
        self.shape = shape
        blk = shape.block
        D, C, Fq = blk.hidden, shape.latent_channels, shape.freq_dim
        self._root = seed_sequence(shape.seed)
        ch = dict(zip(self._ORDER, self._root.spawn(len(self._ORDER))))
        B = blk.batch
        self.latent = _normal_bf16(ch["latent"], (blk.n_vis, C))
        self.text = _normal_bf16(ch["text"], (B, blk.n_txt, D))
        self.t_w1 = _normal_bf16(ch["t_w1"], (D, Fq), 0.02)
        self.t_b1 = _normal_bf16(ch["t_b1"], (D,), 0.02)
        self.t_w2 = _normal_bf16(ch["t_w2"], (D, D), 0.02)
        self.t_b2 = _normal_bf16(ch["t_b2"], (D,), 0.02)
        self.in_w = _normal_bf16(ch["in_w"], (D, C), 0.02)
        self.in_b = _normal_bf16(ch["in_b"], (D,), 0.02)
        self.fin_mod_w = _normal_bf16(ch["fin_mod_w"], (2 * D, D), 0.02)
        self.fin_mod_b = _normal_bf16(ch["fin_mod_b"], (2 * D,), 0.02)
        self.out_w = _normal_bf16(ch["out_w"], (C, D), 0.02)
        self.out_b = _normal_bf16(ch["out_b"], (C,), 0.02)
        self.txt_valid = _valid_lengths(ch["txt_valid"], blk.txt_valid, B, blk.n_txt)

    def layer(self, idx: int) -> dict:
        """Block weights of layer ``idx`` plus its modulation projection
        mod_w [6D, D], mod_b [6D]."""
        blk = self.shape.block
        D, F = blk.hidden, blk.mlp
        ss = np.random.SeedSequence(self._root.entropy, spawn_key=(1000 + int(idx),))
        children = ss.spawn(len(_BLOCK_ORDER) + 2)
        w = block_weights(children[:len(_BLOCK_ORDER)], D, F)
        w["mod_w"] = _normal_bf16(children[-2], (6 * D, D), 0.02)
        w["mod_b"] = _normal_bf16(children[-1], (6 * D,), 0.02)
        return w


def loop_inputs(shape: LoopShape) -> LoopInputs:
    return LoopInputs(shape)


def double_block_inputs(shape: BlockShape) -> dict:
    """Inputs of an MM-DiT double-stream block: the image stream x_img
    [B, n_vis, D], the text stream x_txt [B, n_txt, D], one modulation set per
    stream (mod_img, mod_txt [B, 6, D]), one weight set per stream (w_img,
    w_txt; the DiT block's names and distributions) and txt_valid [B]."""
    B, S, L, D, F = shape.batch, shape.n_vis, shape.n_txt, shape.hidden, shape.mlp
    c = seed_sequence(shape.seed).spawn(6)
    img_w = c[4].spawn(len(_BLOCK_ORDER))
    txt_w = c[5].spawn(len(_BLOCK_ORDER))
    mod_img, mod_txt = c[2].spawn(2)
    return {
        "x_img": _normal_bf16(c[0], (B, S, D)),
        "x_txt": _normal_bf16(c[1], (B, L, D)),
        "mod_img": _normal_bf16(mod_img, (B, 6, D)),
        "mod_txt": _normal_bf16(mod_txt, (B, 6, D)),
        "txt_valid": _valid_lengths(c[3], shape.txt_valid, B, L),
        "w_img": block_weights(img_w, D, F),
        "w_txt": block_weights(txt_w, D, F),
    }


def single_block_inputs(shape: BlockShape) -> dict:
    """Inputs of an MM-DiT single-stream block: the joint stream x [B, N, D],
    mod [B, 3, D] (shift, scale, gate), the fused linears w1 [3D + F, D], b1,
    w2 [D, D + F], b2 (N(0, 0.02)), the Q/K RMSNorm gains g_q, g_k
    (1 + N(0, 0.02)) and txt_valid [B]."""
    B, N, D, F = shape.batch, shape.n_tok, shape.hidden, shape.mlp
    c = seed_sequence(shape.seed).spawn(9)
    return {
        "x": _normal_bf16(c[0], (B, N, D)),
        "mod": _normal_bf16(c[1], (B, 3, D)),
        "w1": _normal_bf16(c[2], (3 * D + F, D), 0.02),
        "b1": _normal_bf16(c[3], (3 * D + F,), 0.02),
        "g_q": _normal_bf16(c[4], (D,), 0.02, 1.0),
        "g_k": _normal_bf16(c[5], (D,), 0.02, 1.0),
        "w2": _normal_bf16(c[6], (D, D + F), 0.02),
        "b2": _normal_bf16(c[7], (D,), 0.02),
        "txt_valid": _valid_lengths(c[8], shape.txt_valid, B, shape.n_txt),
    }


_WAN_ORDER = ("x", "ctx", "mod", "txt_valid", "w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o",
              "w_cq", "b_cq", "w_ckv", "b_ckv", "g_cq", "g_ck", "w_co", "b_co",
              "w_up", "b_up", "w_dn", "b_dn")


def wan_block_inputs(shape: BlockShape) -> dict:
    """Inputs of a Wan-style block: video tokens x [B, n_vis, D], text context
    ctx [B, n_txt, D] (N(0, 1)), mod [B, 6, D], txt_valid [B] and the weights
    of its self-attention (w_qkv, b_qkv, g_q, g_k, w_o, b_o), cross-attention
    (w_cq [D, D], b_cq, w_ckv [2D, D], b_ckv, g_cq, g_ck, w_co [D, D], b_co)
    and MLP (w_up, b_up, w_dn, b_dn); weights and biases N(0, 0.02), gains
    1 + N(0, 0.02)."""
    B, S, L, D, F = shape.batch, shape.n_vis, shape.n_txt, shape.hidden, shape.mlp
    c = dict(zip(_WAN_ORDER, seed_sequence(shape.seed).spawn(len(_WAN_ORDER))))
    shapes = {"w_qkv": (3 * D, D), "b_qkv": (3 * D,), "w_o": (D, D), "b_o": (D,),
              "w_cq": (D, D), "b_cq": (D,), "w_ckv": (2 * D, D), "b_ckv": (2 * D,),
              "w_co": (D, D), "b_co": (D,), "w_up": (F, D), "b_up": (F,), "w_dn": (D, F),
              "b_dn": (D,)}
    out = {
        "x": _normal_bf16(c["x"], (B, S, D)),
        "ctx": _normal_bf16(c["ctx"], (B, L, D)),
        "mod": _normal_bf16(c["mod"], (B, 6, D)),
        "txt_valid": _valid_lengths(c["txt_valid"], shape.txt_valid, B, L),
    }
    for k, shp in shapes.items():
        out[k] = _normal_bf16(c[k], shp, 0.02)
    for k in ("g_q", "g_k", "g_cq", "g_ck"):
        out[k] = _normal_bf16(c[k], (D,), 0.02, 1.0)
    return out
