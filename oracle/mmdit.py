"""MM-DiT blocks written out as plain fp64 formulas (test infrastructure only;
see the package docstring).

Source: "ChunkFlow" Appendix B, Per-Block Compute Model: DiT and MM-DiT.

* Double-stream block (equations (13)-(18)): the image and the text stream
  keep their own weights for the QKV projection, the output projection and
  the FFN; the two streams are concatenated along the token dimension for one
  joint attention and split again afterwards.
* Single-stream block (equations (19)-(22)): image and text tokens form one
  stream; one fused linear (linear1) yields QKV and the MLP up-projection, one
  fused linear (linear2) takes the attention output and the MLP hidden
  together and yields the block's update.

Readings taken where the page leaves a point open (each also listed with the
design notes):

* Both blocks are modulated like the DiT block of ``dit.block_forward``:
  adaLN (LayerNorm without affine, then (1 + scale), + shift) before each
  branch and a gate on each residual update.  The double-stream block has one
  set of six vectors (shift1, scale1, gate1, shift2, scale2, gate2) per
  stream; the single-stream block has three (shift, scale, gate).
* Q/K RMSNorm is over the full hidden width with per-stream gains (the image
  stream's g_q, g_k for image tokens, the text stream's for text tokens);
  RoPE as in the DiT block: image tokens at their (t, h, w) grid position,
  text tokens at position 0.
* The joint sequence is [image; text]; the keys of batch row b are the
  image tokens plus the first txt_valid[b] text tokens (the interval mask of
  "Difflet" section 4.2).
* The single-stream block's MLP activation is GELU (erf form), applied to the
  up-projection half of linear1 before linear2; linear2 reads
  [attention output | GELU(up)] in that column order.
* bf16 rounding points as on the GPU: the adaLN outputs, the QKV projection,
  q^ and k^, the attention output, the MLP hidden; the residual streams are
  never rounded.
"""

from __future__ import annotations

import numpy as np

from .dit import (_dec, adaln_modulate, gelu_erf, joint_attention, linear, rms_norm_full,
                  rope_axial, _rounder, token_positions)


def _norm_rope(t, gain, pos, shape):
    B, R = t.shape[:2]
    return rope_axial(rms_norm_full(t, _dec(gain), shape.rms_eps).reshape(B, R, shape.heads,
                                                                            shape.head_dim),
                      pos, shape.rope, shape.rope_theta)


def double_block_forward(inp, shape, round_points=True, rows=None):
    """One double-stream MM-DiT block.

    ``inp``: x_img [B, S, D], x_txt [B, L, D] (S = n_vis image tokens, L =
    n_txt text slots), mod_img and mod_txt [B, 6, D], w_img and w_txt (dicts
    with the DiT block's weight names: w_qkv, b_qkv, g_q, g_k, w_o, b_o, w_up,
    b_up, w_dn, b_dn), txt_valid [B].  ``rows`` restricts the output to token
    indices of the joint sequence [0, S + L) (keys and values still use every
    token, so the restricted result is exact).  Returns (x_img', x_txt') for
    the selected image rows and text rows (all rows when ``rows`` is None)."""
    R_ = _rounder(round_points)
    B, S, L, D = shape.batch, shape.n_vis, shape.n_txt, shape.hidden
    H, d = shape.heads, shape.head_dim
    xs = {"img": _dec(inp["x_img"]).reshape(B, S, D), "txt": _dec(inp["x_txt"]).reshape(B, L, D)}
    mods = {s: _dec(inp["mod_" + s]).reshape(B, 6, D) for s in ("img", "txt")}
    ws = {s: inp["w_" + s] for s in ("img", "txt")}
    pos = token_positions(shape.grid, L)
    pos_s = {"img": pos[:S], "txt": pos[S:]}
    valid = np.asarray(inp["txt_valid"], dtype=np.int64)

    def m(s, i):
        return mods[s][:, i][:, None, :]

    h = {s: R_(adaln_modulate(xs[s], m(s, 0), m(s, 1), shape.ln_eps)) for s in ("img", "txt")}
    k_hat, v = [], []
    for s in ("img", "txt"):
        w_qkv, b_qkv = _dec(ws[s]["w_qkv"]), _dec(ws[s]["b_qkv"])
        kv = R_(linear(h[s], w_qkv[D:], b_qkv[D:]))
        k_hat.append(R_(_norm_rope(kv[..., :D], ws[s]["g_k"], pos_s[s], shape)))
        v.append(kv[..., D:].reshape(B, -1, H, d))
    k_hat = np.concatenate(k_hat, axis=1)
    v = np.concatenate(v, axis=1)

    sel = np.arange(S + L) if rows is None else np.asarray(rows, dtype=np.int64)
    sel_s = {"img": sel[sel < S], "txt": sel[sel >= S] - S}
    out = {}
    for s in ("img", "txt"):
        r = sel_s[s]
        w = ws[s]
        w_qkv, b_qkv = _dec(w["w_qkv"]), _dec(w["b_qkv"])
        q = R_(linear(h[s][:, r], w_qkv[:D], b_qkv[:D]))
        q_hat = R_(_norm_rope(q, w["g_q"], pos_s[s][r], shape))
        o, _ = joint_attention(q_hat, k_hat, v, S, valid)
        o = R_(o.reshape(B, len(r), D))
        x1 = xs[s][:, r] + m(s, 2) * linear(o, _dec(w["w_o"]), _dec(w["b_o"]))
        h2 = R_(adaln_modulate(x1, m(s, 3), m(s, 4), shape.ln_eps))
        u = R_(gelu_erf(linear(h2, _dec(w["w_up"]), _dec(w["b_up"]))))
        out[s] = x1 + m(s, 5) * linear(u, _dec(w["w_dn"]), _dec(w["b_dn"]))
    return out["img"], out["txt"]


def single_block_forward(inp, shape, round_points=True, rows=None):
    """One single-stream MM-DiT block on the joint stream x [B, N, D]
    (N = n_vis + n_txt, image tokens first).

    ``inp``: x, mod [B, 3, D] (shift, scale, gate), w1 [3D + F, D], b1
    [3D + F], g_q, g_k [D], w2 [D, D + F], b2 [D], txt_valid [B]:

      h = adaLN(x; shift, scale)
      [q | k | v | up] = h w1^T + b1
      q^, k^ = RoPE(RMSNorm_D(q) g_q), RoPE(RMSNorm_D(k) g_k)
      o = JointAttention(q^, k^, v; n_vis + txt_valid[b])
      x' = x + gate * ([o | GELU(up)] w2^T + b2)

    ``rows`` restricts the output rows (exact, as in ``double_block_forward``)."""
    R_ = _rounder(round_points)
    B, N, D, F = shape.batch, shape.n_tok, shape.hidden, shape.mlp
    H, d = shape.heads, shape.head_dim
    x = _dec(inp["x"]).reshape(B, N, D)
    mod = _dec(inp["mod"]).reshape(B, 3, D)
    shift, scale, gate = (mod[:, i][:, None, :] for i in range(3))
    w1, b1 = _dec(inp["w1"]), _dec(inp["b1"])
    pos = token_positions(shape.grid, shape.n_txt)
    valid = np.asarray(inp["txt_valid"], dtype=np.int64)

    h = R_(adaln_modulate(x, shift, scale, shape.ln_eps))
    kv = R_(linear(h, w1[D:3 * D], b1[D:3 * D]))
    k_hat = R_(_norm_rope(kv[..., :D], inp["g_k"], pos, shape))
    v = kv[..., D:].reshape(B, N, H, d)
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    q = R_(linear(h[:, sel], w1[:D], b1[:D]))
    q_hat = R_(_norm_rope(q, inp["g_q"], pos[sel], shape))
    o, _ = joint_attention(q_hat, k_hat, v, shape.n_vis, valid)
    o = R_(o.reshape(B, len(sel), D))
    mlp = R_(gelu_erf(linear(h[:, sel], w1[3 * D:], b1[3 * D:])))
    y = linear(np.concatenate([o, mlp], axis=-1), _dec(inp["w2"]), _dec(inp["b2"]))
    return x[:, sel] + gate * y
