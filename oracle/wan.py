"""A Wan-style DiT block written out as plain fp64 formulas (test
infrastructure only; see the package docstring).

Source: "ChunkFlow" Appendix B, Per-Block Compute Model: DiT and MM-DiT,
equations (7)-(12): a standard DiT block runs, one after the other,
self-attention over the video tokens (QKV and output projections), a
cross-attention from the video tokens to the text context (video-side query
and output projections, text-side key/value projections) and an MLP.

Readings taken where the page leaves a point open (each also listed with the
design notes):

* The self-attention half and the MLP are modulated and gated as in the DiT
  block of ``dit.block_forward`` (shift1, scale1, gate1, shift2, scale2,
  gate2); the self-attention sees the video tokens only, with Q/K RMSNorm over
  the full hidden width and 3D RoPE at each token's grid position.
* The cross-attention reads a plain LayerNorm of the stream (no affine, no
  modulation) and adds its output without a gate:
  x += CrossAttn(LN(x), ctx) with q = RMSNorm_D(LN(x) W_cq^T + b_cq) g_cq,
  [k | v] = ctx W_ckv^T + b_ckv, k normalised the same way with g_ck, no RoPE
  on either side; the keys of batch row b are the valid context tokens
  [0, txt_valid[b]) (the interval mask of "Difflet" section 4.2).  A row with
  no valid context token gets a zero attention output (the empty sum).
* bf16 rounding points as on the GPU: every adaLN/LayerNorm output, every
  projection the GPU stores in bf16 (self q|k|v, cross q, cross k|v), the
  normalised q^/k^, both attention outputs and the MLP hidden; the residual
  stream stays unrounded.
"""

from __future__ import annotations

import numpy as np

from .dit import (_dec, _f, adaln_modulate, gelu_erf, joint_attention, linear, rms_norm_full,
                  rope_axial, _rounder, token_positions)


def wan_block_forward(inp, shape, round_points=True, rows=None):
    """One Wan-style block on the video tokens x [B, S, D] (S = n_vis) with the
    text context ctx [B, L, D] (L = n_txt slots, txt_valid[b] of them valid).

    ``inp``: x, ctx, mod [B, 6, D], txt_valid [B] and the weights w_qkv
    [3D, D], b_qkv, g_q, g_k, w_o [D, D], b_o (self-attention); w_cq [D, D],
    b_cq, w_ckv [2D, D] (key rows, then value rows), b_ckv, g_cq, g_ck, w_co
    [D, D], b_co (cross-attention); w_up [F, D], b_up, w_dn [D, F], b_dn:

      h  = adaLN(x; shift1, scale1)
      x1 = x + gate1 (SelfAttn(h) W_o^T + b_o)
      x2 = x1 + CrossAttn(LN(x1), ctx) W_co^T + b_co
      x3 = x2 + gate2 (GELU(adaLN(x2; shift2, scale2) W_up^T + b_up) W_dn^T + b_dn)

    ``rows`` restricts the output to a subset of video tokens (exact: self
    keys/values use every token, cross keys/values come from the context).
    Returns x3 [B, R, D]."""
    R_ = _rounder(round_points)
    B, S, L, D = shape.batch, shape.n_vis, shape.n_txt, shape.hidden
    H, d = shape.heads, shape.head_dim
    x = _dec(inp["x"]).reshape(B, S, D)
    ctx = _dec(inp["ctx"]).reshape(B, L, D)
    mod = _dec(inp["mod"]).reshape(B, 6, D)
    shift1, scale1, gate1, shift2, scale2, gate2 = (mod[:, i][:, None, :] for i in range(6))
    W = {k: _dec(v) for k, v in inp.items() if k.startswith(("w_", "b_", "g_"))}
    valid = np.asarray(inp["txt_valid"], dtype=np.int64)
    pos = token_positions(shape.grid, 0)
    sel = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)

    def heads(t):
        return t.reshape(B, t.shape[1], H, d)

    # self-attention over the video tokens
    h = R_(adaln_modulate(x, shift1, scale1, shape.ln_eps))
    kv = R_(linear(h, W["w_qkv"][D:], W["b_qkv"][D:]))
    k_hat = R_(rope_axial(heads(rms_norm_full(kv[..., :D], W["g_k"], shape.rms_eps)), pos,
                          shape.rope, shape.rope_theta))
    v = heads(kv[..., D:])
    q = R_(linear(h[:, sel], W["w_qkv"][:D], W["b_qkv"][:D]))
    q_hat = R_(rope_axial(heads(rms_norm_full(q, W["g_q"], shape.rms_eps)), pos[sel], shape.rope,
                          shape.rope_theta))
    o, _ = joint_attention(q_hat, k_hat, v, S, np.zeros(B, dtype=np.int64))
    x1 = x[:, sel] + gate1 * linear(R_(o.reshape(B, len(sel), D)), W["w_o"], W["b_o"])

    # cross-attention to the valid context tokens
    zero = _f(np.zeros((1, 1, D)))
    hc = R_(adaln_modulate(x1, zero, zero, shape.ln_eps))
    qc = R_(heads(rms_norm_full(R_(linear(hc, W["w_cq"], W["b_cq"])), W["g_cq"], shape.rms_eps)))
    kvc = R_(linear(ctx, W["w_ckv"], W["b_ckv"]))
    kc = R_(heads(rms_norm_full(kvc[..., :D], W["g_ck"], shape.rms_eps)))
    vc = heads(kvc[..., D:])
    oc = np.zeros_like(qc)
    for b in range(B):
        if valid[b] > 0:
            ob, _ = joint_attention(qc[b:b + 1], kc[b:b + 1], vc[b:b + 1], 0, valid[b:b + 1])
            oc[b] = ob[0]
    x2 = x1 + linear(R_(oc.reshape(B, len(sel), D)), W["w_co"], W["b_co"])

    # MLP
    h2 = R_(adaln_modulate(x2, shift2, scale2, shape.ln_eps))
    u = R_(gelu_erf(linear(h2, W["w_up"], W["b_up"])))
    return x2 + gate2 * linear(u, W["w_dn"], W["b_dn"])
