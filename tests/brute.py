"""Plain-Python (list and math) statements of the DiT block and of one
denoising step, for brute-force pins of the oracle on tiny shapes.  Written
from the step list, independently of oracle/ (no numpy arithmetic)."""

import math


def lin(row, W, bias):
    return [bias[o] + sum(row[c] * W[o][c] for c in range(len(row))) for o in range(len(W))]


def silu(z):
    return z / (1.0 + math.exp(-z))


def ln_mod(row, sh, sc, eps):
    D = len(row)
    mu = sum(row) / D
    var = sum((r - mu) ** 2 for r in row) / D
    return [(row[c] - mu) / math.sqrt(var + eps) * (1 + sc[c]) + sh[c] for c in range(D)]


def block(x, mod, W, s, valid):
    """x: [B][N][D] floats; mod: [B][6][D]; W: dict of nested float lists."""
    B, N, D, H, d = s.batch, s.n_tok, s.hidden, s.heads, s.head_dim
    T_, Hg, Wg = s.grid

    def pos_of(i):
        if i >= s.n_vis:
            return (0, 0, 0)
        return (i // (Hg * Wg), (i // Wg) % Hg, i % Wg)

    def rms_rope(vec, g, p):
        r = math.sqrt(sum(t * t for t in vec) / D + s.rms_eps)
        v = [vec[c] / r * g[c] for c in range(D)]
        out = list(v)
        for h in range(H):
            off = h * d
            for a, da in enumerate(s.rope):
                for j in range(da // 2):
                    ang = p[a] * s.rope_theta ** (-2.0 * j / da)
                    i0 = off + 2 * j
                    out[i0] = v[i0] * math.cos(ang) - v[i0 + 1] * math.sin(ang)
                    out[i0 + 1] = v[i0] * math.sin(ang) + v[i0 + 1] * math.cos(ang)
                off += da
        return out

    res = []
    for b in range(B):
        mb = mod[b]
        qs, ks, vs = [], [], []
        for i in range(N):
            h = ln_mod(x[b][i], mb[0], mb[1], s.ln_eps)
            qkv = lin(h, W["w_qkv"], W["b_qkv"])
            qs.append(rms_rope(qkv[:D], W["g_q"], pos_of(i)))
            ks.append(rms_rope(qkv[D:2 * D], W["g_k"], pos_of(i)))
            vs.append(qkv[2 * D:])
        nk = s.n_vis + int(valid[b])
        rows = []
        for i in range(N):
            o = [0.0] * D
            for h in range(H):
                sc = [sum(qs[i][h * d + c] * ks[j][h * d + c] for c in range(d)) / math.sqrt(d)
                      for j in range(nk)]
                m = max(sc)
                e = [math.exp(t - m) for t in sc]
                z = sum(e)
                for c in range(d):
                    o[h * d + c] = sum(e[j] / z * vs[j][h * d + c] for j in range(nk))
            y = lin(o, W["w_o"], W["b_o"])
            x1 = [x[b][i][c] + mb[2][c] * y[c] for c in range(D)]
            h2 = ln_mod(x1, mb[3], mb[4], s.ln_eps)
            u = [z_ * 0.5 * (1 + math.erf(z_ / math.sqrt(2))) for z_ in lin(h2, W["w_up"], W["b_up"])]
            y2 = lin(u, W["w_dn"], W["b_dn"])
            rows.append([x1[c] + mb[5][c] * y2[c] for c in range(D)])
        res.append(rows)
    return res


def step(M, latent, sigma, sigma_next, guidance, t_scale=1000.0):
    """M: dict of nested float lists (glue weights, text, layers, txt_valid)
    plus 'shape'; latent: [Bl][n_vis][C].  Returns the new latent."""
    shp = M["shape"]
    s = shp.block
    B, nv, D = s.batch, s.n_vis, s.hidden
    half = shp.freq_dim // 2
    t = t_scale * sigma
    f = [math.cos(t * 10000.0 ** (-j / half)) for j in range(half)] + \
        [math.sin(t * 10000.0 ** (-j / half)) for j in range(half)]
    c = [silu(z) for z in lin(f, M["t_w1"], M["t_b1"])]
    sv = [silu(z) for z in lin(c, M["t_w2"], M["t_b2"])]
    x = []
    for b in range(B):
        lb = 0 if shp.cfg else b
        rows = [lin(latent[lb][i], M["in_w"], M["in_b"]) for i in range(nv)]
        rows += [list(r) for r in M["text"][b]]
        x.append(rows)
    for L in M["layers"]:
        m6 = lin(sv, L["mod_w"], L["mod_b"])
        mod = [[m6[k * D:(k + 1) * D] for k in range(6)] for _ in range(B)]
        x = block(x, mod, L, s, M["txt_valid"])
    fin = lin(sv, M["fin_mod_w"], M["fin_mod_b"])
    v = [[lin(ln_mod(x[b][i], fin[:D], fin[D:], s.ln_eps), M["out_w"], M["out_b"])
          for i in range(nv)] for b in range(B)]
    dt = sigma_next - sigma
    if shp.cfg:
        return [[[latent[0][i][c] + dt * (v[1][i][c] + guidance * (v[0][i][c] - v[1][i][c]))
                  for c in range(len(v[0][i]))] for i in range(nv)]]
    return [[[latent[b][i][c] + dt * v[b][i][c] for c in range(len(v[b][i]))] for i in range(nv)]
            for b in range(B)]


def _pos_fn(s):
    T_, Hg, Wg = s.grid

    def pos_of(i):
        if i >= s.n_vis:
            return (0, 0, 0)
        return (i // (Hg * Wg), (i // Wg) % Hg, i % Wg)
    return pos_of


def _rms_rope(vec, g, p, s):
    D, H, d = s.hidden, s.heads, s.head_dim
    r = math.sqrt(sum(t * t for t in vec) / D + s.rms_eps)
    v = [vec[c] / r * g[c] for c in range(D)]
    out = list(v)
    for h in range(H):
        off = h * d
        for a, da in enumerate(s.rope):
            for j in range(da // 2):
                ang = p[a] * s.rope_theta ** (-2.0 * j / da)
                i0 = off + 2 * j
                out[i0] = v[i0] * math.cos(ang) - v[i0 + 1] * math.sin(ang)
                out[i0 + 1] = v[i0] * math.sin(ang) + v[i0 + 1] * math.cos(ang)
            off += da
    return out


def _attend(q, ks, vs, nk, s):
    D, H, d = s.hidden, s.heads, s.head_dim
    o = [0.0] * D
    for h in range(H):
        sc = [sum(q[h * d + c] * ks[j][h * d + c] for c in range(d)) / math.sqrt(d) for j in range(nk)]
        m = max(sc)
        e = [math.exp(t - m) for t in sc]
        z = sum(e)
        for c in range(d):
            o[h * d + c] = sum(e[j] / z * vs[j][h * d + c] for j in range(nk))
    return o


def _gelu(z):
    return z * 0.5 * (1 + math.erf(z / math.sqrt(2)))


def double_block(x_img, x_txt, mod_img, mod_txt, W_img, W_txt, s, valid):
    """MM-DiT double-stream block, one token at a time: per-stream adaLN,
    QKV, RMSNorm + RoPE, one attention over [image; valid text] keys, then
    per-stream output projection, gated residual and gated GELU MLP."""
    B, S, L, D = s.batch, s.n_vis, s.n_txt, s.hidden
    pos_of = _pos_fn(s)
    out_img, out_txt = [], []
    for b in range(B):
        toks = [(x_img[b][i], mod_img[b], W_img) for i in range(S)] + \
               [(x_txt[b][i], mod_txt[b], W_txt) for i in range(L)]
        qs, ks, vs = [], [], []
        for i, (xr, mb, W) in enumerate(toks):
            h = ln_mod(xr, mb[0], mb[1], s.ln_eps)
            qkv = lin(h, W["w_qkv"], W["b_qkv"])
            qs.append(_rms_rope(qkv[:D], W["g_q"], pos_of(i), s))
            ks.append(_rms_rope(qkv[D:2 * D], W["g_k"], pos_of(i), s))
            vs.append(qkv[2 * D:])
        nk = S + int(valid[b])
        rows = []
        for i, (xr, mb, W) in enumerate(toks):
            o = _attend(qs[i], ks, vs, nk, s)
            y = lin(o, W["w_o"], W["b_o"])
            x1 = [xr[c] + mb[2][c] * y[c] for c in range(D)]
            h2 = ln_mod(x1, mb[3], mb[4], s.ln_eps)
            u = [_gelu(z) for z in lin(h2, W["w_up"], W["b_up"])]
            y2 = lin(u, W["w_dn"], W["b_dn"])
            rows.append([x1[c] + mb[5][c] * y2[c] for c in range(D)])
        out_img.append(rows[:S])
        out_txt.append(rows[S:])
    return out_img, out_txt


def single_block(x, mod, W, s, valid):
    """MM-DiT single-stream block, one token at a time: adaLN, linear1 split
    into q | k | v | up, RMSNorm + RoPE, attention, GELU(up), linear2 on
    [o | GELU(up)], gated residual."""
    B, N, D = s.batch, s.n_tok, s.hidden
    pos_of = _pos_fn(s)
    res = []
    for b in range(B):
        mb = mod[b]
        hs, qs, ks, vs, ups = [], [], [], [], []
        for i in range(N):
            h = ln_mod(x[b][i], mb[0], mb[1], s.ln_eps)
            y1 = lin(h, W["w1"], W["b1"])
            qs.append(_rms_rope(y1[:D], W["g_q"], pos_of(i), s))
            ks.append(_rms_rope(y1[D:2 * D], W["g_k"], pos_of(i), s))
            vs.append(y1[2 * D:3 * D])
            ups.append(y1[3 * D:])
        nk = s.n_vis + int(valid[b])
        rows = []
        for i in range(N):
            o = _attend(qs[i], ks, vs, nk, s)
            y2 = lin(o + [_gelu(z) for z in ups[i]], W["w2"], W["b2"])
            rows.append([x[b][i][c] + mb[2][c] * y2[c] for c in range(D)])
        res.append(rows)
    return res


def wan_block(x, ctx, mod, W, s, valid):
    """Wan-style block, one token at a time: adaLN + self-attention over the
    video tokens (RMSNorm + RoPE), gated residual; plain LayerNorm +
    cross-attention to the valid context tokens (RMSNorm, no RoPE), residual;
    adaLN + GELU MLP, gated residual."""
    B, S, L, D = s.batch, s.n_vis, s.n_txt, s.hidden
    pos_of = _pos_fn(s)
    zeros = [0.0] * D
    res = []
    for b in range(B):
        mb = mod[b]
        qs, ks, vs = [], [], []
        for i in range(S):
            h = ln_mod(x[b][i], mb[0], mb[1], s.ln_eps)
            qkv = lin(h, W["w_qkv"], W["b_qkv"])
            qs.append(_rms_rope(qkv[:D], W["g_q"], pos_of(i), s))
            ks.append(_rms_rope(qkv[D:2 * D], W["g_k"], pos_of(i), s))
            vs.append(qkv[2 * D:])
        kc, vc = [], []
        for j in range(L):
            kv = lin(ctx[b][j], W["w_ckv"], W["b_ckv"])
            kc.append(_rms_rope(kv[:D], W["g_ck"], (0, 0, 0), s))
            vc.append(kv[D:])
        rows = []
        for i in range(S):
            o = _attend(qs[i], ks, vs, S, s)
            y = lin(o, W["w_o"], W["b_o"])
            x1 = [x[b][i][c] + mb[2][c] * y[c] for c in range(D)]
            hc = ln_mod(x1, zeros, zeros, s.ln_eps)
            qc = _rms_rope(lin(hc, W["w_cq"], W["b_cq"]), W["g_cq"], (0, 0, 0), s)
            oc = _attend(qc, kc, vc, int(valid[b]), s) if int(valid[b]) > 0 else [0.0] * D
            yc = lin(oc, W["w_co"], W["b_co"])
            x2 = [x1[c] + yc[c] for c in range(D)]
            h2 = ln_mod(x2, mb[3], mb[4], s.ln_eps)
            u = [_gelu(z) for z in lin(h2, W["w_up"], W["b_up"])]
            y2 = lin(u, W["w_dn"], W["b_dn"])
            rows.append([x2[c] + mb[5][c] * y2[c] for c in range(D)])
        res.append(rows)
    return res
