"""The DiT denoiser step written out as plain fp64 formulas (test
infrastructure only; see the package docstring).

Sources (web pages; cited by title and section):

* "Difflet" paper (paperpeel.com/paper/2610.23047): section 1 Introduction and
  section 3 Model Pipelines (the denoiser predicts a velocity from latent,
  timestep and conditioning; the scheduler turns it into a less noisy
  latent), section 4 (joint attention: one softmax over visual and text
  keys), section 4.2 Representing Attention Mask (padded text keys placed
  after all valid keys, excluded by a contiguous [0, bound) interval).
* "Difflet Engineering Report: Diffusion Inference on AWS Trainium":
  "Terms used in this report" (AdaLN: LayerNorm whose scale and shift come
  from the timestep conditioning; UniPC state kept in fp32), "Wan attention
  head sharding and global RMS" (Q/K RMS over the whole projection, not per
  head shard), "Video output corrections" (scheduler state in fp32),
  "Attention CTE routing and mask representation" (only contiguous hard
  masks take the bounded path).
* "ChunkFlow" Appendix B, equations (13)-(17): a block's dominant work is the
  QKV and output projections, joint attention and the MLP.

Where the pages leave a step open, the plainest reading is taken and stated
in the docstring of the function that implements it.
"""

from __future__ import annotations

import contextlib
import math

import numpy as np
from scipy.special import erf

from .numerics import bf16_decode, round_bf16

# Working precision between the bfloat16 rounding points.  The oracle is fp64;
# ``arithmetic(np.float32)`` re-evaluates the same formulas with fp32 values
# between the same rounding points.  That second evaluation is an instrument
# for measuring how far two correct bf16-storing evaluations of a composite
# (a block, a step) can drift apart, which is what the composite tolerance is
# derived from; it is never the parity reference.
_ARITH = np.float64


@contextlib.contextmanager
def arithmetic(dtype):
    """Evaluate every oracle formula in ``dtype`` (np.float64 or np.float32)
    inside the ``with`` block; bfloat16 rounding points are unchanged."""
    global _ARITH
    if dtype not in (np.float64, np.float32):
        raise ValueError(f"unsupported working precision {dtype}")
    old, _ARITH = _ARITH, dtype
    try:
        yield
    finally:
        _ARITH = old


def _f(a):
    """``a`` as an array in the working precision (no copy when it already is)."""
    return np.asarray(a, dtype=_ARITH)


def _rounder(round_points):
    """The rounding applied at each bf16 storage point: round to the nearest
    bfloat16 (ties to even) and carry on in the working precision; identity
    for the unrounded evaluation."""
    if round_points:
        return lambda a: _f(round_bf16(a))
    return _f


# ----------------------------------------------------------------------------
# per-token steps
# ----------------------------------------------------------------------------

def adaln_modulate(x, shift, scale, eps):
    """Adaptive LayerNorm ("Difflet Engineering Report", Terms used in this
    report: AdaLN).  Normalise every token over the hidden width with the
    biased variance and no learned affine, then apply the timestep
    modulation as x_hat * (1 + scale) + shift.  ``shift`` and ``scale``
    broadcast against ``x`` (one vector per batch row)."""
    x = _f(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    x_hat = (x - mu) / np.sqrt(var + eps)
    return x_hat * (1.0 + scale) + shift


def linear(a, w, b=None):
    """y = a W^T + b with W stored [out, in] ("ChunkFlow" Appendix B, the
    projection and MLP terms of equations (13) and (16))."""
    y = _f(a) @ _f(w).T
    if b is not None:
        y = y + b
    return y


def rms_norm_full(q, gain, eps):
    """RMSNorm of a Q or K projection over its full width (all heads at once):
    q / sqrt(mean(q^2) + eps) * gain.  The pages require the sum of squares
    to cover the whole projection, not each head shard ("Difflet Engineering
    Report", Wan attention head sharding and global RMS)."""
    q = _f(q)
    ms = (q * q).mean(axis=-1, keepdims=True)
    return q / np.sqrt(ms + eps) * gain


def gelu_erf(z):
    """GELU in its exact form z * Phi(z) = z * (1 + erf(z / sqrt 2)) / 2.
    The pages name the MLP but not its activation; the erf form is taken."""
    z = _f(z)
    return z * 0.5 * (1.0 + erf(z / math.sqrt(2.0)))


def silu(z):
    z = _f(z)
    return z / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------
# positions and RoPE
# ----------------------------------------------------------------------------

def token_positions(grid, n_txt):
    """Integer (t, h, w) position of every token of the joint sequence
    [visual; text].  Visual token i of a (T, H, W) latent grid, row-major,
    sits at t = i // (H W), h = (i // W) mod H, w = i mod W.  Text tokens get
    position (0, 0, 0), so RoPE leaves them unrotated (the pages name image
    RoPE but do not define text positions; this is the reading taken)."""
    T, H, W = (int(g) for g in grid)
    i = np.arange(T * H * W, dtype=np.int64)
    vis = np.stack([i // (H * W), (i // W) % H, i % W], axis=1)
    txt = np.zeros((int(n_txt), 3), dtype=np.int64)
    return np.concatenate([vis, txt], axis=0)


def rope_axial(x, pos, dims, theta):
    """Axial rotary embedding on x [..., N, heads, d].

    The head dimension is split into consecutive blocks of dims = (d_t, d_h,
    d_w) for the three axes (a zero entry skips that axis).  Inside the block
    of axis a, the pair (2j, 2j+1) is rotated by the angle
    pos_a * theta**(-2j / d_a), j = 0 .. d_a/2 - 1:
    (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).
    Base theta, interleaved pairing and the block order are the reading taken
    (the pages only name RoPE)."""
    x = _f(x)
    pos = np.asarray(pos)
    d = x.shape[-1]
    pairs = x.reshape(x.shape[:-1] + (d // 2, 2))  # pair j of the head: dims (2j, 2j+1)
    out = np.empty_like(pairs)
    p0 = 0
    for axis, d_a in enumerate(dims):
        n_a = int(d_a) // 2
        if n_a == 0:
            continue
        j = np.arange(n_a, dtype=np.float64)
        inv_freq = float(theta) ** (-2.0 * j / int(d_a))
        ang = pos[:, axis].astype(np.float64)[:, None] * inv_freq[None, :]  # [N, d_a/2]
        c = _f(np.cos(ang))[:, None, :]  # [N, 1, d_a/2] broadcast over heads
        s = _f(np.sin(ang))[:, None, :]
        x0 = pairs[..., p0:p0 + n_a, 0]
        x1 = pairs[..., p0:p0 + n_a, 1]
        out[..., p0:p0 + n_a, 0] = x0 * c - x1 * s
        out[..., p0:p0 + n_a, 1] = x0 * s + x1 * c
        p0 += n_a
    out[..., p0:, :] = pairs[..., p0:, :]
    out = out.reshape(x.shape)
    return out


# ----------------------------------------------------------------------------
# joint attention
# ----------------------------------------------------------------------------

def attention_probs(q, k, n_keys_valid, scale):
    """Softmax weights of one (batch row, head): q [Nq, d], k [Nk, d].

    Scores s_ij = scale * q_i . k_j.  Keys j >= n_keys_valid are padding and
    get weight exactly 0; the valid keys form the interval [0, n_keys_valid)
    ("Difflet", section 4.2 Representing Attention Mask).  Every query row is
    normalised by one softmax over all its valid keys, visual and text
    together ("Difflet", section 4, joint attention)."""
    q = _f(q)
    k = _f(k)
    nv = int(n_keys_valid)
    s = (q @ k[:nv].T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = np.zeros((q.shape[0], k.shape[0]), dtype=_ARITH)
    p[:, :nv] = e / e.sum(axis=1, keepdims=True)
    lse = (m + np.log(e.sum(axis=1, keepdims=True)))[:, 0]
    return p, lse


def joint_attention(q, k, v, n_vis, txt_valid, scale=None, chunk=1024):
    """Joint attention over [visual; text] tokens.

    k, v: [B, N, heads, d] (N = n_vis + n_txt); row b's keys
    j < n_vis + txt_valid[b] are valid.  q: [B, R, heads, d] holds the query
    rows wanted -- all N of them (padded text rows included) or any subset:
    there is no positional mask, so every output row depends only on its own
    query and on all keys, and a subset is exact.  The default scale is
    1/sqrt(d).  Returns (o [B, R, heads, d], lse [B, heads, R]) where lse is
    the natural log of each row's softmax denominator (max included).
    """
    qsel = _f(q)
    k = _f(k)
    v = _f(v)
    B, N, Hh, d = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    R = qsel.shape[1]
    o = np.zeros((B, R, Hh, d), dtype=_ARITH)
    lse = np.zeros((B, Hh, R), dtype=_ARITH)
    for b in range(B):
        nk = int(n_vis) + int(txt_valid[b])
        for h in range(Hh):
            kh = k[b, :, h, :]
            vh = v[b, :, h, :]
            for r0 in range(0, R, chunk):
                r1 = min(R, r0 + chunk)
                p, l = attention_probs(qsel[b, r0:r1, h, :], kh, nk, scale)
                o[b, r0:r1, h, :] = p[:, :nk] @ vh[:nk]
                lse[b, h, r0:r1] = l
    return o, lse


def attention_partial(q, k, v, k_valid, scale):
    """One partial of split joint attention ("Difflet", section 4.3, Ring for
    joint attention): queries q [B, R, heads, d] against one key/value
    partition k, v [B, Nk, heads, d] whose valid keys of batch row b are the
    interval [0, k_valid[b]) in the partition's own coordinates (a text
    partial passes [0, L_text); a visual partition passes all its keys).

    Per query it returns what each partial call hands to the merge: the
    unnormalised weighted value sum  acc = sum_j exp(s_j - m) v_j,  the
    maximum score  m = max_j s_j  and the sum of exponentials relative to it
    l = sum_j exp(s_j - m), all over valid keys only, with s_j = scale q.k_j.
    A partition with no valid key returns acc = 0, m = -inf, l = 0.
    Shapes: acc [B, R, heads, d], m and l [B, heads, R]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, R, Hh, d = q.shape
    acc = np.zeros((B, R, Hh, d), dtype=np.float64)
    m = np.full((B, Hh, R), -np.inf, dtype=np.float64)
    l = np.zeros((B, Hh, R), dtype=np.float64)
    for b in range(B):
        nv = int(k_valid[b])
        if nv == 0:
            continue
        for h in range(Hh):
            s = (q[b, :, h, :] @ k[b, :nv, h, :].T) * scale
            mb = s.max(axis=1)
            e = np.exp(s - mb[:, None])
            acc[b, :, h, :] = e @ v[b, :nv, h, :]
            m[b, h] = mb
            l[b, h] = e.sum(axis=1)
    return acc, m, l


def merge_partials(parts):
    """Joint normalisation from independently computed partials ("Difflet",
    section 4.3): each partial (acc, m, l) of attention_partial uses its own
    maximum, so both sums are first rescaled to the common maximum
    M = max_p m_p, i.e. multiplied by exp(m_p - M), then added over the
    partials; the merged output is the combined weighted sum divided by the
    combined exponential sum.  Returns (o [B, R, heads, d], lse [B, heads, R])
    with lse = M + log(sum_p exp(m_p - M) l_p), the natural log of the joint
    softmax denominator.  A query whose partials are all empty (no valid key
    anywhere) gets the empty sum: o = 0 and lse = -inf, the same neutral
    element an empty partial is."""
    M = np.max(np.stack([m for _, m, _ in parts]), axis=0)
    num = 0.0
    den = 0.0
    for acc, m, l in parts:
        w = np.where(np.isfinite(m), np.exp(m - np.where(np.isfinite(M), M, 0.0)), 0.0)
        num = num + acc * np.transpose(w, (0, 2, 1))[..., None]
        den = den + w * l
    empty = den == 0.0  # [B, heads, R]
    safe = np.where(empty, 1.0, den)
    o = num / np.transpose(safe, (0, 2, 1))[..., None]
    o = np.where(np.transpose(empty, (0, 2, 1))[..., None], 0.0, o)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, M + np.log(safe))
    return o, lse


# ----------------------------------------------------------------------------
# the block
# ----------------------------------------------------------------------------

def _dec(a):
    return _f(bf16_decode(a) if np.asarray(a).dtype == np.uint16 else a)


def block_forward(inp, shape, round_points=True, rows=None, keep=False):
    """One DiT block on x [B, N, D] (N = visual then text tokens).

    Order of steps (a joint-attention block with adaLN modulation; the
    dominant work is equations (13) and (16) of "ChunkFlow" Appendix B, the
    attention is "Difflet" section 4 with the section 4.2 interval mask):

      h  = adaLN(x; shift1, scale1)
      q, k, v = split(h W_qkv^T + b_qkv)
      q^ = RoPE(RMSNorm_D(q) * g_q), k^ = RoPE(RMSNorm_D(k) * g_k)
      o  = JointAttention(q^, k^, v; n_vis + txt_valid[b])
      x1 = x + gate1 * (o W_o^T + b_o)
      h2 = adaLN(x1; shift2, scale2)
      u  = GELU(h2 W_up^T + b_up)
      x2 = x1 + gate2 * (u W_dn^T + b_dn)

    The modulation vector per batch row is (shift1, scale1, gate1, shift2,
    scale2, gate2), each of width D.  With ``round_points`` the value is
    rounded to bfloat16 wherever the GPU path stores bfloat16 (h, qkv, q^,
    k^, o, h2, u); everything between those points is fp64.  The residual
    stream x, x1, x2 is kept in full precision (fp32 on the GPU), so it is
    never rounded.

    ``rows`` restricts the output to a set of token indices (same for every
    batch row): only keys and values need every token, every other step is
    per token, so the restricted result is exact for those rows.
    Returns x2 [B, R, D] (and the intermediates when ``keep``).
    """
    R_ = _rounder(round_points)
    B, N, D = shape.batch, shape.n_tok, shape.hidden
    H, d = shape.heads, shape.head_dim
    x = _dec(inp["x"]).reshape(B, N, D)
    mod = _dec(inp["mod"]).reshape(B, 6, D)
    shift1, scale1, gate1, shift2, scale2, gate2 = (mod[:, i][:, None, :] for i in range(6))
    w_qkv, b_qkv = _dec(inp["w_qkv"]), _dec(inp["b_qkv"])
    valid = np.asarray(inp["txt_valid"], dtype=np.int64)
    pos = token_positions(shape.grid, shape.n_txt)

    h = R_(adaln_modulate(x, shift1, scale1, shape.ln_eps))
    # keys and values for every token
    kv = R_(linear(h, w_qkv[D:], b_qkv[D:]))
    k_raw, v = kv[..., :D], kv[..., D:]
    k_hat = R_(rope_axial(rms_norm_full(k_raw, _dec(inp["g_k"]), shape.rms_eps)
                          .reshape(B, N, H, d), pos, shape.rope, shape.rope_theta))
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    q_raw = R_(linear(h[:, sel], w_qkv[:D], b_qkv[:D]))
    q_hat = R_(rope_axial(rms_norm_full(q_raw, _dec(inp["g_q"]), shape.rms_eps)
                          .reshape(B, len(sel), H, d), pos[sel], shape.rope, shape.rope_theta))
    o, _ = joint_attention(q_hat, k_hat, v.reshape(B, N, H, d), shape.n_vis, valid)
    o = R_(o.reshape(B, len(sel), D))
    xs = x[:, sel]
    x1 = xs + gate1 * linear(o, _dec(inp["w_o"]), _dec(inp["b_o"]))
    h2 = R_(adaln_modulate(x1, shift2, scale2, shape.ln_eps))
    u = R_(gelu_erf(linear(h2, _dec(inp["w_up"]), _dec(inp["b_up"]))))
    x2 = x1 + gate2 * linear(u, _dec(inp["w_dn"]), _dec(inp["b_dn"]))
    if keep:
        return x2, {"h": h[:, sel], "q_hat": q_hat, "k_hat": k_hat, "v": v, "o": o,
                    "x1": x1, "h2": h2, "u": u, "qkv_q": q_raw, "k_raw": k_raw}
    return x2


# ----------------------------------------------------------------------------
# sampler
# ----------------------------------------------------------------------------

def sigma_schedule(steps):
    """Noise levels sigma_i = 1 - i/steps, i = 0..steps (a linear schedule from
    1 to 0; sigma = 0 is only ever a target, never evaluated)."""
    return 1.0 - np.arange(steps + 1, dtype=np.float64) / steps


def cfg_combine(v_cond, v_uncond, guidance):
    """Classifier-free guidance, applied once to the two predictions
    ("Difflet Engineering Report", CFG parallelism applies the guidance
    combination once): v_uncond + g (v_cond - v_uncond)."""
    v_cond = _f(v_cond)
    v_uncond = _f(v_uncond)
    return v_uncond + guidance * (v_cond - v_uncond)


def euler_update(x, v, sigma, sigma_next):
    """Explicit Euler step of the flow-matching ODE dx/dsigma = v: the
    denoiser's velocity moves the latent from sigma to sigma_next
    ("Difflet", section 1 and section 3: the scheduler turns the velocity into
    a less noisy latent).  The latent is kept in full precision (fp32 on the
    GPU, "Difflet Engineering Report", Video output corrections)."""
    return _f(x) + (sigma_next - sigma) * _f(v)


def timestep_features(t, dim):
    """Sinusoidal features of a scalar timestep t (DiT-style): with
    half = dim/2 and f_j = 10000**(-j/half), the vector [cos(t f), sin(t f)].
    The pages do not define the timestep embedding; this is the reading
    taken."""
    half = dim // 2
    f = np.exp(-math.log(10000.0) * np.arange(half, dtype=np.float64) / half)
    a = float(t) * f
    return _f(np.concatenate([np.cos(a), np.sin(a)]))


# ----------------------------------------------------------------------------
# one denoising step of a DiT stack
# ----------------------------------------------------------------------------

def step_tokens(model, latent, sigma, round_points=True, t_scale=1000.0):
    """Timestep conditioning and the token sequence a step feeds to its first
    block (the reading of the parts the pages leave open is stated under
    ``denoise_step``): s = SiLU(SiLU(sinusoidal(t_scale * sigma) W_t1 + b_t1)
    W_t2 + b_t2) and, per batch row b, x[b] = [bf16(latent) W_in + b_in;
    text[b]].  Returns (s [D], x [B, N, D])."""
    R_ = _rounder(round_points)
    shp = model.shape
    blk = shp.block
    B, nv, N, D = blk.batch, blk.n_vis, blk.n_tok, blk.hidden
    sig32 = float(np.float32(sigma))
    f = R_(timestep_features(float(np.float32(t_scale)) * sig32, shp.freq_dim))
    c = R_(silu(linear(f, _dec(model.t_w1), _dec(model.t_b1))))
    s = R_(silu(linear(c, _dec(model.t_w2), _dec(model.t_b2))))
    lat = _f(latent)
    xin = linear(R_(lat), _dec(model.in_w), _dec(model.in_b))  # [Bl, n_vis, D]
    x = np.empty((B, N, D), dtype=_ARITH)
    for b in range(B):
        x[b, :nv] = xin[0 if shp.cfg else b]
        x[b, nv:] = _dec(model.text[b])
    return s, x


def denoise_step(model, latent, sigma, sigma_next, guidance, round_points=True, rows=None,
                 t_scale=1000.0):
    """One step of the denoising loop ("Difflet", section 3: the denoiser
    predicts a velocity from the latent, the timestep and the encoder
    outputs, the scheduler uses it to update the latent; "19. Diffusion,
    Image, Video, and World Models", Follow the diffusion pipeline).

    ``model`` provides ``shape`` (a LoopShape), the conditioning weights
    (t_w1, t_b1, t_w2, t_b2, in_w, in_b, fin_mod_w, fin_mod_b, out_w, out_b),
    ``text`` [B, n_txt, D], ``txt_valid`` [B] and ``layer(l)`` (block weights
    plus mod_w, mod_b).  ``latent`` is [Bl, n_vis, C] (Bl = 1 with guidance,
    else B).  The reading taken for the parts the pages leave open:

      f = sinusoidal(t_scale * sigma); c = SiLU(f W_t1 + b_t1);
      s = SiLU(c W_t2 + b_t2)                       (timestep conditioning)
      tokens of row b: [bf16(latent) W_in + b_in ; text[b]]
      per layer: mod = s W_mod + b_mod (one vector for every batch row), block
      (shift, scale) = s W_fin + b_fin;  v = adaLN(x) W_out + b_out  (visual rows)
      guidance: v_hat = v_uncond + g (v_cond - v_uncond)  (row 0 cond, row 1 uncond)
      latent <- latent + (sigma_next - sigma) v_hat     (Euler, see euler_update)

    With ``round_points`` every value the GPU stores in bfloat16 is rounded
    (features, c, s, modulation vectors, the bf16 copy of the latent, block
    intermediates, final norm output, v).  ``rows`` restricts the visual
    tokens whose velocity and update are returned; it is only exact for a
    single-block model (a later block needs every row of the one before).
    Returns (new latent rows [Bl, R, C], v [B, R, C])."""
    R_ = _rounder(round_points)
    shp = model.shape
    blk = shp.block
    B, nv, N, D = blk.batch, blk.n_vis, blk.n_tok, blk.hidden
    cfg = shp.cfg
    sig32 = float(np.float32(sigma))
    lat = _f(latent)
    s, x = step_tokens(model, lat, sigma, round_points, t_scale)
    if shp.depth > 1 and rows is not None:
        raise ValueError("row subsets are only exact for a single block")
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    for l in range(shp.depth):
        w = model.layer(l)
        mod = R_(linear(s, _dec(w["mod_w"]), _dec(w["mod_b"]))).reshape(6, D)
        inp = dict(w)
        inp["x"] = x
        inp["mod"] = np.broadcast_to(mod, (B, 6, D))
        inp["txt_valid"] = model.txt_valid
        x = block_forward(inp, blk, round_points=round_points,
                          rows=None if shp.depth > 1 else rows)
    fin = R_(linear(s, _dec(model.fin_mod_w), _dec(model.fin_mod_b)))
    h = R_(adaln_modulate(x, fin[:D], fin[D:], blk.ln_eps))
    if rows is not None and shp.depth == 1:
        keep = sel < nv
        h = h[:, keep]
        lat_rows = sel[keep]
    else:
        h = h[:, :nv]
        lat_rows = np.arange(nv)
    v = R_(linear(h, _dec(model.out_w), _dec(model.out_b)))  # [B, R, C]
    v_hat = cfg_combine(v[0:1], v[1:2], guidance) if cfg else v
    new = euler_update(lat[:, lat_rows], v_hat, sig32, float(np.float32(sigma_next)))
    return new, v
