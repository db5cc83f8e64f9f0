"""Pins of the CPU oracle against things other than itself: closed forms,
invariants, brute force on tiny inputs and independent library routines
(torch CPU fp64).  These run without a GPU."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from synthetic import configs as C
from synthetic import gen as G


# ---------------------------------------------------------------- bfloat16

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x3F81, 0x0001],
                    dtype=np.uint16)
    got = O.bf16_decode(bits)
    want = [1.0, -2.0, 0.0, -0.0, np.inf, -np.inf, 1.0 + 2.0 ** -7, 2.0 ** -133]
    assert got.tolist() == want


def test_round_bf16_ties_to_even_and_overflow():
    ulp = 2.0 ** -7
    x = np.array([1.0 + ulp / 2, 1.0 + 3 * ulp / 2, 1.0 + ulp / 2 + 1e-12, -(1.0 + ulp / 2),
                  3.5e38, 2.0 ** -130 * 1.25, 0.0, 10.5 * 2.0 ** -133, 11.5 * 2.0 ** -133])
    got = O.round_bf16(x)
    assert got[0] == 1.0
    assert got[1] == 1.0 + 2 * ulp
    assert got[2] == 1.0 + ulp
    assert got[3] == -1.0
    assert np.isinf(got[4])
    assert got[5] == 2.0 ** -130 * 1.25  # 10 units of the subnormal spacing 2**-133: exact
    assert got[6] == 0.0
    assert got[7] == 10 * 2.0 ** -133 and got[8] == 12 * 2.0 ** -133  # subnormal ties to even


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(5000)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), want)


def _round_bf16_frexp(x):
    """Round to the nearest bfloat16, ties to even, written from the format's
    definition: x = m 2**e with 0.5 <= |m| < 1 (frexp); a normal bfloat16
    keeps 8 significant bits, so round m * 2**8 to an integer (numpy rounds
    halves to even) and scale back; below 2**-126 the spacing is fixed at
    2**-133; beyond the largest finite bfloat16 the result is infinite."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.round(m * 256.0), e - 8)
    sub = np.abs(x) < 2.0 ** -126
    r[sub] = np.ldexp(np.round(np.ldexp(x[sub], 133)), -133)
    big = np.abs(r) > (2.0 - 2.0 ** -7) * 2.0 ** 127
    r[big] = np.copysign(np.inf, x[big])
    return r


def test_round_bf16_random_fp64_against_frexp_definition():
    """fp64 inputs that are not float32 values: random mantissas over the
    whole exponent range, exact ties between neighbouring bfloat16 values,
    and values one fp64 ulp either side of a tie (where a detour through
    float32 would round twice)."""
    rng = np.random.default_rng(21)
    n = 200000
    x = rng.standard_normal(n) * np.ldexp(1.0, rng.integers(-140, 128, n))
    b = O.bf16_decode(rng.integers(0, 0x7F7F, 20000, dtype=np.uint16)) * rng.choice([-1.0, 1.0], 20000)
    ulp = np.ldexp(1.0, np.frexp(b)[1] - 8)
    ulp[np.abs(b) < 2.0 ** -126] = 2.0 ** -133
    ties = b + ulp / 2
    x = np.concatenate([x, ties, np.nextafter(ties, np.inf), np.nextafter(ties, -np.inf)])
    with np.errstate(over="ignore"):
        assert not np.array_equal(x.astype(np.float32).astype(np.float64), x)
    np.testing.assert_array_equal(O.round_bf16(x), _round_bf16_frexp(x))


def test_input_generator_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50000) * 3).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(G.f32_to_bf16_bits(x), want)


def test_generator_is_chunk_independent_and_seeded(monkeypatch):
    ss = G.seed_sequence(11)
    a = G._normal_bf16(ss, (1000, 7))
    monkeypatch.setattr(G, "_CHUNK", 333)
    b = G._normal_bf16(G.seed_sequence(11), (1000, 7))
    np.testing.assert_array_equal(a, b)
    c = G._normal_bf16(G.seed_sequence(12), (1000, 7))
    assert (a != c).mean() > 0.9
    x = O.bf16_decode(a)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05


def test_valid_length_draws_in_range():
    inp = G.block_inputs(C.C2, weights=False)
    L = inp["txt_valid"]
    assert L.shape == (2,) and ((L >= 77) & (L <= 512)).all()
    assert G.block_inputs(C.C3, weights=False)["txt_valid"].tolist() == [226]


# ---------------------------------------------------------------- adaLN

def test_adaln_matches_torch_layer_norm_and_invariants():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 5, 64)) * 2.0 + 0.7
    shift = rng.standard_normal((3, 1, 64))
    scale = rng.standard_normal((3, 1, 64))
    eps = 1e-6
    got = O.adaln_modulate(x, shift, scale, eps)
    ln = torch.nn.functional.layer_norm(torch.from_numpy(x), (64,), eps=eps).numpy()
    np.testing.assert_allclose(got, ln * (1 + scale) + shift, rtol=1e-12, atol=1e-12)
    plain = O.adaln_modulate(x, 0.0, 0.0, eps)
    var = x.var(axis=-1)
    np.testing.assert_allclose(plain.mean(-1), 0.0, atol=1e-12)
    np.testing.assert_allclose((plain ** 2).mean(-1), var / (var + eps), rtol=1e-12)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_full_width_invariant_and_scope():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 4, 32))
    q[..., :16] *= 10.0  # head 0 much larger than head 1
    eps = 1e-6
    out = O.rms_norm_full(q, np.ones(32), eps)
    ms = (q * q).mean(-1)
    np.testing.assert_allclose((out ** 2).mean(-1), ms / (ms + eps), rtol=1e-12)
    # one normaliser for all heads: out / q is the same across the whole width
    ratio = out / q
    np.testing.assert_allclose(ratio, np.broadcast_to(ratio[..., :1], ratio.shape), rtol=1e-12)
    g = rng.standard_normal(32)
    np.testing.assert_allclose(O.rms_norm_full(q, g, eps), out * g, rtol=1e-12)
    # scale invariance (eps -> 0)
    np.testing.assert_allclose(O.rms_norm_full(q * 7.0, 1.0, 0.0),
                               O.rms_norm_full(q, 1.0, 0.0), rtol=1e-12)


# ---------------------------------------------------------------- positions / RoPE

def test_positions_brute_force():
    grid = (3, 4, 5)
    want = []
    for t in range(grid[0]):
        for h in range(grid[1]):
            for w in range(grid[2]):
                want.append([t, h, w])
    want += [[0, 0, 0]] * 6
    np.testing.assert_array_equal(O.token_positions(grid, 6), np.array(want))


def test_rope_hand_values():
    # dims (4, 4, 4): pair 0 of each axis turns by pos, pair 1 by pos/100
    x = np.ones((1, 1, 12))
    pos = np.array([[3, 5, 7]])
    got = O.rope_axial(x.reshape(1, 1, 1, 12), pos, (4, 4, 4), 10000.0).reshape(12)
    want = []
    for p in (3, 5, 7):
        for a in (p * 1.0, p * 0.01):
            want += [math.cos(a) - math.sin(a), math.sin(a) + math.cos(a)]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
    # a unit vector on the first dim of the h block turns into (cos 5, sin 5)
    e = np.zeros((1, 1, 1, 12))
    e[..., 4] = 1.0
    got = O.rope_axial(e, pos, (4, 4, 4), 10000.0).reshape(12)
    assert got[4] == math.cos(5.0) and got[5] == math.sin(5.0)
    assert np.count_nonzero(got) == 2


def test_rope_invariants():
    rng = np.random.default_rng(2)
    dims = (44, 42, 42)
    x = rng.standard_normal((2, 30, 3, 128))
    pos = O.token_positions((2, 3, 5), 0)
    y = O.rope_axial(x, pos, dims, 10000.0)
    # norm of every rotated pair (hence of every vector) is preserved
    np.testing.assert_allclose((y ** 2).reshape(2, 30, 3, 64, 2).sum(-1),
                               (x ** 2).reshape(2, 30, 3, 64, 2).sum(-1), rtol=1e-12)
    # position 0 is the identity
    np.testing.assert_array_equal(y[:, 0], x[:, 0])
    # relative position: <R(p) q, R(p') k> = <R(p - p') q, k>
    q = rng.standard_normal((1, 1, 1, 128))
    k = rng.standard_normal((1, 1, 1, 128))
    p1, p2 = np.array([[4, 9, 2]]), np.array([[1, 3, 7]])
    lhs = (O.rope_axial(q, p1, dims, 1e4) * O.rope_axial(k, p2, dims, 1e4)).sum()
    rhs = (O.rope_axial(q, p1 - p2, dims, 1e4) * k).sum()
    assert abs(lhs - rhs) < 1e-10
    # 2D split (0, d/2, d/2) ignores the t position
    np.testing.assert_array_equal(O.rope_axial(q, np.array([[5, 9, 2]]), (0, 64, 64), 1e4),
                                  O.rope_axial(q, np.array([[0, 9, 2]]), (0, 64, 64), 1e4))


# ---------------------------------------------------------------- attention

def _rand_qkv(rng, B, N, H, d):
    return (rng.standard_normal((B, N, H, d)), rng.standard_normal((B, N, H, d)),
            rng.standard_normal((B, N, H, d)))


def test_softmax_rows_sum_to_one_and_padding_gets_zero():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((40, 16)), rng.standard_normal((50, 16))
    p, _ = O.attention_probs(q * 3, k, 37, 0.25)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-12)
    assert (p[:, 37:] == 0.0).all() and (p[:, :37] > 0).all()


def test_attention_two_key_closed_form():
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [math.log(3.0), 0.0], [50.0, 0.0]])  # third key is padding
    p, lse = O.attention_probs(q, k, 2, 1.0)
    np.testing.assert_allclose(p, [[0.25, 0.75, 0.0]], rtol=1e-15)
    assert abs(lse[0] - math.log(4.0)) < 1e-15


def test_attention_q_zero_gives_mean_of_valid_values():
    rng = np.random.default_rng(4)
    B, nv, nt, H, d = 2, 13, 7, 3, 8
    q, k, v = _rand_qkv(rng, B, nv + nt, H, d)
    valid = [5, 0]
    o, lse = O.joint_attention(np.zeros_like(q), k, v, nv, valid)
    for b in range(B):
        want = v[b, :nv + valid[b]].mean(axis=0)
        np.testing.assert_allclose(o[b], np.broadcast_to(want, o[b].shape), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[b], math.log(nv + valid[b]), rtol=1e-14)


def test_attention_single_valid_key_returns_that_value():
    rng = np.random.default_rng(5)
    q, k, v = _rand_qkv(rng, 1, 1 + 4, 2, 8)
    o, _ = O.joint_attention(q, k, v, 1, [0])
    np.testing.assert_allclose(o[0], np.broadcast_to(v[0, 0], o[0].shape), rtol=1e-15)


def test_attention_padding_content_is_ignored_bitwise():
    rng = np.random.default_rng(6)
    nv, nt = 20, 12
    q, k, v = _rand_qkv(rng, 2, nv + nt, 2, 16)
    valid = [3, 9]
    o1, l1 = O.joint_attention(q, k, v, nv, valid)
    k2, v2 = k.copy(), v.copy()
    for b in range(2):
        k2[b, nv + valid[b]:] = rng.standard_normal(k2[b, nv + valid[b]:].shape) * 100
        v2[b, nv + valid[b]:] = rng.standard_normal(v2[b, nv + valid[b]:].shape) * 100
    o2, l2 = O.joint_attention(q, k2, v2, nv, valid)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # while changing the valid length moves the output
    o3, _ = O.joint_attention(q, k, v, nv, [4, 9])
    assert np.abs(o3[0] - o1[0]).max() > 1e-3


def test_attention_permuting_valid_keys_is_invariant():
    rng = np.random.default_rng(8)
    nv, nt, L = 17, 6, 4
    q, k, v = _rand_qkv(rng, 1, nv + nt, 2, 8)
    perm = np.concatenate([rng.permutation(nv + L), np.arange(nv + L, nv + nt)])
    o1, _ = O.joint_attention(q, k, v, nv, [L])
    o2, _ = O.joint_attention(q, k[:, perm], v[:, perm], nv, [L])
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)


def test_attention_brute_force_loops():
    rng = np.random.default_rng(9)
    B, nv, nt, H, d = 2, 5, 3, 2, 4
    q, k, v = _rand_qkv(rng, B, nv + nt, H, d)
    valid = [2, 1]
    scale = 1.0 / math.sqrt(d)
    o, lse = O.joint_attention(q, k, v, nv, valid)
    for b in range(B):
        nk = nv + valid[b]
        for h in range(H):
            for i in range(nv + nt):
                s = [scale * sum(q[b, i, h, c] * k[b, j, h, c] for c in range(d)) for j in range(nk)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = sum(e)
                for c in range(d):
                    want = sum(e[j] / z * v[b, j, h, c] for j in range(nk))
                    assert abs(o[b, i, h, c] - want) < 1e-13
                assert abs(lse[b, h, i] - (m + math.log(z))) < 1e-13


def test_attention_matches_torch_sdpa_with_prefix_mask():
    rng = np.random.default_rng(10)
    B, nv, nt, H, d = 2, 24, 8, 3, 16
    q, k, v = _rand_qkv(rng, B, nv + nt, H, d)
    valid = [8, 2]
    o, _ = O.joint_attention(q, k, v, nv, valid)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    mask = torch.zeros(B, 1, nv + nt, nv + nt, dtype=torch.bool)
    for b in range(B):
        mask[b, :, :, :nv + valid[b]] = True
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    np.testing.assert_allclose(o, want.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- GELU / linear

def test_gelu_values_and_torch():
    assert O.gelu_erf(np.array([0.0]))[0] == 0.0
    assert abs(O.gelu_erf(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    assert abs(O.gelu_erf(np.array([-1.0]))[0] + 0.15865525393145707) < 1e-15
    z = np.linspace(-8, 8, 1001)
    want = torch.nn.functional.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(O.gelu_erf(z), want, rtol=1e-14, atol=1e-15)


def test_silu_values_odd_identity_and_torch():
    """SiLU(z) = z sigma(z): hand values, the identity SiLU(z) - SiLU(-z) = z
    (sigma(z) + sigma(-z) = 1, which a sign or term error breaks), the limits
    and torch's fp64 silu."""
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert abs(O.silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-15
    assert abs(O.silu(np.array([-1.0]))[0] + 0.2689414213699951) < 1e-15
    assert abs(O.silu(np.array([2.0]))[0] - 1.7615941559557646) < 1e-15
    z = np.linspace(-30, 30, 6001)
    np.testing.assert_allclose(O.silu(z) - O.silu(-z), z, rtol=1e-13, atol=1e-13)
    assert abs(O.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15
    want = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(O.silu(z), want, rtol=1e-14, atol=1e-300)


def test_linear_explicit_loops():
    rng = np.random.default_rng(11)
    a, w, b = rng.standard_normal((3, 5)), rng.standard_normal((4, 5)), rng.standard_normal(4)
    y = O.linear(a, w, b)
    for i in range(3):
        for j in range(4):
            assert abs(y[i, j] - (b[j] + sum(a[i, c] * w[j, c] for c in range(5)))) < 1e-13


# ---------------------------------------------------------------- the block

TINY = C.BlockShape("tiny_bf", batch=2, grid=(1, 2, 3), n_txt=3, heads=2, head_dim=4, mlp=16,
                    rope=(0, 2, 2), txt_valid=("fixed", (1, 3)), seed=77)


def _brute_block(inp, s):
    """Whole block in plain Python loops, written from the step list."""
    B, N, D, H, d, F = s.batch, s.n_tok, s.hidden, s.heads, s.head_dim, s.mlp
    dec = lambda a: O.bf16_decode(a).tolist()
    x, mod = dec(inp["x"]), dec(inp["mod"])
    Wqkv, bqkv, gq, gk = dec(inp["w_qkv"]), dec(inp["b_qkv"]), dec(inp["g_q"]), dec(inp["g_k"])
    Wo, bo, Wu, bu, Wd, bd = (dec(inp[n]) for n in ("w_o", "b_o", "w_up", "b_up", "w_dn", "b_dn"))
    T_, Hg, Wg = s.grid

    def ln_mod(row, sh, sc):
        mu = sum(row) / D
        var = sum((r - mu) ** 2 for r in row) / D
        return [(row[c] - mu) / math.sqrt(var + s.ln_eps) * (1 + sc[c]) + sh[c] for c in range(D)]

    def lin(row, W, bias):
        return [bias[o] + sum(row[c] * W[o][c] for c in range(len(row))) for o in range(len(W))]

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
            h = ln_mod(x[b][i], mb[0], mb[1])
            qkv = lin(h, Wqkv, bqkv)
            qs.append(rms_rope(qkv[:D], gq, pos_of(i)))
            ks.append(rms_rope(qkv[D:2 * D], gk, pos_of(i)))
            vs.append(qkv[2 * D:])
        nk = s.n_vis + int(inp["txt_valid"][b])
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
            y = lin(o, Wo, bo)
            x1 = [x[b][i][c] + mb[2][c] * y[c] for c in range(D)]
            h2 = ln_mod(x1, mb[3], mb[4])
            u = [z_ * 0.5 * (1 + math.erf(z_ / math.sqrt(2))) for z_ in lin(h2, Wu, bu)]
            y2 = lin(u, Wd, bd)
            rows.append([x1[c] + mb[5][c] * y2[c] for c in range(D)])
        res.append(rows)
    return np.array(res)


def test_block_brute_force_tiny():
    inp = G.block_inputs(TINY)
    got = O.block_forward(inp, TINY, round_points=False)
    want = _brute_block(inp, TINY)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_block_zero_gates_is_identity():
    inp = G.block_inputs(C.C1)
    inp["mod"] = inp["mod"].copy()
    inp["mod"][:, 2] = 0
    inp["mod"][:, 5] = 0
    x2 = O.block_forward(inp, C.C1, round_points=True)
    np.testing.assert_array_equal(x2, O.bf16_decode(inp["x"]))


def test_block_gate1_zero_ignores_attention_inputs():
    inp = G.block_inputs(TINY)
    inp["mod"] = inp["mod"].copy()
    inp["mod"][:, 2] = 0
    a = O.block_forward(inp, TINY)
    inp2 = dict(inp)
    inp2["w_qkv"] = G._normal_bf16(G.seed_sequence(999), inp["w_qkv"].shape, 0.5)
    b = O.block_forward(inp2, TINY)
    np.testing.assert_array_equal(a, b)


def test_block_row_subset_is_exact():
    inp = G.block_inputs(C.C1)
    full = O.block_forward(inp, C.C1)
    rows = np.array([0, 5, 100, 255, 256, 275, 276, 287])
    sub = O.block_forward(inp, C.C1, rows=rows)
    np.testing.assert_allclose(sub, full[:, rows], rtol=0, atol=0)


def test_block_rounding_points_close_to_unrounded():
    inp = G.block_inputs(C.C1)
    a = O.block_forward(inp, C.C1, round_points=True)
    b = O.block_forward(inp, C.C1, round_points=False)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel < 5e-3


# ---------------------------------------------------------------- sampler

def test_sigma_schedule():
    s = O.sigma_schedule(30)
    assert s.shape == (31,) and s[0] == 1.0 and s[-1] == 0.0
    np.testing.assert_allclose(np.diff(s), -1.0 / 30, rtol=1e-12)


def _run_loop(x0, vel, steps=30):
    s = O.sigma_schedule(steps)
    x = x0
    for i in range(steps):
        x = O.euler_update(x, vel(x, s[i]), s[i], s[i + 1])
    return x


def test_euler_lands_on_target_for_straight_flow():
    rng = np.random.default_rng(12)
    x0, c = rng.standard_normal(50), rng.standard_normal(50)
    x = _run_loop(x0, lambda x, s: (x - c) / s)
    np.testing.assert_allclose(x, c, rtol=1e-12, atol=1e-12)


def test_euler_cfg_lands_on_guided_target():
    rng = np.random.default_rng(13)
    x0, c0, c1 = (rng.standard_normal(40) for _ in range(3))
    g = 5.0
    x = _run_loop(x0, lambda x, s: O.cfg_combine((x - c1) / s, (x - c0) / s, g))
    np.testing.assert_allclose(x, c0 + g * (c1 - c0), rtol=1e-11, atol=1e-11)


def test_euler_constant_velocity_and_equal_branches():
    rng = np.random.default_rng(14)
    x0, v = rng.standard_normal(20), rng.standard_normal(20)
    np.testing.assert_allclose(_run_loop(x0, lambda x, s: v), x0 - v, rtol=1e-12, atol=1e-12)
    a = O.cfg_combine(v, v, 5.0)
    np.testing.assert_array_equal(a, v)


def test_timestep_features():
    f = O.timestep_features(0.0, 256)
    np.testing.assert_array_equal(f, np.concatenate([np.ones(128), np.zeros(128)]))
    f = O.timestep_features(500.0, 256)
    assert f[0] == math.cos(500.0) and f[128] == math.sin(500.0)
    np.testing.assert_allclose(f[:128] ** 2 + f[128:] ** 2, 1.0, rtol=1e-14)
    # frequencies fall geometrically from 1 towards 1/10000
    assert abs(O.timestep_features(1.0, 256)[127] - math.cos(10000.0 ** (-127 / 128))) < 1e-15
