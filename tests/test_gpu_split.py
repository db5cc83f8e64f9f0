"""GPU parity of split joint attention ("Difflet", section 4.3): a text
partial with bounds [0, L_text) plus visual K/V partitions, each attended by
dit_attention_partial, merged by dit_attention_merge, compared with the
oracle's partials and merge (and its unsplit joint attention), and with the
unsplit GPU kernel on the same inputs."""

import numpy as np
import pytest
import torch

import diffusion_transformer_denoising_dit_amd as D
import oracle as O
from synthetic import configs as C
from synthetic import gen as G
from tests.gpu_util import assert_parity, dev_bf16, host
from tests.sampling import sample_rows

pytestmark = pytest.mark.gpu

SPLIT_CASES = [
    # (shape, visual cuts)
    (C.AttnShape("split_d64", batch=2, n_vis=300, n_txt=40, heads=3, head_dim=64,
                 txt_valid=("fixed", (7, 40)), seed=51), [0, 64, 129, 300]),
    (C.AttnShape("split_d128_empty_text", batch=2, n_vis=257, n_txt=77, heads=2, head_dim=128,
                 txt_valid=("fixed", (0, 13)), seed=52), [0, 100, 257]),
    (C.AttnShape("split_one_chunk", batch=1, n_vis=70, n_txt=9, heads=1, head_dim=128,
                 txt_valid=("fixed", (9,)), seed=53), [0, 70]),
]


def _split_gpu(shape, inp, cuts):
    """Run the partials on the GPU: returns (merged bf16 out, merged lse,
    list of (out_p, lse_p))."""
    B, N, H, d, HD = shape.batch, shape.n_tok, shape.heads, shape.head_dim, shape.hidden
    q = dev_bf16(inp["q"])
    k = dev_bf16(inp["k"]).view(B, N, HD)
    v = dev_bf16(inp["v"]).view(B, N, HD)
    segs = [(shape.n_vis, N, list(inp["txt_valid"]))]
    segs += [(a, b, [b - a] * B) for a, b in zip(cuts[:-1], cuts[1:])]
    parts = []
    for a, b, valid in segs:
        kp = k[:, a:b].contiguous()
        vp = v[:, a:b].contiguous()
        out = torch.empty((B, N, HD), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        D.dit_attention_partial(D.partial_desc(B, N, b - a, H, d, valid), q, HD, kp, vp, HD, out, HD,
                                lse)
        parts.append((out, lse))
    merged = torch.empty((B, N, HD), dtype=torch.bfloat16, device="cuda")
    mlse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    D.dit_attention_merge(B, N, H, d, [o for o, _ in parts], HD, [l for _, l in parts], merged, HD,
                          mlse)
    torch.cuda.synchronize()
    return merged, mlse, parts, segs


def _oracle_split(shape, inp, segs):
    B, N, H, d = shape.batch, shape.n_tok, shape.heads, shape.head_dim
    q = O.bf16_decode(inp["q"]).reshape(B, N, H, d)
    k = O.bf16_decode(inp["k"]).reshape(B, N, H, d)
    v = O.bf16_decode(inp["v"]).reshape(B, N, H, d)
    scale = 1.0 / np.sqrt(d)
    return [O.attention_partial(q, k[:, a:b], v[:, a:b], valid, scale) for a, b, valid in segs]


@pytest.mark.parametrize("shape,cuts", SPLIT_CASES, ids=lambda c: getattr(c, "name", ""))
def test_split_attention_matches_oracle_and_unsplit_kernel(shape, cuts):
    inp = G.attention_inputs(shape, 2.0)
    merged, mlse, parts, segs = _split_gpu(shape, inp, cuts)
    oparts = _oracle_split(shape, inp, segs)
    B, N, H, d = shape.batch, shape.n_tok, shape.heads, shape.head_dim
    # each partial: normalised output and log-denominator (empty partitions: 0 and -inf)
    for (out, lse), (acc, m, l), (a, b, valid) in zip(parts, oparts, segs):
        got_lse = host(lse)
        empty = np.array(valid)[:, None, None] == 0
        want_lse = np.where(empty, -np.inf, m + np.log(np.where(l > 0, l, 1.0)))
        assert np.array_equal(np.isinf(got_lse), np.isinf(want_lse)), f"[{a},{b}) empty rows"
        fin = np.isfinite(want_lse)
        assert_parity(got_lse[fin], want_lse[fin], f"{shape.name} partial [{a},{b}) lse",
                      max_abs=1e-3, rel_l2=1e-5)
        want_o = acc / np.where(l > 0, l, 1.0).transpose(0, 2, 1)[..., None]
        assert_parity(host(out).reshape(B, N, H, d), want_o, f"{shape.name} partial [{a},{b}) out")
    # merged: the oracle merge, which itself equals the unsplit oracle attention
    o_want, lse_want = O.merge_partials(oparts)
    assert_parity(host(merged).reshape(B, N, H, d), o_want, f"{shape.name} merged out")
    assert_parity(host(mlse), lse_want, f"{shape.name} merged lse", max_abs=1e-3, rel_l2=1e-5)
    # and the unsplit kernel on the same inputs, to the same bar: both paths round
    # the probabilities to bf16, each relative to its own running maximum, so
    # they agree to about twice the error each has against the oracle
    full = torch.empty_like(merged)
    desc = D.attn_desc(B, shape.n_vis, shape.n_txt, H, d, inp["txt_valid"])
    D.dit_joint_attention(desc, dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"]),
                          shape.hidden, full, shape.hidden)
    torch.cuda.synchronize()
    assert_parity(host(merged), host(full), f"{shape.name} split vs unsplit kernel")


def test_merge_formula_on_synthetic_partials():
    """The merge alone on arbitrary fp32 partials and log-denominators (some
    -inf): out = sum_p e^(lse_p - M) out_p / sum_p e^(lse_p - M)."""
    B, N, H, d, P = 2, 37, 3, 64, 5
    rng = np.random.default_rng(61)
    outs = rng.standard_normal((P, B, N, H * d)).astype(np.float32)
    lses = (rng.standard_normal((P, B, H, N)) * 6).astype(np.float32)
    lses[1, 0] = -np.inf  # an empty partial in batch row 0
    lses[3, :, 1, :5] = -np.inf
    lses[:, 1, 2, 7:10] = -np.inf  # three queries of one head with every partial empty
    parts = [(outs[p].reshape(B, N, H, d).astype(np.float64), lses[p].astype(np.float64),
              np.ones((B, H, N))) for p in range(P)]
    o_want, lse_want = O.merge_partials(parts)
    dev_o = [torch.from_numpy(outs[p]).cuda() for p in range(P)]
    dev_l = [torch.from_numpy(lses[p]).cuda() for p in range(P)]
    out = torch.empty((B, N, H * d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    D.dit_attention_merge(B, N, H, d, dev_o, H * d, dev_l, out, H * d, lse)
    torch.cuda.synchronize()
    empty = np.isneginf(lse_want)
    assert empty.sum() == 3
    lse_h = host(lse)
    assert np.all(np.isneginf(lse_h[empty])), "all-empty rows: lse must be -inf"
    out_h = host(out).reshape(B, N, H, d)
    assert np.all(out_h[1, 7:10, 2] == 0.0), "all-empty rows: output must be 0"
    assert_parity(out_h, o_want, "merge formula")
    assert_parity(np.where(empty, 0.0, lse_h), np.where(empty, 0.0, lse_want), "merge lse",
                  max_abs=1e-4, rel_l2=1e-6)


@pytest.mark.slow
def test_split_attention_c2_shape_sampled_rows():
    """The c2 image shape (2 x (4096 + 512), 24 x 128, valid lengths drawn per
    row): text partial + 4 visual partitions of unequal length, sampled query
    rows against the oracle's partials and merge."""
    s = C.C2
    shape = C.AttnShape("split_c2", batch=s.batch, n_vis=s.n_vis, n_txt=s.n_txt, heads=s.heads,
                        head_dim=s.head_dim, txt_valid=("uniform", 77, 512), seed=71)
    inp = G.attention_inputs(shape, 1.0)
    cuts = [0, 1000, 1024, 3001, 4096]
    merged, _, _, segs = _split_gpu(shape, inp, cuts)
    B, N, H, d = shape.batch, shape.n_tok, shape.heads, shape.head_dim
    rows = sample_rows(shape.n_vis, shape.n_txt, inp["txt_valid"], n_random=24, seed=5)
    q = O.bf16_decode(inp["q"]).reshape(B, N, H, d)[:, rows]
    k = O.bf16_decode(inp["k"]).reshape(B, N, H, d)
    v = O.bf16_decode(inp["v"]).reshape(B, N, H, d)
    oparts = [O.attention_partial(q, k[:, a:b], v[:, a:b], valid, 1.0 / np.sqrt(d))
              for a, b, valid in segs]
    o_want, _ = O.merge_partials(oparts)
    assert_parity(host(merged).reshape(B, N, H, d)[:, rows], o_want, "c2 split merged (sampled)")
