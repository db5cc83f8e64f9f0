"""Pins of the oracle's split joint attention ("Difflet", section 4.3: a text
partial with bounds [0, L_text) plus visual K/V partitions, each returning the
unnormalised weighted value sum, its max and its exponential sum, merged by
rescaling to a common max).  The merge is checked against the unsplit joint
attention (itself pinned by closed forms, brute force and torch SDPA), against
a two-key closed form, and for the invariants the statement implies."""

import math

import numpy as np

import oracle as O


def _qkv(seed, B=2, R=9, N=23, H=2, d=16, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, R, H, d)) * scale
    k = rng.standard_normal((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    return q, k, v


def _split(q, k, v, n_vis, txt_valid, cuts, scale):
    """Text partial over keys [n_vis, N) with bounds [0, L_b) plus one partial
    per visual chunk [cuts[i], cuts[i+1])."""
    B = k.shape[0]
    parts = [O.attention_partial(q, k[:, n_vis:], v[:, n_vis:], txt_valid, scale)]
    for a, b in zip(cuts[:-1], cuts[1:]):
        parts.append(O.attention_partial(q, k[:, a:b], v[:, a:b], [b - a] * B, scale))
    return parts


def test_split_merge_equals_unsplit_joint_attention():
    n_vis, n_txt = 15, 8
    q, k, v = _qkv(1, N=n_vis + n_txt, scale=2.0)
    txt_valid = [3, 8]
    scale = 1.0 / math.sqrt(q.shape[-1])
    want_o, want_lse = O.joint_attention(q, k, v, n_vis, txt_valid)
    for cuts in ([0, 15], [0, 4, 5, 15], [0, 7, 14, 15]):
        o, lse = O.merge_partials(_split(q, k, v, n_vis, txt_valid, cuts, scale))
        np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-12)


def test_empty_text_partial_is_neutral():
    n_vis, n_txt = 10, 6
    q, k, v = _qkv(2, N=n_vis + n_txt)
    scale = 0.3
    parts = _split(q, k, v, n_vis, [0, 0], [0, 6, 10], scale)
    acc, m, l = parts[0]
    assert np.all(m == -np.inf) and np.all(l == 0) and np.all(acc == 0)
    o, lse = O.merge_partials(parts)
    o2, lse2 = O.merge_partials(parts[1:])
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    want_o, want_lse = O.joint_attention(q, k, v, n_vis, [0, 0], scale=scale)
    np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-12)


def test_merge_is_order_independent():
    n_vis, n_txt = 12, 5
    q, k, v = _qkv(3, N=n_vis + n_txt, scale=3.0)
    parts = _split(q, k, v, n_vis, [5, 2], [0, 3, 9, 12], 0.25)
    o, lse = O.merge_partials(parts)
    o2, lse2 = O.merge_partials(parts[::-1])
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


def test_two_single_key_partials_closed_form():
    # one query, two partitions of one key each: o = (e^a v1 + e^b v2) / (e^a + e^b)
    q = np.array([[[[1.0, 2.0]]]])
    k1 = np.array([[[[0.5, -1.0]]]])
    k2 = np.array([[[[3.0, 1.0]]]])
    v1 = np.array([[[[1.0, 10.0]]]])
    v2 = np.array([[[[-2.0, 4.0]]]])
    a, b = 1.0 * 0.5 + 2.0 * -1.0, 1.0 * 3.0 + 2.0 * 1.0
    parts = [O.attention_partial(q, k1, v1, [1], 1.0), O.attention_partial(q, k2, v2, [1], 1.0)]
    acc, m, l = parts[0]
    assert m[0, 0, 0] == a and l[0, 0, 0] == 1.0 and np.all(acc[0, 0, 0] == v1[0, 0, 0])
    o, lse = O.merge_partials(parts)
    wa, wb = math.exp(a), math.exp(b)
    np.testing.assert_allclose(o[0, 0, 0], (wa * v1[0, 0, 0] + wb * v2[0, 0, 0]) / (wa + wb),
                               rtol=1e-15)
    assert abs(lse[0, 0, 0] - math.log(wa + wb)) < 1e-14


def test_single_partial_normalises_to_softmax():
    q, k, v = _qkv(4, B=1, R=5, N=7, H=1, d=8)
    acc, m, l = O.attention_partial(q, k, v, [6], 0.4)
    p, lse = O.attention_probs(q[0, :, 0], k[0, :, 0], 6, 0.4)
    np.testing.assert_allclose(acc[0, :, 0] / l[0, 0][:, None], p @ v[0, :, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(m[0, 0] + np.log(l[0, 0]), lse, rtol=0, atol=1e-13)


def test_merge_of_only_empty_partials_is_the_empty_sum():
    """A query none of whose partitions holds a valid key: every partial is
    the neutral element (acc 0, m -inf, l 0), so the merge is the empty sum,
    o = 0 with log-denominator -inf; adding one non-empty partial to them
    gives exactly that partial's normalised output."""
    q, k, v = _qkv(9, B=2, R=5, N=6)
    scale = 0.25
    empty = O.attention_partial(q, k, v, [0, 0], scale)
    assert np.all(empty[0] == 0) and np.all(empty[1] == -np.inf) and np.all(empty[2] == 0)
    o, lse = O.merge_partials([empty, empty])
    assert np.all(o == 0.0) and np.all(lse == -np.inf)
    full = O.attention_partial(q, k, v, [6, 4], scale)
    o2, lse2 = O.merge_partials([empty, full, empty])
    want_o, want_lse = O.joint_attention(q, k, v, 0, [6, 4], scale)
    np.testing.assert_allclose(o2, want_o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, want_lse, rtol=1e-13, atol=1e-14)
