"""Pins of the oracle's step caching (controller, relative L1 change, output
estimator, block-0 probe) against the pages' worked numbers (the TeaCache
accumulator run lengths, cadence-2 skip counts and speedup ceilings, kept in
tests/golden/stepcache_worked_examples.json with their citations), hand-worked
values and closed forms (exact extrapolation of linear trajectories, the
second-difference error of quadratic ones, a geometric online-delta schedule)
and invariants of the rules (no skip at the boundary, never two online-delta
skips in a row, LayerNorm statistics of the probe's signal)."""

import json
import math
import os

import numpy as np
import pytest

import oracle as O
from oracle import stepcache as S

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "stepcache_worked_examples.json")))


def _runs_of_skips(acts):
    """Lengths of maximal runs of SKIP that are closed by a FULL."""
    runs, cur = [], 0
    for a in acts:
        if a == S.SKIP:
            cur += 1
        else:
            if cur:
                runs.append(cur)
            cur = 0
    return runs


@pytest.mark.parametrize("case", GOLDEN["teacache_accumulator"]["cases"])
def test_teacache_worked_example(case):
    thr = GOLDEN["teacache_accumulator"]["threshold"]
    n = 60
    c = S.Controller(S.TEACACHE, n, warmup=2, cooldown=0, threshold=thr, coef=(1.0, 0.0))
    probe = [math.inf] + [case["rescaled_distance"]] * (n - 1)
    acts = S.decisions(c, probe)
    assert acts[:2] == [S.FULL, S.FULL]
    runs = _runs_of_skips(acts)
    assert runs and all(r == case["consecutive_skips"] for r in runs), runs
    # every compute after the warm-up is preceded by exactly that many skips
    period = case["consecutive_skips"] + 1
    assert acts[2:2 + 3 * period] == ([S.SKIP] * case["consecutive_skips"] + [S.FULL]) * 3


def test_teacache_polynomial_rescale_and_reset():
    # rescale r -> 2r + 0.01 (coefficients highest degree first): raw 0.02
    # becomes 0.05, so a threshold of 0.15 is crossed on the third step
    c = S.Controller(S.TEACACHE, 12, warmup=2, cooldown=0, threshold=0.15, coef=(2.0, 0.01))
    assert c.rescale(0.02) == pytest.approx(0.05, abs=1e-15)
    acts = S.decisions(c, [math.inf] + [0.02] * 11)
    assert acts == [S.FULL, S.FULL, S.SKIP, S.SKIP, S.FULL, S.SKIP, S.SKIP, S.FULL, S.SKIP,
                    S.SKIP, S.FULL, S.SKIP]
    # a boundary compute also resets the sum: in the cooldown nothing skips
    c = S.Controller(S.TEACACHE, 10, warmup=2, cooldown=4, threshold=1.0)
    acts = S.decisions(c, [math.inf] + [0.01] * 9)
    assert acts == [S.FULL, S.FULL, S.SKIP, S.SKIP, S.SKIP, S.SKIP, S.FULL, S.FULL, S.FULL, S.FULL]
    # a missing previous input (infinite score) forces a compute mid-window
    c = S.Controller(S.TEACACHE, 8, warmup=2, cooldown=0, threshold=1.0)
    acts = S.decisions(c, [math.inf, 0.01, 0.01, math.inf, 0.01, 0.01, 0.01, 0.01])
    assert acts == [S.FULL, S.FULL, S.SKIP, S.FULL, S.SKIP, S.SKIP, S.SKIP, S.SKIP]


@pytest.mark.parametrize("case", GOLDEN["fixed_cadence"]["cases"])
def test_cadence_two_skip_counts_and_ceiling(case):
    g = GOLDEN["fixed_cadence"]
    n = case["n_steps"]
    c = S.Controller(S.CADENCE, n, warmup=g["warmup"], cooldown=g["cooldown"], cadence=g["cadence"])
    acts = S.decisions(c)
    assert acts.count(S.SKIP) == case["skips"]
    full = acts.count(S.FULL)
    assert round(n / full, 2) == pytest.approx(case["ceiling"], abs=1e-9)
    # boundary steps compute; inside the window compute and skip alternate
    assert all(a == S.FULL for a in acts[:g["warmup"]] + acts[n - g["cooldown"]:])
    win = acts[g["warmup"]:n - g["cooldown"]]
    assert win == [S.FULL, S.SKIP] * (len(win) // 2)


def test_cadence_three_and_two_full_steps_rule():
    c = S.Controller(S.CADENCE, 10, warmup=1, cooldown=1, cadence=3)
    assert S.decisions(c) == [S.FULL, S.FULL, S.SKIP, S.SKIP, S.FULL, S.SKIP, S.SKIP, S.FULL,
                              S.SKIP, S.FULL]
    # no warm-up: the window starts at step 0, but two completed full steps
    # are needed before the first skip
    c = S.Controller(S.CADENCE, 6, warmup=0, cooldown=0, cadence=2)
    assert S.decisions(c) == [S.FULL, S.FULL, S.FULL, S.SKIP, S.FULL, S.SKIP]


def test_online_delta_geometric_closed_form():
    """Output changes c_i = 0.9**i: the first measured change is c_1 = 0.9,
    so a full step i asks to cache the next one exactly when
    0.9**(i-1) < alpha = 0.6, i.e. from i = 6 on (0.9**5 = 0.59049); after
    that, cached and full steps alternate until the cooldown."""
    alpha = GOLDEN["online_delta"]["alpha"]
    n, w, cd = 50, 5, 5
    ch = [math.inf] + [0.9 ** i for i in range(1, n)]
    c = S.Controller(S.ONLINE_DELTA, n, warmup=w, cooldown=cd, alpha=alpha)
    acts = S.decisions(c, output_changes=ch)
    skips = [i for i, a in enumerate(acts) if a == S.SKIP]
    assert skips == list(range(7, 44, 2))
    assert c.first_change == pytest.approx(0.9, abs=0)


def test_online_delta_invariants():
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(3, 60))
        w, cd = int(rng.integers(0, 6)), int(rng.integers(0, 6))
        ch = [math.inf] + list(rng.uniform(0.0, 1.0, n - 1))
        c = S.Controller(S.ONLINE_DELTA, n, warmup=w, cooldown=cd, alpha=float(rng.uniform(0.2, 1.5)))
        acts = S.decisions(c, output_changes=ch)
        for i, a in enumerate(acts):
            if a == S.SKIP:
                assert w <= i < n - cd
                assert acts[i - 1] == S.FULL          # a cached step follows a full one
                assert acts[:i].count(S.FULL) >= 2     # two completed full steps
    # constant output changes never drop below alpha * first (alpha < 1)
    c = S.Controller(S.ONLINE_DELTA, 30, warmup=2, cooldown=2, alpha=0.6)
    assert S.decisions(c, output_changes=[math.inf] + [0.3] * 29).count(S.SKIP) == 0


def test_off_mode_and_order_check():
    c = S.Controller(S.OFF, 5)
    assert S.decisions(c) == [S.FULL] * 5
    c = S.Controller(S.CADENCE, 5)
    c.decide(0)
    with pytest.raises(ValueError):
        c.decide(2)


def test_rel_l1_hand_values_and_invariants():
    assert S.rel_l1([1.0, 2.0], [1.0, 1.0]) == 0.5
    assert S.rel_l1([3.0, -1.0, 0.0], [2.0, 1.0, -1.0]) == pytest.approx(4.0 / 4.0)
    rng = np.random.default_rng(0)
    a, b = rng.standard_normal(1000), rng.standard_normal(1000)
    assert S.rel_l1(a, a) == 0.0
    assert S.rel_l1(7.5 * a, 7.5 * b) == pytest.approx(S.rel_l1(a, b), rel=1e-13)  # scale-free
    assert S.rel_l1(a, b) == pytest.approx(np.mean(np.abs(a - b)) / np.mean(np.abs(b)), rel=1e-13)
    assert S.rel_l1(np.zeros(4), np.zeros(4)) == 0.0
    assert S.rel_l1(np.ones(4), np.zeros(4)) == math.inf
    # b = a + e with |e| << |a|: close to mean|e| / mean|a|
    e = 1e-3 * rng.standard_normal(1000)
    assert S.rel_l1(a, a + e) == pytest.approx(np.abs(e).sum() / np.abs(a + e).sum(), rel=1e-12)


def test_estimator_hand_values():
    c = S.OutputCache()
    assert c.full(np.array([1.0, 1.0])) == math.inf
    assert c.full(np.array([2.0, 2.0])) == pytest.approx(1.0)     # |2-1| / |1|
    np.testing.assert_array_equal(c.skip(), [3.0, 3.0])
    # the change after a skip is measured against the estimate, not the last full output
    assert c.full(np.array([5.0, 5.0])) == pytest.approx(2.0 / 3.0)
    np.testing.assert_array_equal(c.delta, [2.0, 2.0])
    np.testing.assert_array_equal(c.skip(), [7.0, 7.0])
    with pytest.raises(ValueError):
        S.OutputCache().skip()


def test_estimator_linear_exact_quadratic_second_difference():
    rng = np.random.default_rng(1)
    a, b, q = rng.standard_normal(16), rng.standard_normal(16), rng.standard_normal(16)
    # linear in the step index: every cached estimate is exact
    c = S.OutputCache()
    c.full(a)
    c.full(a + b)
    for i in range(2, 6):
        np.testing.assert_allclose(c.skip(), a + i * b, rtol=0, atol=1e-12)
    # quadratic v_i = i^2 q: after full steps at i-1 and i the estimate of
    # step i+1 is 2 i^2 - (i-1)^2 = (i+1)^2 - 2, one second difference short
    for i in range(1, 6):
        c = S.OutputCache()
        c.full((i - 1) ** 2 * q)
        c.full(i ** 2 * q)
        np.testing.assert_allclose(c.skip(), (i + 1) ** 2 * q - 2 * q, rtol=0, atol=1e-12)


def test_cached_loop_of_linear_velocity_field_equals_uncached():
    """A velocity that is linear in the step index is extrapolated exactly,
    so any cadence reproduces the uncached Euler trajectory."""
    rng = np.random.default_rng(2)
    a, b = rng.standard_normal(32), rng.standard_normal(32)
    sig = O.sigma_schedule(20)
    x_ref = x = rng.standard_normal(32)
    ctl = S.Controller(S.CADENCE, 20, warmup=2, cooldown=2, cadence=3)
    cache = S.OutputCache()
    for i in range(20):
        v = a + i * b
        x_ref = O.euler_update(x_ref, v, sig[i], sig[i + 1])
        act = ctl.decide(i)
        u = v if act == S.FULL else cache.skip()
        if act == S.FULL:
            cache.full(v)
        x = O.euler_update(x, u, sig[i], sig[i + 1])
    np.testing.assert_allclose(x, x_ref, rtol=0, atol=1e-12)


class _TinyModel:
    """A tiny seeded model object for the probe (shape + conditioning + one layer)."""

    def __init__(self, zero_mod=False):
        from synthetic import configs as C
        from synthetic import gen as G
        self.shape = C.TINY_LOOP
        inp = G.loop_inputs(self.shape)
        for n in ("t_w1", "t_b1", "t_w2", "t_b2", "in_w", "in_b", "text", "txt_valid"):
            setattr(self, n, getattr(inp, n))
        self._l0 = dict(inp.layer(0))
        if zero_mod:
            self._l0["mod_w"] = np.zeros_like(self._l0["mod_w"])
            self._l0["mod_b"] = np.zeros_like(self._l0["mod_b"])

    def layer(self, l):
        assert l == 0
        return self._l0


def test_probe_features_are_block0_modulated_input():
    from synthetic import gen as G
    m = _TinyModel()
    b = m.shape.block
    lat = O.bf16_decode(G.normal_bf16(5, (1, b.n_vis, m.shape.latent_channels)))
    h = S.probe_features(m, lat, 0.7)
    # the same tokens through the block: its first intermediate is the probe's signal
    s, x = O.step_tokens(m, lat, 0.7)
    w = m.layer(0)
    mod = O.round_bf16(O.linear(s, O.bf16_decode(w["mod_w"]), O.bf16_decode(w["mod_b"])))
    inp = dict(w)
    inp["x"], inp["mod"], inp["txt_valid"] = x, np.broadcast_to(mod.reshape(6, -1), (b.batch, 6, b.hidden)), m.txt_valid
    _, keep = O.block_forward(inp, b, keep=True)
    np.testing.assert_array_equal(h, keep["h"])
    # same latent and timestep: no change; text rows do not see the latent
    assert S.rel_l1(h, S.probe_features(m, lat, 0.7)) == 0.0
    h2 = S.probe_features(m, 2.0 * lat, 0.7)
    np.testing.assert_array_equal(h2[:, b.n_vis:], h[:, b.n_vis:])
    assert S.rel_l1(h2, h) > 0.0


def test_probe_with_zero_modulation_is_layernorm():
    from synthetic import gen as G
    m = _TinyModel(zero_mod=True)
    b = m.shape.block
    lat = O.bf16_decode(G.normal_bf16(6, (1, b.n_vis, m.shape.latent_channels)))
    h = S.probe_features(m, lat, 0.3, round_points=False)
    np.testing.assert_allclose(h.mean(axis=-1), 0.0, atol=1e-12)
    var = h.var(axis=-1)
    # x / sqrt(var + eps): variance var / (var + eps) of every token row
    _, x = O.step_tokens(m, lat, 0.3, round_points=False)
    vx = x.var(axis=-1)
    np.testing.assert_allclose(var, vx / (vx + b.ln_eps), rtol=1e-12)


@pytest.mark.parametrize("cfg", [True, False])
def test_cached_denoise_step_full_and_skip(cfg):
    """FULL is the plain denoising step (and records the used velocity);
    SKIP moves the latent with 2 v_1 - v_0 (the last two used velocities)."""
    from synthetic import gen as G
    from tests.test_oracle_loop import _Model, _tiny
    shape = _tiny(cfg)
    m = _Model(shape)
    Bl = 1 if cfg else shape.block.batch
    lat0 = O.bf16_decode(G.normal_bf16(9, (Bl, shape.block.n_vis, 4)))
    sig = [1.0, 0.75, 0.5, 0.25]  # exact in fp32
    cache = S.OutputCache()
    x, sc0 = S.cached_denoise_step(m, lat0, sig[0], sig[1], 3.0, S.FULL, cache)
    want, v0 = O.denoise_step(m, lat0, sig[0], sig[1], 3.0)
    np.testing.assert_array_equal(x, want)
    assert sc0 == math.inf
    u0 = O.cfg_combine(v0[0:1], v0[1:2], 3.0) if cfg else v0
    x1, sc1 = S.cached_denoise_step(m, x, sig[1], sig[2], 3.0, S.FULL, cache)
    _, v1 = O.denoise_step(m, x, sig[1], sig[2], 3.0)
    u1 = O.cfg_combine(v1[0:1], v1[1:2], 3.0) if cfg else v1
    assert sc1 == pytest.approx(np.abs(u1 - u0).sum() / np.abs(u0).sum(), rel=1e-12)
    x2, sc2 = S.cached_denoise_step(m, x1, sig[2], sig[3], 3.0, S.SKIP, cache)
    assert sc2 is None
    np.testing.assert_allclose(x2, x1 + (sig[3] - sig[2]) * (2 * u1 - u0), rtol=0, atol=1e-12)
