"""The library's host-side step-cache controller (dit_cache_ctrl_*, C) against
the oracle's controller (Python), which is itself pinned by the pages' worked
numbers: the same policies and score sequences must give identical FULL/SKIP
decisions, step by step.  Runs on the CPU (no device work)."""

import json
import math
import os

import numpy as np
import pytest

import diffusion_transformer_denoising_dit_amd as D
from oracle import stepcache as S

MODES = {D.CACHE_OFF: S.OFF, D.CACHE_CADENCE: S.CADENCE, D.CACHE_ONLINE_DELTA: S.ONLINE_DELTA,
         D.CACHE_TEACACHE: S.TEACACHE}
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "stepcache_worked_examples.json")))


def _both(mode, n, warmup, cooldown, cadence=2, alpha=0.6, threshold=0.0, coef=(1.0, 0.0)):
    c = D.CacheController(D.cache_policy(mode, n, warmup, cooldown, cadence, alpha, threshold, coef))
    o = S.Controller(MODES[mode], n, warmup=warmup, cooldown=cooldown, cadence=cadence, alpha=alpha,
                     threshold=threshold, coef=coef)
    return c, o


def _run(c, o, probe, change):
    """Drive both controllers with fp32 scores; returns the two action lists."""
    ca, oa = [], []
    for i in range(len(probe)):
        p = float(np.float32(probe[i]))
        a = c.decide(i, p)
        b = o.decide(i, p)
        ca.append(a)
        oa.append(b)
        if a == D.STEP_FULL:
            c.observe(float(np.float32(change[i])))
        if b == S.FULL:
            o.observe(float(np.float32(change[i])))
    return ca, oa


@pytest.mark.parametrize("mode", [D.CACHE_OFF, D.CACHE_CADENCE, D.CACHE_ONLINE_DELTA,
                                  D.CACHE_TEACACHE])
def test_controller_matches_oracle_on_random_schedules(mode):
    rng = np.random.default_rng(100 + mode)
    for trial in range(300):
        n = int(rng.integers(1, 70))
        w, cd = int(rng.integers(0, 7)), int(rng.integers(0, 7))
        cad = int(rng.integers(1, 5))
        alpha = float(rng.uniform(0.1, 1.2))
        thr = float(rng.uniform(0.01, 0.5))
        coef = tuple(float(x) for x in rng.uniform(-1, 1, int(rng.integers(1, 5))))
        probe = [math.inf] + list(rng.exponential(0.05, n - 1))
        if trial % 7 == 0 and n > 3:
            probe[int(rng.integers(1, n))] = math.inf           # a lost probe mid-run
        change = [math.inf] + list(rng.exponential(0.1, n - 1))
        c, o = _both(mode, n, w, cd, cad, alpha, thr, coef)
        ca, oa = _run(c, o, probe, change)
        assert ca == oa, (trial, n, w, cd, cad, alpha, thr, coef)


@pytest.mark.parametrize("case", GOLDEN["teacache_accumulator"]["cases"])
def test_controller_teacache_worked_example(case):
    c = D.CacheController(D.cache_policy(D.CACHE_TEACACHE, 40, 2, 0,
                                         threshold=GOLDEN["teacache_accumulator"]["threshold"]))
    acts = [c.decide(0, math.inf)] + [c.decide(i, case["rescaled_distance"]) for i in range(1, 40)]
    k = case["consecutive_skips"]
    assert acts[2:2 + 3 * (k + 1)] == ([D.STEP_SKIP] * k + [D.STEP_FULL]) * 3


@pytest.mark.parametrize("case", GOLDEN["fixed_cadence"]["cases"])
def test_controller_cadence_counts(case):
    g = GOLDEN["fixed_cadence"]
    c = D.CacheController(D.cache_policy(D.CACHE_CADENCE, case["n_steps"], g["warmup"], g["cooldown"],
                                         g["cadence"]))
    acts = [c.decide(i) for i in range(case["n_steps"])]
    assert acts.count(D.STEP_SKIP) == case["skips"]


def test_controller_argument_errors():
    bad = [D.cache_policy(7, 10), D.cache_policy(D.CACHE_CADENCE, 0),
           D.cache_policy(D.CACHE_CADENCE, 10, -1), D.cache_policy(D.CACHE_CADENCE, 10, cadence=0),
           D.cache_policy(D.CACHE_ONLINE_DELTA, 10, alpha=-0.5),
           D.cache_policy(D.CACHE_TEACACHE, 10, threshold=math.nan),
           D.cache_policy(D.CACHE_TEACACHE, 10, coef=())]
    for p in bad:
        with pytest.raises(D.DitError) as e:
            D.CacheController(p)
        assert e.value.status_name == "DIT_EINVAL"
    c = D.CacheController(D.cache_policy(D.CACHE_CADENCE, 3))
    c.decide(0)
    with pytest.raises(D.DitError):
        c.decide(2)               # out of order
    c.decide(1)
    c.decide(2)
    with pytest.raises(D.DitError):
        c.decide(3)               # past n_steps
