"""Step caching written out plainly (test infrastructure only; see the
package docstring).

Sources (web pages; cited by title and section):

* "Difflet" paper, section 5 Adaptive Step Caching on Trainium: nearby steps
  give similar denoiser outputs; a full execution measures the change of its
  output against the previously used output and saves the new output; a
  cached step adds the saved change to the previous output and keeps the
  estimate as the next previous output; both paths apply the same latent
  update.  Three modes: fixed cadence, calibrated adaptive (a probe computes a
  feature-change score on the device, a fitted curve turns it into an
  estimated output change, compared per step or accumulated against a
  threshold, a full step resets the sum), online-delta (at a full step the
  output change is compared with alpha times the first change measured in the
  generation; below it the next step is cached, and a cached step is always
  followed by a full one).  All modes keep initial and final full steps.
  Section 7.5: cadence 2 with 5 initial and 5 final full steps skips 20 of 50
  steps and 15 of 40; online-delta's default alpha is 0.6.
* "Difflet Engineering Report", DiT caching: adaptive TeaCache, online delta,
  and fixed cadence: warmup, cooldown and two completed full steps are needed
  before a skip; the probe measures the change of block 0's modulated input;
  fixed cadence skips by step index inside the warmup/cooldown window.
* "19. Diffusion, Image, Video, and World Models", Inside TeaCache's skip
  decision: the signal is the modulated input (after timestep conditioning);
  its change is the relative L1 distance mean|cur - prev| / mean|prev|; a
  per-model polynomial rescales it; the running sum since the last real
  compute is the decision variable; crossing the threshold computes and
  resets; boundary steps always compute; a missing previous input forces a
  compute.  Worked numbers: rescaled distances of 0.02 against a threshold
  of 0.15 skip seven steps in a row, 0.06 skip two.

Readings taken where the pages leave a point open (each also listed with
the design notes):

* The saved change is the difference between the new full output and the
  previously *used* output (which may be an estimate), as section 5 of the
  paper states; the engineering report's "two most recent full predictions"
  coincides with it whenever no skip lies between them.
* Fixed cadence c: inside the window [warmup, n_steps - cooldown) step i is
  computed when (i - warmup) is a multiple of c and cached otherwise (c = 2:
  compute, skip, compute, ...).
* The TeaCache accumulator is compared with ">= threshold" (crossing) and is
  reset to 0 by every full step, whatever caused it.
* A probe with no saved features reports an infinite change (fails open).
* The relative L1 change of an all-zero reference is 0 when the new array
  is also zero, else infinite.
"""

from __future__ import annotations

import numpy as np

from .dit import _dec, adaln_modulate, linear, round_bf16, step_tokens

FULL, SKIP = 0, 1
OFF, CADENCE, ONLINE_DELTA, TEACACHE = 0, 1, 2, 3


def rel_l1(cur, prev):
    """Relative L1 change of ``cur`` against ``prev``: mean|cur - prev| /
    mean|prev| ("19. Diffusion, Image, Video, and World Models", Inside
    TeaCache's skip decision), in fp64.  The two means share the element
    count, so this is the ratio of the two sums."""
    cur = np.asarray(cur, dtype=np.float64).ravel()
    prev = np.asarray(prev, dtype=np.float64).ravel()
    num = np.abs(cur - prev).sum()
    den = np.abs(prev).sum()
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return float(num / den)


class OutputCache:
    """The output estimator of "Difflet" section 5: state is the previously
    used output and the most recently measured change."""

    def __init__(self):
        self.prev = None
        self.delta = None

    def full(self, v):
        """A full execution produced ``v``: measure the change against the
        previously used output, save both; returns the relative L1 change
        (infinite when nothing was used before)."""
        v = np.asarray(v, dtype=np.float64)
        if self.prev is None:
            score = np.inf
        else:
            self.delta = v - self.prev
            score = rel_l1(v, self.prev)
        self.prev = v
        return score

    def skip(self):
        """A cached step: previous output plus the saved change, which
        becomes the previous output of the next step."""
        if self.prev is None or self.delta is None:
            raise ValueError("a cached step needs a previous output and a measured change")
        v = self.prev + self.delta
        self.prev = v
        return v


class Controller:
    """Host-side skip decision for one generation ("Difflet" section 5;
    "Difflet Engineering Report", DiT caching).  Call ``decide`` for steps
    0, 1, ... in order and, after every full step, ``observe`` with the output
    change that step measured."""

    def __init__(self, mode, n_steps, warmup=0, cooldown=0, cadence=2, alpha=0.6,
                 threshold=0.0, coef=(1.0, 0.0)):
        self.mode, self.n_steps = mode, n_steps
        self.warmup, self.cooldown, self.cadence = warmup, cooldown, cadence
        self.alpha, self.threshold = alpha, threshold
        self.coef = list(coef)          # highest degree first
        self.n_full = 0                 # completed full steps
        self.last_skipped = False
        self.skip_next = False          # online-delta: the last full step asked for a skip
        self.first_change = None        # online-delta: first output change of the generation
        self.acc = 0.0                  # TeaCache: rescaled change summed since the last full step
        self.step = 0

    def rescale(self, r):
        """The fitted polynomial applied to a probe score (Horner's rule)."""
        y = 0.0
        for c in self.coef:
            y = y * r + c
        return y

    def decide(self, step, probe_score=None):
        if step != self.step:
            raise ValueError(f"steps must be decided in order: expected {self.step}, got {step}")
        self.step += 1
        boundary = step < self.warmup or step >= self.n_steps - self.cooldown
        allowed = not boundary and self.n_full >= 2
        if self.mode == OFF:
            skip = False
        elif self.mode == CADENCE:
            skip = allowed and (step - self.warmup) % self.cadence != 0
        elif self.mode == ONLINE_DELTA:
            skip = allowed and not self.last_skipped and self.skip_next
        elif self.mode == TEACACHE:
            if probe_score is None or not np.isfinite(probe_score):
                skip = False            # no previous features: compute
            else:
                self.acc += self.rescale(float(probe_score))
                skip = allowed and self.acc < self.threshold
        else:
            raise ValueError(f"unknown mode {self.mode}")
        if skip:
            self.last_skipped = True
            self.skip_next = False
            return SKIP
        self.last_skipped = False
        self.acc = 0.0
        self.n_full += 1
        return FULL

    def observe(self, output_change):
        """The output change measured by the full step just decided."""
        if self.mode != ONLINE_DELTA or not np.isfinite(output_change):
            return
        if self.first_change is None:
            self.first_change = float(output_change)
        self.skip_next = float(output_change) < self.alpha * self.first_change


def decisions(controller, probe_scores=None, output_changes=None):
    """Run a controller over a whole schedule with given per-step scores
    (the probe score of step i, the output change a full step i would
    measure); returns the list of FULL/SKIP actions."""
    acts = []
    for i in range(controller.n_steps):
        p = None if probe_scores is None else probe_scores[i]
        a = controller.decide(i, p)
        acts.append(a)
        if a == FULL and output_changes is not None:
            controller.observe(output_changes[i])
    return acts


def probe_features(model, latent, sigma, round_points=True, t_scale=1000.0):
    """The probe's signal: block 0's modulated input for this latent and
    timestep ("Difflet" section 5: the denoiser's input projection and the
    first block's normalisation and modulation, stopping before attention).
    Returns h = adaLN(x; shift1, scale1) of every token, [B, N, D]."""
    R_ = round_bf16 if round_points else (lambda a: a)
    blk = model.shape.block
    D = blk.hidden
    s, x = step_tokens(model, latent, sigma, round_points, t_scale)
    w = model.layer(0)
    mod = R_(linear(s, _dec(w["mod_w"]), _dec(w["mod_b"]))).reshape(6, D)
    return R_(adaln_modulate(x, mod[0], mod[1], blk.ln_eps))


def cached_denoise_step(model, latent, sigma, sigma_next, guidance, action, cache,
                        round_points=True):
    """One step of the denoising loop under step caching ("Difflet" section
    5: both paths apply the same latent update).  FULL runs the denoiser
    (``dit.denoise_step``), combines the guidance branches and hands the used
    velocity to ``cache.full``; SKIP takes ``cache.skip()``'s estimate.
    Returns (new latent, output change measured by a full step or None)."""
    from .dit import cfg_combine, denoise_step, euler_update
    lat = np.asarray(latent, dtype=np.float64)
    s32 = float(np.float32(sigma))
    n32 = float(np.float32(sigma_next))
    if action == FULL:
        _, v = denoise_step(model, lat, sigma, sigma_next, guidance, round_points=round_points)
        v_hat = cfg_combine(v[0:1], v[1:2], guidance) if model.shape.cfg else v
        score = cache.full(v_hat)
        return euler_update(lat, v_hat, s32, n32), score
    if action == SKIP:
        return euler_update(lat, cache.skip(), s32, n32), None
    raise ValueError(f"unknown action {action}")
