"""Benchmark of the DiT denoiser hot path on one MI355X.

A step is one denoising step of a single-block video DiT at the 480p shape
(32,760 visual + 512 text tokens, 226 valid, hidden 5120, 40 heads x 128,
MLP 13824, batch 1): timestep conditioning, input projection, the block
(adaLN, QKV GEMM, Q/K RMSNorm + 3D RoPE, joint attention, output projection
with gated residual, GELU MLP with gated residual), final adaLN + projection
and the Euler update -- one call of dit_denoise_step.  Inputs are seeded
synthetic tensors already resident in HBM.

Prints ONE JSON line: ms/step (the value), the block alone, joint
attention's TFLOP/s against the bf16 dense MFMA peak (the roofline object),
split joint attention (a text partial plus 4 visual partials, merged), step
caching (probe, skipped step, change-score kernel, a 30-step cadence-2 loop),
the MM-DiT double- and single-stream blocks at the FLUX-like image shape,
the Wan-style block (self- plus cross-attention) at the c3 video shape, the
block's four GEMMs alone (beside torch's hipBLASLt matmul of the same shapes,
for reference), plus the CPU oracle timed on a bounded sample of the same step.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--gemm-only]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DiT block ms/step + joint-attn TFLOP/s (% bf16 MFMA peak) @32760+512 tok"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (no sparsity)

# HBM traffic of one c3 joint-attention call (the attention kernel and the
# merge of its split last round) from two rocprofv3 counter passes
# (FETCH_SIZE, then WRITE_SIZE, of `bench.py --traffic-probe`), scaled by what
# the same counters read for a plain 1 GiB device copy (FETCH x2.0, WRITE
# x1.0); summary and commands in profiles/attn_c3_hbm_traffic.md.  Valid only
# for the kernel source they were taken on.
ATTN_TRAFFIC = {
    "source_sha256": "36de9ff5cc4916a5f0abf43eacb27e7d84ba19c4071fe628692982e9c974185c",
    "fetch_bytes": 3.8461e9,
    "write_bytes": 0.3765e9,
    "fetch_scale": 2.0,
    "write_scale": 1.0,
    "profile": "profiles/attn_c3_hbm_traffic.md",
}
ATTN_SOURCES = ("diffusion_transformer_denoising_dit_amd/csrc/attention.hip",
                "diffusion_transformer_denoising_dit_amd/csrc/common.h")


def attn_traffic():
    """Counter-measured bytes per attention launch, or None once the kernel
    source differs from the one the counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != ATTN_TRAFFIC["source_sha256"]:
        return None
    return ATTN_TRAFFIC
BLOCK_NAMES = ("w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "w_up", "b_up", "w_dn", "b_dn")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--traffic-probe", action="store_true",
                   help="only launch c3 joint attention --steps times and a plain 1 GiB copy "
                        "--steps times (for hardware-counter runs), print nothing else")
    p.add_argument("--hbm-probe", action="store_true",
                   help="only launch the bandwidth-bound kernels at their workload sizes --steps "
                        "times each and a plain 1 GiB copy --steps times (for counter runs)")
    p.add_argument("--gemm-only", action="store_true",
                   help="time only the block's GEMMs (ours and hipBLASLt) and print them")
    p.add_argument("--cpu-rows", type=int, default=64,
                   help="query rows in the CPU oracle's bounded sample")
    return p.parse_args()


def dev_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def attention_flops(n_tok, n_valid_keys, heads, head_dim, batch=1):
    """Algorithmic FLOPs of joint attention: QK^T and PV over the valid keys
    of every query row (2 * 2 * d per query-key pair and head)."""
    return 4.0 * batch * heads * head_dim * n_tok * n_valid_keys


def block_flops(s, valid):
    M = s.batch * s.n_tok
    D, F = s.hidden, s.mlp
    gemm = 2.0 * M * D * (3 * D) + 2.0 * M * D * D + 2.0 * M * D * F * 2
    attn = sum(attention_flops(s.n_tok, s.n_vis + int(L), s.heads, s.head_dim) for L in valid)
    return gemm + attn


def timed(fn, reps, stream):
    """Average ms of `fn` over `reps` calls, HIP events on the launch stream."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / reps


class ClockSampler:
    """Samples the GPU's current shader clock (the starred level of the
    driver's pp_dpm_sclk) every 20 ms on a background thread while a timed
    region runs; the MI355X runs below its 2.4 GHz peak under load (power
    limit), which the roofline fractions against the nominal peak include.
    Reading that file asks the power-management firmware; at a 5 ms period
    it stretched a 30-call run of the 2.3 ms c2 block from 2.27 to 2.34 ms
    per call (p90 2.30 -> 2.44), so after a first read 5 ms into the region
    (short regions still get one) the period is kept long."""

    def __init__(self, period_s=0.02, first_s=0.005):
        self.first = first_s
        import glob
        self.path = next(iter(sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))), None)
        self.period = period_s
        self.samples = []

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().split("M")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def __enter__(self):
        import threading
        self.samples = []
        self._stop = threading.Event()
        if self.path:
            def run():
                wait = self.first
                while not self._stop.wait(wait):
                    v = self._read()
                    if v is not None:
                        self.samples.append(v)
                    wait = self.period
            self._t = threading.Thread(target=run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._t.join()

    def summary(self):
        import numpy as np
        busy = [v for v in self.samples if v >= 500]  # drop idle readings between launches
        if not busy:
            return None
        a = np.asarray(busy, dtype=np.float64)
        return {"median_mhz": int(np.median(a)), "p10_mhz": int(np.percentile(a, 10)),
                "p90_mhz": int(np.percentile(a, 90)), "samples": len(busy)}


def timed_stats(fn, reps, stream, drop_first=False):
    """Per-call ms of `fn` over `reps` back-to-back calls (a HIP event between
    consecutive calls on the launch stream): mean, median, p10, p90 (of the
    calls after the first with drop_first), plus the shader clock sampled
    while they ran."""
    import numpy as np
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        ev[0].record(stream)
        for i in range(reps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
    per = np.asarray([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])
    total = ev[0].elapsed_time(ev[reps])
    if drop_first:
        per = per[1:]
    return {"ms": round(total / reps, 4), "median_ms": round(float(np.median(per)), 4),
            "p10_ms": round(float(np.percentile(per, 10)), 4),
            "p90_ms": round(float(np.percentile(per, 90)), 4), "reps": reps,
            "clock": clk.summary()}


def cpu_baseline(shape, model, n_rows):
    """The oracle's denoising step (fp64 NumPy, as it stands) on a bounded
    sample: n_rows seeded query rows, with keys and values computed for every
    token.  The full-step figure scales the measured time by the ratio of
    algorithmic FLOPs (full step / sample); the oracle's materialised-softmax
    attention runs slower than its BLAS GEMMs, so this underestimates a full
    oracle step."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:  # noqa: BLE001
        threads = 1
    b = shape.block
    sig = O.sigma_schedule(shape.steps)
    lat = O.bf16_decode(model["latent"]).reshape(1, b.n_vis, shape.latent_channels)
    rng = np.random.default_rng(0xD17 + n_rows)
    rows = np.sort(rng.choice(b.n_vis, size=n_rows, replace=False))
    t0 = time.perf_counter()
    O.denoise_step(model["oracle_view"], lat, sig[0], sig[1], shape.guidance, rows=rows)
    t = time.perf_counter() - t0
    D, F, C = b.hidden, b.mlp, shape.latent_channels
    nk = b.n_vis + int(model["oracle_view"].txt_valid[0])
    per_row = (2.0 * D * D * 2 + 2.0 * D * F * 2 + 4.0 * b.heads * b.head_dim * nk
               + 2.0 * C * D * 2)
    kv_all = 2.0 * b.n_tok * D * 2 * D
    f_sample = kv_all + n_rows * per_row
    f_full = kv_all + b.n_tok * per_row
    return {"value": round(t * f_full / f_sample * 1e3, 1), "unit": "ms/step (extrapolated)",
            "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 NumPy oracle, one c3 denoising step restricted to {n_rows} seeded query "
                       f"rows (keys/values for all {b.n_tok} tokens): {t:.1f} s measured; scaled by "
                       f"algorithmic FLOPs x{f_full / f_sample:.1f} to the full step (an "
                       "underestimate: the oracle's attention is slower than its GEMMs)"),
            "measured_s": round(t, 2),
            "affinity_cores": len(os.sched_getaffinity(0))}


def traffic_probe(steps):
    """The kernels a hardware-counter pass needs and nothing else: joint
    attention at the c3 shape (q/k/v as column blocks of one [N, 3*H*d]
    buffer, as in the block), then a plain device copy of exactly 1 GiB read +
    1 GiB written, whose FETCH_SIZE / WRITE_SIZE calibrate the counters."""
    import torch

    import diffusion_transformer_denoising_dit_amd as D
    from synthetic import configs as C
    blk = C.C3_STEP.block
    HD = blk.hidden
    g = torch.Generator("cuda").manual_seed(5)
    qkv = torch.randn((blk.batch, blk.n_tok, 3 * HD), generator=g, device="cuda").to(torch.bfloat16)
    o = torch.empty((blk.batch, blk.n_tok, HD), dtype=torch.bfloat16, device="cuda")
    adesc = D.attn_desc(blk.batch, blk.n_vis, blk.n_txt, blk.heads, blk.head_dim, [226])
    wsb = D.dit_joint_attention_workspace_bytes()
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    for _ in range(steps):
        D.dit_joint_attention(adesc, qkv, qkv[..., HD:], qkv[..., 2 * HD:], 3 * HD, o, HD,
                              workspace=ws, workspace_bytes=wsb)
    torch.cuda.synchronize()
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[traffic-probe] {steps} attention launches + {steps} copies of 1 GiB done",
          file=sys.stderr, flush=True)


HBM_KERNELS = ("adaln", "qk_rmsnorm_rope", "merge5", "change_score", "modulation_gemv", "euler_c5")


def hbm_probe(steps, reps=None):
    """The bandwidth-bound kernels at their c3 (Euler: c5) sizes, each
    launched `steps` times, then a plain device copy of exactly 1 GiB read +
    1 GiB written (the counter calibration).  With `reps`, time each kernel
    (HIP events, mean of `reps` calls) and return algorithmic bytes and GB/s.
    Algorithmic bytes per launch:
      adaLN: fp32 x read + bf16 h written, 6 B per element of [33272, 5120];
      Q/K RMSNorm + RoPE: q and k read and written in place, bf16, 8 B per
        (q, k) element pair of [33272, 5120];
      merge of 5 partials: 5 fp32 outputs read + bf16 written per element
        ((4*5 + 2) B) plus 5 fp32 LSE per (row, head);
      change score with update: bf16 current read, saved read and written
        (6 B per element of [33272, 5120]);
      modulation matrix-vector (one timestep row through the [30720, 5120]
        modulation projection): the bf16 weight read once, 2 B per element;
      CFG + Euler at the c5 latent (4096 x 64): v_c, v_u bf16 read, x fp32
        read and written, 12 B per element."""
    import torch

    import diffusion_transformer_denoising_dit_amd as D
    from synthetic import configs as C
    blk = C.C3_STEP.block
    M, HD = blk.batch * blk.n_tok, blk.hidden
    g = torch.Generator("cuda").manual_seed(21)

    def rnd(*shape, std=1.0):
        return (torch.randn(shape, generator=g, device="cuda") * std).to(torch.bfloat16)

    x = torch.randn((M, HD), generator=g, device="cuda")
    h = torch.empty((M, HD), dtype=torch.bfloat16, device="cuda")
    mod = rnd(6, HD, std=0.1)
    qkv = rnd(M, 3 * HD)
    gq, gk = rnd(HD, std=0.02) + 1, rnd(HD, std=0.02) + 1
    bdesc = D.block_desc(blk, [226], 0)
    P = 5
    outs = [torch.randn((M, HD), generator=g, device="cuda") for _ in range(P)]
    lses = [torch.randn((blk.batch, blk.heads, blk.n_tok), generator=g, device="cuda") for _ in range(P)]
    o = torch.empty((M, HD), dtype=torch.bfloat16, device="cuda")
    feat = rnd(M * HD)
    saved = rnd(M * HD)
    sws = torch.empty(D.dit_change_score_workspace_bytes(), dtype=torch.uint8, device="cuda")
    score = torch.zeros(1, device="cuda")
    wmod, bmod = rnd(6 * HD, HD, std=0.02), rnd(6 * HD, std=0.02)
    srow, mrow = rnd(1, HD), torch.empty((1, 6 * HD), dtype=torch.bfloat16, device="cuda")
    n_lat = 4096 * 64
    vc, vu = rnd(n_lat), rnd(n_lat)
    xl = torch.zeros(n_lat, device="cuda")
    kern = {
        "adaln": (lambda: D.dit_adaln_modulate(x, M, HD, blk.n_tok, mod[0], mod[1], 0, 1e-6, h),
                  6.0 * M * HD),
        "qk_rmsnorm_rope": (lambda: D.dit_qk_rmsnorm_rope(bdesc, qkv, 3 * HD, gq, gk), 8.0 * M * HD),
        "merge5": (lambda: D.dit_attention_merge(blk.batch, blk.n_tok, blk.heads, blk.head_dim, outs,
                                                 HD, lses, o, HD),
                   (4.0 * P + 2) * M * HD + 4.0 * P * blk.batch * blk.heads * blk.n_tok),
        "change_score": (lambda: D.dit_change_score(feat, saved, D.DTYPE_BF16, M * HD, 1, score, sws,
                                                    sws.numel()), 6.0 * M * HD),
        "modulation_gemv": (lambda: D.dit_linear(srow, HD, wmod, bmod, 1, 6 * HD, HD, D.EPI_BF16,
                                                 mrow, 6 * HD), 2.0 * 6 * HD * HD),
        "euler_c5": (lambda: D.dit_euler_step(xl, vc, vu, n_lat, 5.0, 0.5, 0.5 - 1.0 / 30),
                     12.0 * n_lat),
    }
    result = {}
    for name in HBM_KERNELS:
        fn, nbytes = kern[name]
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        if reps:
            st = timed_stats(fn, reps, torch.cuda.current_stream())
            ms = st["ms"]
            result[name] = {"us": round(ms * 1e3, 2), "algorithmic_bytes": int(nbytes),
                            "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 8e12, 4), "timing": st}
    del x, h, qkv, outs, lses, o, feat, saved, wmod
    torch.cuda.empty_cache()
    if not reps:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[hbm-probe] {len(HBM_KERNELS)} kernels x {steps} launches + {steps} copies of 1 GiB "
              "done", file=sys.stderr, flush=True)
    return result


def block_gemms(reps, stream):
    """The DiT block's four large GEMMs at the c3 shape (33,272 tokens, hidden
    5120, MLP 13824), each through dit_linear with the epilogue and the K-split
    scratch the block uses, and beside each the same product as a plain torch
    matmul (hipBLASLt, no epilogue) for reference.  Seeded N(0,1) activations,
    N(0, 0.02) weights."""
    import torch

    import diffusion_transformer_denoising_dit_amd as D
    from synthetic import configs as C
    blk = C.C3_STEP.block
    M, Dh, F = blk.batch * blk.n_tok, blk.hidden, blk.mlp
    g = torch.Generator("cuda").manual_seed(13)
    wsb = D.dit_linear_workspace_bytes()
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = {}
    for name, n, k, epi in (("qkv", 3 * Dh, Dh, D.EPI_BF16), ("out_proj", Dh, Dh, D.EPI_GATED_RES_F32),
                            ("mlp_up", F, Dh, D.EPI_GELU_BF16), ("mlp_down", Dh, F, D.EPI_GATED_RES_F32)):
        a = torch.randn((M, k), generator=g, device="cuda").to(torch.bfloat16)
        w = (torch.randn((n, k), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        bias = (torch.randn((n,), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        gated = epi == D.EPI_GATED_RES_F32
        y = torch.zeros((M, n), dtype=torch.float32 if gated else torch.bfloat16, device="cuda")
        gate = torch.randn((1, n), generator=g, device="cuda").to(torch.bfloat16) if gated else None

        def ours():
            D.dit_linear(a, k, w, bias, M, n, k, epi, y, n, gate=gate, gate_stride=n, gate_rows=M,
                         workspace=ws, workspace_bytes=wsb)

        wt = w.t()

        def ref():
            torch.matmul(a, wt)

        ours()
        ref()
        flop = 2.0 * M * n * k
        st_o = timed_stats(ours, reps, stream)
        st_r = timed_stats(ref, reps, stream)
        ms_o, ms_r = st_o["ms"], st_r["ms"]
        out[name] = {"m": M, "n": n, "k": k, "ms": round(ms_o, 3),
                     "tflops": round(flop / (ms_o * 1e-3) / 1e12, 1),
                     "hipblaslt_ms": round(ms_r, 3),
                     "hipblaslt_tflops": round(flop / (ms_r * 1e-3) / 1e12, 1),
                     "timing": st_o, "hipblaslt_timing": st_r}
        del a, w, bias, y, gate, wt
    del ws
    torch.cuda.empty_cache()
    return out


def mmdit_blocks(reps, stream):
    """MM-DiT double-stream and single-stream blocks at the FLUX-like image
    shape (4096 image + 512 text tokens, hidden 3072, 24 heads x 128, MLP
    12288, CFG batch 2 with valid text lengths 77 and 512): ms and TFLOP/s of
    one block.  Seeded N(0,1) activations and modulation, N(0, 0.02) weights,
    drawn on the device."""
    import torch

    import diffusion_transformer_denoising_dit_amd as D
    from synthetic import configs as C
    s = C.C2
    B, S, L, Dh, F = s.batch, s.n_vis, s.n_txt, s.hidden, s.mlp
    valid = [77, 512]
    g = torch.Generator("cuda").manual_seed(11)

    def rnd(*shape, std=1.0):
        return (torch.randn(shape, generator=g, device="cuda") * std).to(torch.bfloat16)

    def block_w():
        return {"w_qkv": rnd(3 * Dh, Dh, std=0.02), "b_qkv": rnd(3 * Dh, std=0.02),
                "g_q": 1 + rnd(Dh, std=0.02), "g_k": 1 + rnd(Dh, std=0.02),
                "w_o": rnd(Dh, Dh, std=0.02), "b_o": rnd(Dh, std=0.02),
                "w_up": rnd(F, Dh, std=0.02), "b_up": rnd(F, std=0.02),
                "w_dn": rnd(Dh, F, std=0.02), "b_dn": rnd(Dh, std=0.02)}

    attn = sum(attention_flops(S + L, S + v, s.heads, s.head_dim) for v in valid)
    out = {}
    # double stream
    desc = D.block_desc(s, valid, 6 * Dh)
    wi, wt = block_w(), block_w()
    mi, mt = rnd(B, 6, Dh), rnd(B, 6, Dh)
    xi = torch.randn((B, S, Dh), generator=g, device="cuda")
    xt = torch.randn((B, L, Dh), generator=g, device="cuda")
    nb = D.dit_double_block_workspace_bytes(desc)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    bwi, bwt = D.block_weights(wi), D.block_weights(wt)

    def dbl():
        D.dit_double_block_forward(desc, bwi, bwt, mi, mt, xi, xt, ws, nb)

    dbl()
    st = timed_stats(dbl, max(30, reps), stream)
    ms = st["ms"]
    M = B * (S + L)
    fl = 2.0 * M * Dh * 4 * Dh + 2.0 * M * Dh * F * 2 + attn
    out["double_block"] = {"ms": round(ms, 3), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                           "algorithmic_tflop": round(fl / 1e12, 3), "timing": st}
    del wi, wt, bwi, bwt, xi, xt, ws
    # single stream
    desc = D.block_desc(s, valid, 3 * Dh)
    w = {"w1": rnd(3 * Dh + F, Dh, std=0.02), "b1": rnd(3 * Dh + F, std=0.02),
         "g_q": 1 + rnd(Dh, std=0.02), "g_k": 1 + rnd(Dh, std=0.02),
         "w2": rnd(Dh, Dh + F, std=0.02), "b2": rnd(Dh, std=0.02)}
    sw = D.single_block_weights(w)
    mod = rnd(B, 3, Dh)
    x = torch.randn((B, S + L, Dh), generator=g, device="cuda")
    nb = D.dit_single_block_workspace_bytes(desc)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def sgl():
        D.dit_single_block_forward(desc, sw, mod, x, ws, nb)

    sgl()
    st = timed_stats(sgl, max(30, reps), stream)
    ms = st["ms"]
    fl = 2.0 * M * Dh * (3 * Dh + F) + 2.0 * M * (Dh + F) * Dh + attn
    out["single_block"] = {"ms": round(ms, 3), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                           "algorithmic_tflop": round(fl / 1e12, 3), "timing": st}
    out["shape"] = ("FLUX-like 1024x1024: 4096 image + 512 text tokens (valid 77, 512), hidden 3072, "
                    "24x128, MLP 12288, batch 2")
    return out


def other_configs(reps, stream):
    """ms and TFLOP/s of the other workloads, each through the same entry
    points: the DiT block at the tiny shape (256 + 32 tokens, hidden 256) and
    at the FLUX-like image shape (CFG batch 2, 4096 + 512 tokens, hidden 3072),
    joint attention alone at the Wan-like 720p shape (75600 + 512 tokens, 300
    valid, 40 heads x 128), and the full denoising loop (24-block image DiT,
    CFG batch 2, guidance 5, 30 Euler steps from sigma 1 to 0) as end-to-end
    ms per step.  Valid text lengths are the seeded draws of the parity
    inputs; activations N(0,1) and weights N(0, 0.02) are drawn on the device
    (timing does not depend on the values)."""
    import torch

    import diffusion_transformer_denoising_dit_amd as D
    from synthetic import configs as C
    from synthetic import gen as G
    g = torch.Generator("cuda").manual_seed(12)

    def rnd(*shape, std=1.0, mean=0.0):
        return (torch.randn(shape, generator=g, device="cuda") * std + mean).to(torch.bfloat16)

    def block_w(Dh, F):
        return {"w_qkv": rnd(3 * Dh, Dh, std=0.02), "b_qkv": rnd(3 * Dh, std=0.02),
                "g_q": rnd(Dh, std=0.02, mean=1.0), "g_k": rnd(Dh, std=0.02, mean=1.0),
                "w_o": rnd(Dh, Dh, std=0.02), "b_o": rnd(Dh, std=0.02),
                "w_up": rnd(F, Dh, std=0.02), "b_up": rnd(F, std=0.02),
                "w_dn": rnd(Dh, F, std=0.02), "b_dn": rnd(Dh, std=0.02)}

    out = {}
    for key, s, valid in (("c1_block", C.C1, [20]),
                          ("c2_block", C.C2, [int(v) for v in G.block_inputs(C.C2, weights=False)["txt_valid"]])):
        desc = D.block_desc(s, valid)
        w = block_w(s.hidden, s.mlp)
        mod = rnd(s.batch, 6, s.hidden)
        x = torch.randn((s.batch, s.n_tok, s.hidden), generator=g, device="cuda")
        nb = D.dit_block_workspace_bytes(desc)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

        def blk(desc=desc, w=w, mod=mod, x=x, ws=ws, nb=nb):
            D.dit_block_forward(desc, w, mod, x, ws, nb)

        blk()
        st = timed_stats(blk, max(30, reps), stream)
        ms = st["ms"]
        fl = block_flops(s, valid)
        out[key] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                    "algorithmic_tflop": round(fl / 1e12, 4), "txt_valid": valid, "timing": st}
        del w, mod, x, ws

    s = C.C4
    HD = s.heads * s.head_dim
    q, k, v = (rnd(s.batch, s.n_tok, HD) for _ in range(3))
    o = torch.empty_like(q)
    adesc = D.attn_desc(s.batch, s.n_vis, s.n_txt, s.heads, s.head_dim, [300])
    a_wsb = D.dit_joint_attention_workspace_bytes()
    a_ws = torch.empty(a_wsb, dtype=torch.uint8, device="cuda")

    def attn():
        # (11920 query tiles on 256 CUs: a last round of 144, split 3 ways)
        D.dit_joint_attention(adesc, q, k, v, HD, o, HD, workspace=a_ws, workspace_bytes=a_wsb)

    attn()
    st = timed_stats(attn, max(3, reps // 2), stream)
    ms = st["ms"]
    fl = attention_flops(s.n_tok, s.n_vis + 300, s.heads, s.head_dim, s.batch)
    out["c4_attention"] = {"ms": round(ms, 3), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                           "frac_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "algorithmic_tflop": round(fl / 1e12, 3), "txt_valid": [300],
                           "timing": st}
    del q, k, v, o

    shape = C.C5
    b = shape.block
    Dh, F, Cl = b.hidden, b.mlp, shape.latent_channels
    valid = [int(v) for v in G.loop_inputs(shape).txt_valid]
    glue = {"t_w1": rnd(Dh, shape.freq_dim, std=0.02), "t_b1": rnd(Dh, std=0.02),
            "t_w2": rnd(Dh, Dh, std=0.02), "t_b2": rnd(Dh, std=0.02),
            "in_w": rnd(Dh, Cl, std=0.02), "in_b": rnd(Dh, std=0.02),
            "fin_w": rnd(2 * Dh, Dh, std=0.02), "fin_b": rnd(2 * Dh, std=0.02),
            "out_w": rnd(Cl, Dh, std=0.02), "out_b": rnd(Cl, std=0.02),
            "text": rnd(b.batch, b.n_txt, Dh)}
    layers = [block_w(Dh, F) for _ in range(shape.depth)]
    mod_w = [rnd(6 * Dh, Dh, std=0.02) for _ in range(shape.depth)]
    mod_b = [rnd(6 * Dh, std=0.02) for _ in range(shape.depth)]
    weights = D.model_weights(glue, layers, mod_w, mod_b)
    desc = D.model_desc(shape, valid)
    nb = D.dit_denoise_workspace_bytes(desc)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    lat = rnd(1, b.n_vis, Cl).float()
    sig = [1.0 - i / shape.steps for i in range(shape.steps + 1)]

    def loop(n):
        for i in range(n):
            D.dit_denoise_step(desc, weights, lat, sig[i], sig[i + 1], shape.guidance, ws, nb)

    loop(2)
    counter = {"i": 0}

    def one_step():
        i = counter["i"]
        D.dit_denoise_step(desc, weights, lat, sig[i], sig[i + 1], shape.guidance, ws, nb)
        counter["i"] += 1

    # one 30-step loop, an event between steps; median and percentiles over
    # the steps after the first (the pages' method: the first step is dropped)
    st = timed_stats(one_step, shape.steps, stream, drop_first=True)
    ms = st["ms"]
    assert torch.isfinite(lat).all(), "non-finite latent in the denoising loop"

    # the CFG + Euler update alone at this latent size (launch-latency bound)
    n_lat = b.n_vis * Cl
    vc, vu = rnd(n_lat), rnd(n_lat)
    xe = torch.zeros(n_lat, dtype=torch.float32, device="cuda")

    def euler():
        D.dit_euler_step(xe, vc, vu, n_lat, shape.guidance, 0.5, 0.5 - 1.0 / 30)

    euler()
    ms_e = timed(euler, 200, stream)
    out["euler_step"] = {"us": round(ms_e * 1e3, 2), "n": n_lat, "cfg": True,
                         "gbps": round(12 * n_lat / (ms_e * 1e-3) / 1e9, 1),
                         "note": "mean per call over 200 back-to-back calls (launch-latency "
                                 "bound: 12 B/element, 3.1 MB)"}
    fl = shape.depth * block_flops(b, valid)
    out["c5_loop"] = {"ms_per_step": round(ms, 3), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                      "timing": st,
                      "algorithmic_tflop_per_step": round(fl / 1e12, 3),
                      "steps": shape.steps, "depth": shape.depth, "guidance": shape.guidance,
                      "txt_valid": valid,
                      "note": "end-to-end denoiser step (timestep MLP, modulation, input projection, "
                              "24 blocks, final projection, guided Euler update); TFLOP/s counts the "
                              "blocks' algorithmic work only"}
    del layers, mod_w, mod_b, weights, ws, lat, glue
    torch.cuda.empty_cache()
    return out


def wan_block(reps, stream):
    """The Wan-style block (self-attention over the video tokens, text
    cross-attention, MLP) at the c3 video shape: 32760 video tokens, 512
    context slots of which 226 valid, hidden 5120, 40 heads x 128, MLP 13824,
    batch 1.  Seeded device draws (activations N(0,1), weights N(0, 0.02))."""
    import torch

    import diffusion_transformer_denoising_dit_amd as D
    from synthetic import configs as C
    s = C.C3
    B, S, L, Dh, F = s.batch, s.n_vis, s.n_txt, s.hidden, s.mlp
    valid = [226]
    g = torch.Generator("cuda").manual_seed(12)

    def rnd(*shape, std=1.0, mean=0.0):
        return (torch.randn(shape, generator=g, device="cuda") * std + mean).to(torch.bfloat16)

    shapes = {"w_qkv": (3 * Dh, Dh), "b_qkv": (3 * Dh,), "w_o": (Dh, Dh), "b_o": (Dh,),
              "w_cq": (Dh, Dh), "b_cq": (Dh,), "w_ckv": (2 * Dh, Dh), "b_ckv": (2 * Dh,),
              "w_co": (Dh, Dh), "b_co": (Dh,), "w_up": (F, Dh), "b_up": (F,), "w_dn": (Dh, F),
              "b_dn": (Dh,)}
    w = {k: rnd(*v, std=0.02) for k, v in shapes.items()}
    for k in ("g_q", "g_k", "g_cq", "g_ck"):
        w[k] = rnd(Dh, std=0.02, mean=1.0)
    ww = D.wan_block_weights(w)
    desc = D.block_desc(s, valid, 6 * Dh)
    mod = rnd(B, 6, Dh)
    x = torch.randn((B, S, Dh), generator=g, device="cuda")
    ctx = rnd(B, L, Dh)
    nb = D.dit_wan_block_workspace_bytes(desc)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def run():
        D.dit_wan_block_forward(desc, ww, mod, x, ctx, ws, nb)

    run()
    st = timed_stats(run, reps, stream)
    ms = st["ms"]
    M = B * S
    fl = (2.0 * M * Dh * 4 * Dh + attention_flops(S, S, s.heads, s.head_dim, B)
          + 2.0 * M * Dh * 2 * Dh + 2.0 * B * L * Dh * 2 * Dh
          + sum(attention_flops(S, v, s.heads, s.head_dim) for v in valid) + 2.0 * M * Dh * F * 2)
    return {"ms": round(ms, 3), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
            "algorithmic_tflop": round(fl / 1e12, 3), "timing": st,
            "shape": "Wan 480p: 32760 video tokens, 512 context slots (226 valid), hidden 5120, "
                     "40x128, MLP 13824, batch 1"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import diffusion_transformer_denoising_dit_amd as D
    from synthetic import configs as C
    from synthetic import gen as G

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.traffic_probe:
        traffic_probe(args.steps)
        return
    if args.hbm_probe:
        hbm_probe(args.steps)
        return
    if args.gemm_only:
        print(json.dumps({"block_gemms": block_gemms(max(3, args.steps), torch.cuda.current_stream())}),
              flush=True)
        return
    shape = C.C3_STEP
    blk = shape.block
    t_gen = time.perf_counter()
    inp = G.loop_inputs(shape)
    layer = inp.layer(0)
    print(f"[bench] inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)

    glue = {"t_w1": inp.t_w1, "t_b1": inp.t_b1, "t_w2": inp.t_w2, "t_b2": inp.t_b2,
            "in_w": inp.in_w, "in_b": inp.in_b, "fin_w": inp.fin_mod_w, "fin_b": inp.fin_mod_b,
            "out_w": inp.out_w, "out_b": inp.out_b, "text": inp.text}
    dglue = {k: dev_bf16(v) for k, v in glue.items()}
    dl = {k: dev_bf16(v) for k, v in layer.items()}
    weights = D.model_weights(dglue, [{n: dl[n] for n in BLOCK_NAMES}], [dl["mod_w"]], [dl["mod_b"]])
    desc = D.model_desc(shape, inp.txt_valid)
    ws_bytes = D.dit_denoise_workspace_bytes(desc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    lat0 = torch.from_numpy(
        (inp.latent.astype(np.uint32) << 16).view(np.float32).reshape(1, blk.n_vis, -1)).cuda()
    lat = lat0.clone()
    stream = torch.cuda.current_stream()
    sig = [1.0 - i / shape.steps for i in range(shape.steps + 1)]
    counter = {"i": 0}

    def step():
        i = counter["i"] % shape.steps
        D.dit_denoise_step(desc, weights, lat, sig[i], sig[i + 1], shape.guidance, ws, ws_bytes)
        counter["i"] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st_step = timed_stats(step, args.steps, stream)
    ms_step = st_step["ms"]
    assert torch.isfinite(lat).all(), "non-finite latent"

    # step caching at the same shape: the block-0 probe, a cached (skipped)
    # step, the change-score kernel alone on the probe's features, and a
    # 30-step cadence-2 loop (5 initial and 5 final full steps) driven by the
    # library's controller
    Bl = 1 if shape.cfg else blk.batch
    prev_v = torch.zeros((Bl, blk.n_vis, shape.latent_channels), dtype=torch.float32, device="cuda")
    delta_v = torch.zeros_like(prev_v)
    score = torch.zeros(1, dtype=torch.float32, device="cuda")
    saved = torch.zeros((blk.batch, blk.n_tok, blk.hidden), dtype=torch.bfloat16, device="cuda")
    pscore = torch.zeros(1, dtype=torch.float32, device="cuda")
    lat_c = lat0.clone()

    def cached(i, action, have_prev):
        D.dit_denoise_step_cached(desc, weights, lat_c, sig[i], sig[i + 1], shape.guidance, action,
                                  have_prev, prev_v, delta_v, score, ws, ws_bytes)

    def probe():
        D.dit_cache_probe(desc, weights, lat_c, sig[3], saved, 1, pscore, ws, ws_bytes)

    cached(0, D.STEP_FULL, 0)
    cached(1, D.STEP_FULL, 1)
    probe()
    st_probe = timed_stats(probe, max(5, args.steps), stream)
    st_skip = timed_stats(lambda: cached(2, D.STEP_SKIP, 1), max(5, args.steps), stream)
    ms_probe, ms_skip = st_probe["ms"], st_skip["ms"]
    feat_n = blk.batch * blk.n_tok * blk.hidden
    cur_f = torch.randn(feat_n, generator=torch.Generator("cuda").manual_seed(6),
                        device="cuda").to(torch.bfloat16)
    sws = torch.empty(D.dit_change_score_workspace_bytes(), dtype=torch.uint8, device="cuda")

    def change_score():
        D.dit_change_score(cur_f, saved, D.DTYPE_BF16, feat_n, 1, pscore, sws, sws.numel())

    change_score()
    st_score = timed_stats(change_score, max(5, args.steps), stream)
    ms_score = st_score["ms"]
    score_bytes = 3 * feat_n * 2  # read current and saved, write saved

    def cadence_loop():
        ctl = D.CacheController(D.cache_policy(D.CACHE_CADENCE, shape.steps, 5, 5, cadence=2))
        n_full = 0
        for i in range(shape.steps):
            a = ctl.decide(i)
            cached(i, a, 1 if n_full else 0)
            n_full += a == D.STEP_FULL
        return n_full

    lat_c.copy_(lat0)
    n_full_loop = cadence_loop()
    torch.cuda.synchronize()
    lat_c.copy_(lat0)
    ms_loop = timed(cadence_loop, 1, stream) / shape.steps
    del cur_f, saved

    # the block alone (same weights, modulation from the step's own buffers)
    bdesc = D.block_desc(blk, inp.txt_valid, 0)
    bws_bytes = D.dit_block_workspace_bytes(bdesc)
    bws = torch.empty(bws_bytes, dtype=torch.uint8, device="cuda")
    x = torch.randn((blk.batch, blk.n_tok, blk.hidden), generator=torch.Generator("cuda").manual_seed(3),
                    device="cuda")
    mod = (torch.randn((6, blk.hidden), generator=torch.Generator("cuda").manual_seed(4), device="cuda")
           * 0.1).to(torch.bfloat16)
    bw = {n: dl[n] for n in BLOCK_NAMES}

    def block():
        D.dit_block_forward(bdesc, bw, mod, x, bws, bws_bytes)

    block()
    st_block = timed_stats(block, max(50, args.steps), stream)
    ms_block = st_block["ms"]

    # joint attention alone, q/k/v as column blocks of one [N, 3*H*d] buffer (the block layout)
    HD = blk.hidden
    qkv = torch.randn((blk.batch, blk.n_tok, 3 * HD), generator=torch.Generator("cuda").manual_seed(5),
                      device="cuda").to(torch.bfloat16)
    o = torch.empty((blk.batch, blk.n_tok, HD), dtype=torch.bfloat16, device="cuda")
    adesc = D.attn_desc(blk.batch, blk.n_vis, blk.n_txt, blk.heads, blk.head_dim, inp.txt_valid)
    # with the workspace the block passes it (an under-filled last round of
    # query tiles -- 80 of 5200 on 256 CUs -- splits along the keys; the
    # timed call includes the merge of those partials)
    a_wsb = D.dit_joint_attention_workspace_bytes()
    a_ws = torch.empty(a_wsb, dtype=torch.uint8, device="cuda")

    def attn():
        D.dit_joint_attention(adesc, qkv, qkv[..., HD:], qkv[..., 2 * HD:], 3 * HD, o, HD,
                              workspace=a_ws, workspace_bytes=a_wsb)

    attn()
    st_attn = timed_stats(attn, max(50, args.steps), stream)
    ms_attn = st_attn["ms"]
    # peaked softmax rows: q scaled by 4 (exact in bf16), so the running
    # maxima move more often and the O/l rescale is skipped less often
    qkv[..., :HD].mul_(4.0)
    attn()
    st_attn_peaked = timed_stats(attn, max(50, args.steps), stream)
    qkv[..., :HD].mul_(0.25)
    attn()  # o back to the unscaled inputs' output (the split comparison reads it)
    valid = [int(v) for v in inp.txt_valid]
    a_flop = sum(attention_flops(blk.n_tok, blk.n_vis + L, blk.heads, blk.head_dim) for L in valid)
    a_dense = attention_flops(blk.n_tok, blk.n_tok, blk.heads, blk.head_dim) * blk.batch
    a_tflops = a_flop / (ms_attn * 1e-3) / 1e12
    b_flop = block_flops(blk, valid)

    # split joint attention (Difflet, section 4.3): the text keys [0, L) as one
    # partial plus the visual keys in 4 partitions, each attended by every
    # query row into fp32 (out, LSE) buffers, then merged to bf16
    cuts = [round(i * blk.n_vis / 4) for i in range(5)]
    segs = [(blk.n_vis, blk.n_tok, valid)] + [(a, b, [b - a] * blk.batch)
                                               for a, b in zip(cuts[:-1], cuts[1:])]
    p_out = [torch.empty((blk.batch, blk.n_tok, HD), dtype=torch.float32, device="cuda")
             for _ in segs]
    p_lse = [torch.empty((blk.batch, blk.heads, blk.n_tok), dtype=torch.float32, device="cuda")
             for _ in segs]
    p_desc = [D.partial_desc(blk.batch, blk.n_tok, b - a, blk.heads, blk.head_dim, kv)
              for a, b, kv in segs]
    o_split = torch.empty_like(o)

    def split_partials():
        for (a, b, _), pd, po, pl in zip(segs, p_desc, p_out, p_lse):
            D.dit_attention_partial(pd, qkv, 3 * HD, qkv[:, a:, HD:], qkv[:, a:, 2 * HD:], 3 * HD,
                                    po, HD, pl)

    def split_merge():
        D.dit_attention_merge(blk.batch, blk.n_tok, blk.heads, blk.head_dim, p_out, HD, p_lse,
                              o_split, HD)

    def split():
        split_partials()
        split_merge()

    split()
    torch.cuda.synchronize()
    split_err = (o_split.float() - o.float()).abs().max().item()
    st_split = timed_stats(split, max(3, args.steps // 2), stream)
    st_merge = timed_stats(split_merge, max(5, args.steps), stream)
    ms_split, ms_merge = st_split["ms"], st_merge["ms"]
    del p_out, p_lse, o_split

    gemms = block_gemms(max(3, args.steps // 2), stream)
    hbm = hbm_probe(2, reps=max(10, args.steps))
    mm = mmdit_blocks(max(5, args.steps), stream)
    wan = wan_block(max(3, args.steps // 2), stream)
    others = other_configs(args.steps, stream)
    traffic = attn_traffic()
    result = {
        "metric": METRIC,
        "value": round(ms_step, 3),
        "unit": "ms/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("c3 video 480p denoising step, 1 DiT block: 81 frames -> latent 21x30x52 "
                         "after (1,2,2) patchify = 32760 visual + 512 text tokens (226 valid), "
                         "hidden 5120, 40 heads x 128, MLP 13824, batch 1, 3D RoPE 44/42/42"),
            "tokens": blk.n_tok, "valid_keys": blk.n_vis + valid[0], "hidden": blk.hidden,
            "heads": blk.heads, "head_dim": blk.head_dim, "mlp": blk.mlp, "batch": blk.batch,
        },
        "block_ms": round(ms_block, 3),
        "block_tflops": round(b_flop / (ms_block * 1e-3) / 1e12, 1),
        "timing": {"step": st_step, "block": st_block},
        "attention": {
            "ms": round(ms_attn, 3),
            "tflops": round(a_tflops, 1),
            "frac_bf16_peak": round(a_tflops / PEAK_BF16_TFLOPS, 4),
            "algorithmic_tflop": round(a_flop / 1e12, 3),
            "dense_tflop": round(a_dense / 1e12, 3),
            "inputs": "q, k, v N(0,1) bf16 (nearly flat softmax rows)",
            "timing": st_attn,
            "peaked": {"inputs": "q x 4 (peaked softmax rows)", "timing": st_attn_peaked,
                       "tflops": round(a_flop / (st_attn_peaked["ms"] * 1e-3) / 1e12, 1),
                       "frac_bf16_peak": round(a_flop / (st_attn_peaked["ms"] * 1e-3) / 1e12
                                               / PEAK_BF16_TFLOPS, 4)},
        },
        "split_attention": {
            "partials": len(segs),
            "ms": round(ms_split, 3),
            "merge_ms": round(ms_merge, 3),
            "tflops": round(a_flop / (ms_split * 1e-3) / 1e12, 1),
            "max_abs_vs_unsplit": round(split_err, 5),
            "timing": st_split, "merge_timing": st_merge,
        },
        "step_cache": {
            "probe_ms": round(ms_probe, 3),
            "skip_step_ms": round(ms_skip, 4),
            "change_score_ms": round(ms_score, 4),
            "change_score_gbps": round(score_bytes / (ms_score * 1e-3) / 1e9, 1),
            "change_score_frac_hbm_peak": round(score_bytes / (ms_score * 1e-3) / 8e12, 4),
            "cadence2_loop_ms_per_step": round(ms_loop, 3),
            "cadence2_full_steps": int(n_full_loop),
            "steps": shape.steps,
            "timing": {"probe": st_probe, "skip_step": st_skip, "change_score": st_score},
        },
        "block_gemms": gemms,
        "hbm_kernels": hbm,
        "mmdit": mm,
        "wan_block": wan,
        "other_configs": others,
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_kernel<128, false> + tail_merge_kernel<128> (joint attention; the "
                      "under-filled last round of query tiles split along the keys and merged)",
            "achieved": round(a_tflops, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(a_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": (None if traffic is None
                        else round(traffic["fetch_bytes"] + traffic["write_bytes"])),
            "traffic_unit": "bytes per launch (L2-to-fabric, counter-measured)",
            "traffic_detail": None if traffic is None else {
                "fetch_bytes": traffic["fetch_bytes"], "write_bytes": traffic["write_bytes"],
                "algorithmic_bytes": 4 * blk.batch * blk.n_tok * HD * 2,
                "fetch_scale": traffic["fetch_scale"], "write_scale": traffic["write_scale"],
                "profile": traffic["profile"]},
        },
    }
    if not args.no_cpu_baseline:
        # the oracle reads the same seeded model (its layer cached: drawn once)
        view = G.loop_inputs(shape)
        view.layer = lambda l, _w=layer: _w
        del dl, dglue, weights, ws, bws, qkv
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(shape, {"latent": inp.latent, "oracle_view": view},
                                              args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
