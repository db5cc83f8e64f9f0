"""GPU parity of each kernel, called through the C ABI, against the fp64
oracle on the same seeded inputs (small shapes spanning several tiles and a
ragged tail)."""

import math

import numpy as np
import pytest
import torch

import diffusion_transformer_denoising_dit_amd as D
import oracle as O
from synthetic import configs as C
from synthetic import gen as G
from tests.sampling import sample_rows
from tests.gpu_util import (assert_bf16_ulp, assert_parity, bits_of, dev_bf16,
                            dev_f32_from_bf16, host)

pytestmark = pytest.mark.gpu


def _dec(bits):
    return O.bf16_decode(bits)


# ------------------------------------------------------------------ GEMM

def _gemm_case(seed, M, N, K):
    a = G.normal_bf16(seed, (M, K))
    w = G.normal_bf16(seed + 1, (N, K), 0.05)
    b = G.normal_bf16(seed + 2, (N,), 0.5)
    return a, w, b


@pytest.mark.parametrize("M,N,K", [(300, 200, 192), (33, 64, 64), (513, 392, 256)])
@pytest.mark.parametrize("epi", ["bf16", "gelu", "silu", "f32"])
def test_linear_epilogues(M, N, K, epi):
    a, w, b = _gemm_case(100 + M, M, N, K)
    y = O.linear(_dec(a), _dec(w), _dec(b))
    code = {"bf16": D.EPI_BF16, "gelu": D.EPI_GELU_BF16, "silu": D.EPI_SILU_BF16,
            "f32": D.EPI_F32}[epi]
    da, dw, db = dev_bf16(a), dev_bf16(w), dev_bf16(b)
    out = torch.empty((M, N), dtype=torch.float32 if epi == "f32" else torch.bfloat16,
                      device="cuda")
    D.dit_linear(da, K, dw, db, M, N, K, code, out, N)
    torch.cuda.synchronize()
    got = host(out)
    if epi == "f32":
        assert_parity(got, y, f"linear f32 {M}x{N}x{K}", max_abs=1e-4 * np.abs(y).max(),
                      rel_l2=1e-5)
    else:
        ref = {"bf16": y, "gelu": O.gelu_erf(y), "silu": O.silu(y)}[epi]
        assert_bf16_ulp(got, ref, f"linear {epi} {M}x{N}x{K}")


def _linear_every_epilogue(M, N, K, epi, seed, what):
    """One linear layer through dit_linear twice (bitwise-equal reruns) against the oracle."""
    a, w, b = _gemm_case(seed, M, N, K)
    y = O.linear(_dec(a), _dec(w), _dec(b))
    da, dw, db = dev_bf16(a), dev_bf16(w), dev_bf16(b)
    if epi == "res":
        x0 = G.normal_bf16(13, (M, N))
        want = _dec(x0) + y
        outs = []
        for _ in range(2):
            x = dev_f32_from_bf16(x0)
            D.dit_linear(da, K, dw, db, M, N, K, D.EPI_RES_F32, x, N)
            outs.append(x)
        torch.cuda.synchronize()
        assert_parity(host(outs[0]), want, f"{what} residual {M}x{N}x{K}",
                      max_abs=1e-4 * np.abs(want).max(), rel_l2=1e-5)
    elif epi == "gated":
        rows_g = M // 2 + 1
        gate = G.normal_bf16(11, (2, N))
        x0 = G.normal_bf16(12, (M, N))
        want = _dec(x0) + _dec(gate)[np.arange(M) // rows_g] * y
        outs = []
        for _ in range(2):
            x = dev_f32_from_bf16(x0)
            D.dit_linear(da, K, dw, db, M, N, K, D.EPI_GATED_RES_F32, x, N, gate=dev_bf16(gate),
                         gate_stride=N, gate_rows=rows_g)
            outs.append(x)
        torch.cuda.synchronize()
        assert_parity(host(outs[0]), want, f"{what} gated {M}x{N}x{K}",
                      max_abs=1e-4 * np.abs(want).max(), rel_l2=1e-5)
    else:
        code = {"bf16": D.EPI_BF16, "gelu": D.EPI_GELU_BF16, "f32": D.EPI_F32}[epi]
        outs = []
        for _ in range(2):
            out = torch.empty((M, N), dtype=torch.float32 if epi == "f32" else torch.bfloat16,
                              device="cuda")
            D.dit_linear(da, K, dw, db, M, N, K, code, out, N)
            outs.append(out)
        torch.cuda.synchronize()
        got = host(outs[0])
        if epi == "f32":
            assert_parity(got, y, f"{what} f32 {M}x{N}x{K}", max_abs=1e-4 * np.abs(y).max(),
                          rel_l2=1e-5)
        else:
            ref = {"bf16": y, "gelu": O.gelu_erf(y)}[epi]
            assert_bf16_ulp(got, ref, f"{what} {epi} {M}x{N}x{K}")
    assert torch.equal(outs[0], outs[1]), f"{what} GEMM rerun differs"


# Shapes with M >= 1024, N >= 256 and K >= 256 run the large-tile kernel
# (256 x 256 workgroup tiles, 64-wide K slices streamed through a 3-stage W
# ring and 2-stage A rings): ragged M and N, 4 to 8 K slices (every residue of
# the slice count modulo both ring depths), every epilogue, bitwise-equal
# reruns.  (K = 64 with N >= 256 and M >= 1024 goes to the short-K stream
# kernel instead: the (1031, 264, 64) shape checks that routing.)
@pytest.mark.parametrize("M,N,K", [(1100, 520, 256), (1031, 264, 384), (2304, 512, 320),
                                   (1100, 520, 448), (2304, 512, 512), (1031, 264, 64)])
@pytest.mark.parametrize("epi", ["bf16", "gelu", "f32", "gated", "res"])
def test_linear_large_tiles(M, N, K, epi):
    _linear_every_epilogue(M, N, K, epi, 200 + M + K, "large")


# Few features over a long K (N <= 64, K >= 1024 and a multiple of 256,
# M >= 256: the projection to the latent channels) runs the long-K stream
# kernel: K split over the 4 waves of a workgroup (odd and even chunk counts
# per wave), on 256 compute units 32-row workgroups up to 16383 rows, 64-row
# ones up to 32640 (20000 and 17000 rows), 128-row ones above (33000), N not
# a multiple of 16.
@pytest.mark.parametrize("M,N,K", [(300, 64, 1024), (1000, 56, 2048), (20000, 64, 1280),
                                   (17000, 16, 1024), (33000, 40, 1280)])
@pytest.mark.parametrize("epi", ["bf16", "gelu", "f32", "gated", "res"])
def test_linear_long_k_few_features(M, N, K, epi):
    _linear_every_epilogue(M, N, K, epi, 300 + M + N, "long-K stream")


# A short K onto many features (K of 64 or 128, N >= 256, M >= 1024: the
# projection from the latent channels) runs the short-K stream kernel: W rows
# held in registers, 32-row token blocks walked with a stride, ragged M and N
# (a partly and a wholly out-of-range wave of 64 features).
@pytest.mark.parametrize("M,N,K", [(1100, 520, 64), (3001, 256, 128), (2051, 1288, 64)])
@pytest.mark.parametrize("epi", ["bf16", "gelu", "f32", "gated", "res"])
def test_linear_short_k_many_features(M, N, K, epi):
    _linear_every_epilogue(M, N, K, epi, 400 + M + N, "short-K stream")


def test_linear_stream_kernels_grouped_rows():
    """The two projections of a denoising step in their real addressing: the
    input projection reads one shared block of latent rows for two batch rows
    (a_group_stride 0) and writes the visual rows of each batch row, leaving
    the text rows between them untouched; the output projection reads the
    visual rows of each batch row out of [batch, n_vis + n_txt, D] and writes
    them contiguously."""
    nv, nt, C, Dh = 1500, 37, 64, 512
    lat, w_in, b_in = _gemm_case(51, nv, Dh, C)
    y_in = O.linear(_dec(lat), _dec(w_in), _dec(b_in))
    x = torch.full((2, nv + nt, Dh), float("nan"), dtype=torch.float32, device="cuda")
    D.dit_linear(dev_bf16(lat), C, dev_bf16(w_in), dev_bf16(b_in), 2 * nv, Dh, C, D.EPI_F32, x, Dh,
                 group_rows=nv, a_group_stride=0, c_group_stride=(nv + nt) * Dh)
    torch.cuda.synchronize()
    got = host(x)
    assert np.isnan(got[:, nv:]).all(), "text rows were written by the input projection"
    for bi in range(2):
        assert_parity(got[bi, :nv], y_in, f"input projection rows of batch row {bi}",
                      max_abs=1e-4 * np.abs(y_in).max(), rel_l2=1e-5)

    Dk = 1024
    h = G.normal_bf16(52, (2, nv + nt, Dk))
    w_out = G.normal_bf16(53, (C, Dk), 0.05)
    b_out = G.normal_bf16(54, (C,), 0.5)
    want = np.stack([O.linear(_dec(h[bi, :nv]), _dec(w_out), _dec(b_out)) for bi in range(2)])
    v = torch.empty((2, nv, C), dtype=torch.bfloat16, device="cuda")
    D.dit_linear(dev_bf16(h), Dk, dev_bf16(w_out), dev_bf16(b_out), 2 * nv, C, Dk, D.EPI_BF16, v, C,
                 group_rows=nv, a_group_stride=(nv + nt) * Dk, c_group_stride=nv * C)
    torch.cuda.synchronize()
    assert_bf16_ulp(host(v), want, "output projection of the visual rows")


# With the optional workspace, the tiles of a last round that would fill fewer
# than half of the compute units are split along K (up to 8 parts of >= 2
# slices) and their fp32 partials summed in K order by a second kernel.  The
# shape is chosen from the device's CU count so that 6-10 tiles spill into a
# last round (266 tiles of 256 x 256 on 256 CUs; ragged M and N); K = 1024
# splits each tail tile 8 ways, K = 320 (5 slices) into uneven parts of 2 and
# 3.  Every epilogue against the oracle, bitwise-equal reruns, and the split
# result compared with the unsplit one (same values up to fp32 summation
# order; the f32 output must differ somewhere, i.e. the split path ran).
@pytest.mark.parametrize("K", [1024, 320])
@pytest.mark.parametrize("epi", ["bf16", "gelu", "f32", "gated", "res"])
def test_linear_k_split_tail(K, epi):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles_n = 14
    tiles_m = (cus + 6 + tiles_n - 1) // tiles_n
    f = tiles_m * tiles_n % cus
    assert 0 < 2 * f <= cus, (cus, tiles_m, f)
    M, N = tiles_m * 256 - 40, tiles_n * 256 - 8
    a, w, b = _gemm_case(500 + K, M, N, K)
    y = O.linear(_dec(a), _dec(w), _dec(b))
    da, dw, db = dev_bf16(a), dev_bf16(w), dev_bf16(b)
    wsb = D.dit_linear_workspace_bytes()
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    code = {"bf16": D.EPI_BF16, "gelu": D.EPI_GELU_BF16, "f32": D.EPI_F32, "gated": D.EPI_GATED_RES_F32,
            "res": D.EPI_RES_F32}[epi]
    rows_g = M // 2 + 1
    gate = G.normal_bf16(21, (2, N))
    x0 = G.normal_bf16(22, (M, N))
    if epi == "gated":
        want = _dec(x0) + _dec(gate)[np.arange(M) // rows_g] * y
    elif epi == "res":
        want = _dec(x0) + y
    else:
        want = {"bf16": y, "gelu": O.gelu_erf(y), "f32": y}[epi]

    def run(workspace):
        if epi in ("gated", "res", "f32"):
            out = dev_f32_from_bf16(x0) if epi != "f32" else torch.empty((M, N), device="cuda")
        else:
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        kw = dict(gate=dev_bf16(gate), gate_stride=N, gate_rows=rows_g) if epi == "gated" else {}
        D.dit_linear(da, K, dw, db, M, N, K, code, out, N, workspace=workspace,
                     workspace_bytes=wsb if workspace is not None else 0, **kw)
        return out

    split1, split2, whole = run(ws), run(ws), run(None)
    torch.cuda.synchronize()
    got = host(split1)
    if epi in ("bf16", "gelu"):
        assert_bf16_ulp(got, want, f"k-split {epi} {M}x{N}x{K}")
    else:
        assert_parity(got, want, f"k-split {epi} {M}x{N}x{K}", max_abs=1e-4 * np.abs(want).max(),
                      rel_l2=1e-5)
    assert torch.equal(split1, split2), "k-split rerun differs"
    d = (split1.float() - whole.float()).abs().max().item()
    assert d <= 1e-4 * float(np.abs(want).max()) + (2 ** -7 * float(np.abs(want).max()) if epi in ("bf16", "gelu") else 0)
    if epi == "f32":
        assert not torch.equal(split1, whole), "the split path did not run"


# M <= 8 token rows (the conditioning MLP and modulation projections) run the
# matrix-vector kernel: every epilogue, row counts 1..8, K below and above one
# 512-wide wave step, grouped rows, bitwise-equal reruns.
@pytest.mark.parametrize("M,N,K", [(1, 8, 64), (2, 264, 320), (3, 96, 1088), (8, 520, 5120),
                                   (1, 5120, 5120)])
@pytest.mark.parametrize("epi", ["bf16", "gelu", "silu", "f32", "gated", "res"])
def test_linear_matrix_vector(M, N, K, epi):
    a, w, b = _gemm_case(300 + M + K, M, N, K)
    y = O.linear(_dec(a), _dec(w), _dec(b))
    da, dw, db = dev_bf16(a), dev_bf16(w), dev_bf16(b)
    outs = []
    if epi in ("gated", "res"):
        x0 = G.normal_bf16(31, (M, N))
        gate = G.normal_bf16(32, (1, N))
        want = _dec(x0) + (_dec(gate) * y if epi == "gated" else y)
        for _ in range(2):
            x = dev_f32_from_bf16(x0)
            if epi == "gated":
                D.dit_linear(da, K, dw, db, M, N, K, D.EPI_GATED_RES_F32, x, N, gate=dev_bf16(gate),
                             gate_stride=N, gate_rows=M)
            else:
                D.dit_linear(da, K, dw, db, M, N, K, D.EPI_RES_F32, x, N)
            outs.append(x)
        torch.cuda.synchronize()
        assert_parity(host(outs[0]), want, f"gemv {epi} {M}x{N}x{K}",
                      max_abs=1e-4 * np.abs(want).max(), rel_l2=1e-5)
    else:
        code = {"bf16": D.EPI_BF16, "gelu": D.EPI_GELU_BF16, "silu": D.EPI_SILU_BF16,
                "f32": D.EPI_F32}[epi]
        for _ in range(2):
            out = torch.empty((M, N), dtype=torch.float32 if epi == "f32" else torch.bfloat16,
                              device="cuda")
            D.dit_linear(da, K, dw, db, M, N, K, code, out, N)
            outs.append(out)
        torch.cuda.synchronize()
        got = host(outs[0])
        if epi == "f32":
            assert_parity(got, y, f"gemv f32 {M}x{N}x{K}", max_abs=1e-4 * np.abs(y).max(),
                          rel_l2=1e-5)
        else:
            ref = {"bf16": y, "gelu": O.gelu_erf(y), "silu": O.silu(y)}[epi]
            assert_bf16_ulp(got, ref, f"gemv {epi} {M}x{N}x{K}")
    assert torch.equal(outs[0], outs[1]), "matrix-vector rerun differs"


def test_linear_matrix_vector_row_groups():
    """Two token rows in two row groups of a larger buffer (one row each, with gaps)."""
    M, N, K = 2, 264, 320
    a, w, b = _gemm_case(41, M, N, K)
    y = O.linear(_dec(a), _dec(w), _dec(b))
    a_pad = np.zeros((2, 3, K), np.uint16)
    a_pad[:, 1] = a
    out = torch.full((2, 2, N), float("nan"), dtype=torch.float32, device="cuda")
    da_pad = dev_bf16(a_pad)
    D.dit_linear(da_pad[:, 1], K, dev_bf16(w), dev_bf16(b), M, N, K, D.EPI_F32, out, N,
                 group_rows=1, a_group_stride=3 * K, c_group_stride=2 * N)
    torch.cuda.synchronize()
    got = host(out)
    assert np.isnan(got[:, 1]).all(), "rows outside the groups were written"
    assert_parity(got[:, 0], y, "gemv grouped rows", max_abs=1e-4 * np.abs(y).max(), rel_l2=1e-5)


def test_linear_gated_residual_and_row_groups():
    M, N, K, rows_g = 300, 128, 128, 150
    a, w, b = _gemm_case(7, M, N, K)
    gate = G.normal_bf16(9, (2, N))
    x0 = G.normal_bf16(10, (M, N))
    y = O.linear(_dec(a), _dec(w), _dec(b))
    want = _dec(x0) + _dec(gate)[np.arange(M) // rows_g] * y
    x = dev_f32_from_bf16(x0)
    D.dit_linear(dev_bf16(a), K, dev_bf16(w), dev_bf16(b), M, N, K, D.EPI_GATED_RES_F32, x, N,
                 gate=dev_bf16(gate), gate_stride=N, gate_rows=rows_g)
    torch.cuda.synchronize()
    assert_parity(host(x), want, "gated residual", max_abs=1e-4 * np.abs(want).max(), rel_l2=1e-5)

    # grouped addressing: A rows and C rows in two groups with gaps between them
    G_rows = 100
    a_pad = np.zeros((2, G_rows + 3, K), np.uint16)
    a_pad[:, :G_rows] = a[:2 * G_rows].reshape(2, G_rows, K)
    out = torch.full((2, G_rows + 5, N), float("nan"), dtype=torch.float32, device="cuda")
    D.dit_linear(dev_bf16(a_pad), K, dev_bf16(w), dev_bf16(b), 2 * G_rows, N, K, D.EPI_F32, out, N,
                 group_rows=G_rows, a_group_stride=(G_rows + 3) * K, c_group_stride=(G_rows + 5) * N)
    torch.cuda.synchronize()
    got = host(out)
    assert np.isnan(got[:, G_rows:]).all(), "rows outside the groups were written"
    assert_parity(got[:, :G_rows].reshape(2 * G_rows, N), y[:2 * G_rows], "grouped rows",
                  max_abs=1e-4 * np.abs(y).max(), rel_l2=1e-5)

    # the same grouped addressing through the large-tile kernel (M >= 1024, N >= 256, K >= 256)
    M2, N2, G2, K2 = 1200, 256, 600, 256
    a2, w2, b2 = _gemm_case(17, M2, N2, K2)
    y2 = O.linear(_dec(a2), _dec(w2), _dec(b2))
    a2_pad = np.zeros((2, G2 + 3, K2), np.uint16)
    a2_pad[:, :G2] = a2.reshape(2, G2, K2)
    out2 = torch.full((2, G2 + 5, N2), float("nan"), dtype=torch.float32, device="cuda")
    D.dit_linear(dev_bf16(a2_pad), K2, dev_bf16(w2), dev_bf16(b2), M2, N2, K2, D.EPI_F32, out2, N2,
                 group_rows=G2, a_group_stride=(G2 + 3) * K2, c_group_stride=(G2 + 5) * N2)
    torch.cuda.synchronize()
    got2 = host(out2)
    assert np.isnan(got2[:, G2:]).all(), "rows outside the groups were written (large tiles)"
    assert_parity(got2[:, :G2].reshape(M2, N2), y2, "grouped rows (large tiles)",
                  max_abs=1e-4 * np.abs(y2).max(), rel_l2=1e-5)


def test_linear_operand_past_4gib():
    """An A operand whose rows span more than 4 GiB (two row groups 4 GiB + 128 bytes apart):
    the large-tile kernel addresses operands by 32-bit byte offsets, so the launcher must hand
    this shape (M >= 1024, N >= 256) to the kernel with 64-bit addressing; the result must
    still match the oracle."""
    M, N, K, G_rows = 1200, 256, 256, 600       # a large-tile shape but for the 4 GiB span
    stride = (1 << 31) + 64                       # elements between the two groups' first rows
    a, w, b = _gemm_case(23, M, N, K)
    y = O.linear(_dec(a), _dec(w), _dec(b))
    big = torch.empty(stride + G_rows * K, dtype=torch.bfloat16, device="cuda")
    big[:G_rows * K].copy_(dev_bf16(a[:G_rows]).reshape(-1))
    big[stride:].copy_(dev_bf16(a[G_rows:]).reshape(-1))
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    D.dit_linear(big, K, dev_bf16(w), dev_bf16(b), M, N, K, D.EPI_F32, out, N,
                 group_rows=G_rows, a_group_stride=stride, c_group_stride=G_rows * N)
    torch.cuda.synchronize()
    del big
    torch.cuda.empty_cache()
    assert_parity(host(out), y, "A operand past 4 GiB", max_abs=1e-4 * np.abs(y).max(), rel_l2=1e-5)


def test_linear_rejects_bad_k_without_launch():
    a = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 96), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(D.DitError) as e:
        D.dit_linear(a, 96, w, None, 4, 8, 96, D.EPI_BF16, out, 8)
    assert e.value.status_name == "DIT_EUNSUPPORTED"


# ------------------------------------------------------------------ adaLN

@pytest.mark.parametrize("rows,hidden,rpb,shared", [(300, 256, 150, False), (77, 3072, 40, True),
                                                     (5, 5120, 5, False)])
def test_adaln(rows, hidden, rpb, shared):
    x = G.normal_bf16(20, (rows, hidden), 2.0, 0.3)
    nb = (rows + rpb - 1) // rpb
    mod = G.normal_bf16(21, (nb, 2, hidden))
    stride = 0 if shared else 2 * hidden
    xf = _dec(x)
    bidx = np.zeros(rows, int) if shared else np.arange(rows) // rpb
    shift = _dec(mod)[bidx, 0]
    scale = _dec(mod)[bidx, 1]
    want = O.adaln_modulate(xf, shift, scale, 1e-6)
    dmod = dev_bf16(mod)
    out = torch.empty((rows, hidden), dtype=torch.bfloat16, device="cuda")
    # shift of batch row b at mod[b, 0], scale at mod[b, 1]: one row stride 2*hidden
    D.dit_adaln_modulate(dev_f32_from_bf16(x), rows, hidden, rpb, dmod, dmod.view(-1)[hidden:],
                         stride, 1e-6, out)
    torch.cuda.synchronize()
    assert_bf16_ulp(host(out), want, f"adaln {rows}x{hidden}")


# ------------------------------------------------------------------ RMSNorm + RoPE

ROPE_SHAPES = [
    C.BlockShape("rope_small", batch=2, grid=(2, 3, 5), n_txt=9, heads=2, head_dim=64, mlp=64,
                 rope=(20, 22, 22), seed=31),
    C.BlockShape("rope_128", batch=1, grid=(3, 4, 6), n_txt=7, heads=3, head_dim=128, mlp=64,
                 rope=(44, 42, 42), seed=32),
]


@pytest.mark.parametrize("shape", ROPE_SHAPES, ids=lambda s: s.name)
def test_qk_rmsnorm_rope(shape):
    B, N, Dh, H, d = shape.batch, shape.n_tok, shape.hidden, shape.heads, shape.head_dim
    qkv = G.normal_bf16(shape.seed, (B, N, 3 * Dh), 1.5)
    gq = G.normal_bf16(shape.seed + 1, (Dh,), 0.02, 1.0)
    gk = G.normal_bf16(shape.seed + 2, (Dh,), 0.02, 1.0)
    pos = O.token_positions(shape.grid, shape.n_txt)
    f = _dec(qkv)
    want_q = O.rope_axial(O.rms_norm_full(f[..., :Dh], _dec(gq), 1e-6).reshape(B, N, H, d), pos,
                          shape.rope, 1e4).reshape(B, N, Dh)
    want_k = O.rope_axial(O.rms_norm_full(f[..., Dh:2 * Dh], _dec(gk), 1e-6).reshape(B, N, H, d),
                          pos, shape.rope, 1e4).reshape(B, N, Dh)
    t = dev_bf16(qkv)
    desc = D.block_desc(shape, [0] * B)
    D.dit_qk_rmsnorm_rope(desc, t, 3 * Dh, dev_bf16(gq), dev_bf16(gk))
    torch.cuda.synchronize()
    got = host(t)
    assert_bf16_ulp(got[..., :Dh], want_q, f"{shape.name} q")
    assert_bf16_ulp(got[..., Dh:2 * Dh], want_k, f"{shape.name} k")
    np.testing.assert_array_equal(bits_of(t)[..., 2 * Dh:], qkv[..., 2 * Dh:])  # v untouched


def test_positions_exact():
    s = C.C3
    desc = D.block_desc(s, [0])
    out = torch.empty((s.n_tok, 3), dtype=torch.int32, device="cuda")
    D.dit_debug_positions(desc, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), O.token_positions(s.grid, s.n_txt))


# ------------------------------------------------------------------ attention

ATTN_SHAPES = [
    C.AttnShape("attn_d64", batch=2, n_vis=300, n_txt=40, heads=3, head_dim=64,
                txt_valid=("fixed", (7, 40)), seed=41),
    C.AttnShape("attn_d128", batch=2, n_vis=257, n_txt=77, heads=2, head_dim=128,
                txt_valid=("fixed", (0, 13)), seed=42),
    C.AttnShape("attn_tiny", batch=1, n_vis=5, n_txt=3, heads=1, head_dim=128,
                txt_valid=("fixed", (2,)), seed=43),
    # eight batch rows, each with its own valid text length (none, all, and between):
    # exercises the workgroup -> (batch row, head, query tile) decode past batch 2
    C.AttnShape("attn_b8", batch=8, n_vis=300, n_txt=20, heads=3, head_dim=64,
                txt_valid=("fixed", (0, 1, 5, 19, 20, 7, 13, 2)), seed=44),
    # one launch whose batch rows hold 120, 128, 129, 192, 193, 256, 257 and
    # 320 valid keys: 2 to 5 key tiles of 64, the last one full or ragged --
    # every path of the K/V ring (tiles from the prologue only, the first
    # tile issued inside the loop, the last tile with and without a newer
    # load in flight)
    C.AttnShape("attn_tiles_d128", batch=8, n_vis=120, n_txt=200, heads=2, head_dim=128,
                txt_valid=("fixed", (0, 8, 9, 72, 73, 136, 137, 200)), seed=45),
    C.AttnShape("attn_tiles_d64", batch=8, n_vis=120, n_txt=200, heads=2, head_dim=64,
                txt_valid=("fixed", (0, 8, 9, 72, 73, 136, 137, 200)), seed=46),
]


def _run_attention(shape, inp, lse=True, scale=0.0):
    B, N, HD = shape.batch, shape.n_tok, shape.hidden
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    out = torch.empty((B, N, HD), dtype=torch.bfloat16, device="cuda")
    l = torch.empty((B, shape.heads, N), dtype=torch.float32, device="cuda") if lse else None
    desc = D.attn_desc(B, shape.n_vis, shape.n_txt, shape.heads, shape.head_dim, inp["txt_valid"])
    D.dit_joint_attention(desc, q, k, v, HD, out, HD, l, scale)
    torch.cuda.synchronize()
    return out, l


def _oracle_attention(shape, inp, q_bits=None):
    B, N, H, d = shape.batch, shape.n_tok, shape.heads, shape.head_dim
    q = _dec(inp["q"] if q_bits is None else q_bits).reshape(B, -1, H, d)
    k = _dec(inp["k"]).reshape(B, N, H, d)
    v = _dec(inp["v"]).reshape(B, N, H, d)
    return O.joint_attention(q, k, v, shape.n_vis, inp["txt_valid"])


@pytest.mark.parametrize("shape", ATTN_SHAPES, ids=lambda s: s.name)
@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_attention_parity(shape, q_scale):
    inp = G.attention_inputs(shape, q_scale)
    out, lse = _run_attention(shape, inp)
    o, l = _oracle_attention(shape, inp)
    assert_parity(host(out), o.reshape(host(out).shape), f"{shape.name} q*{q_scale} out")
    assert_parity(host(lse), l, f"{shape.name} lse", max_abs=1e-3, rel_l2=1e-5)


def test_attention_reference_lag():
    """Designed scores that drive the softmax reference through both of its
    paths.  q is nonzero in one dimension only, so query i's log2-domain score
    of key j is f_i * b_j: keys 0..383 are flat (b in [-1, 0]), key 340 (tile
    5) rises 1.5 above them, key 390 (the last, partly valid tile) rises to 4.
    With f = 0.5 and 1 a query has summed its weights past 32 (per half row)
    after two tiles, so at key 340 its reference lags instead of rescaling,
    and at key 390 (a rise of 2 and 4) it rescales; f = 4 rescales at both;
    f = 0 keeps every weight at 1.  Every output element must lie within one
    bf16 unit of the exact value (its own rounding to bf16 is half of that)
    plus 5e-4 (absolute) for the bf16 rounding of the weights
    (the lag adds at most 2^-12 of max |v| per lagged key).  Measured on
    MI355X: the worst element, 7.5e-3 at |o| = 2.9, in the f = 4 rows (the
    output's own rounding; 0.84 of the bound), the lagged rows within 4.6e-4."""
    s = C.AttnShape("lag", batch=1, n_vis=384, n_txt=16, heads=1, head_dim=128,
                    txt_valid=("fixed", (16,)), seed=91)
    N, d = s.n_tok, s.head_dim
    rng = np.random.default_rng(91)
    c = math.log2(math.e) / math.sqrt(d)
    b = rng.uniform(-1.0, 0.0, N)
    b[340], b[390] = 1.5, 4.0
    f = np.array([0.0, 0.5, 1.0, 4.0])[np.arange(N) % 4]
    q = np.zeros((1, N, d), np.float32)
    q[0, :, 0] = f / c
    k = rng.normal(0.0, 0.3, (1, N, d)).astype(np.float32)
    k[0, :, 0] = b
    inp = {"q": G.f32_to_bf16_bits(q), "k": G.f32_to_bf16_bits(k),
           "v": G.normal_bf16(92, (1, N, d)), "txt_valid": np.array([16])}
    out, lse = _run_attention(s, inp)
    o, l = _oracle_attention(s, inp)
    got = host(out)
    want = o.reshape(got.shape)
    atol = 5e-4 / float(np.abs(want).max())  # 5e-4 absolute, as a fraction of max |output|
    assert_bf16_ulp(got, want, "reference lag", atol_rel=atol)
    assert_parity(host(lse), l, "reference lag lse", max_abs=1e-3, rel_l2=1e-5)
    for fi in (0.0, 0.5, 1.0, 4.0):  # each regime on its own rows
        rows = np.nonzero(f == fi)[0]
        ma = float(np.abs(want[:, rows]).max())
        assert_bf16_ulp(got[:, rows], want[:, rows], f"reference lag, f = {fi:g}",
                        atol_rel=5e-4 / max(ma, 1e-30))


# With a workspace, the f query tiles of an under-filled last round (after
# at least one full round; one 512-thread workgroup per CU) are split along
# the keys into the p ranges (2..4) whose f * p workgroups finish soonest,
# ceil(f p / CUs) / p of a round, and a second kernel merges the partials.
# Shapes whose tile count leaves such a round on 256 CUs: 264 tiles (8 split
# 4 ways; head_dim 128 and 64), 336 tiles of two batch rows with different
# valid lengths (80 split 3 ways: the last range holds the ragged bound) and
# 400 tiles (144, more than half the CUs, split 3 ways).  Checked: against
# the oracle on sampled rows that include the split tiles' rows, output and
# log-denominator at the strict bar; bitwise equal to the call without
# workspace outside the split tiles, not equal inside them (the split path
# ran); bitwise-equal reruns.
SPLIT_SHAPES = [
    C.AttnShape("split4_d128", batch=1, n_vis=8384, n_txt=64, heads=8, head_dim=128,
                txt_valid=("fixed", (40,)), seed=47),
    C.AttnShape("split3_b2", batch=2, n_vis=10600, n_txt=100, heads=4, head_dim=128,
                txt_valid=("fixed", (37, 100)), seed=48),
    C.AttnShape("split4_d64", batch=1, n_vis=8400, n_txt=48, heads=8, head_dim=64,
                txt_valid=("fixed", (48,)), seed=49),
    C.AttnShape("split3_f144", batch=1, n_vis=12600, n_txt=100, heads=8, head_dim=128,
                txt_valid=("fixed", (64,)), seed=50),
]


def _split_tiles(shape, cu):
    """(b, h, query tile) of the tiles the launcher splits, [] if none."""
    n_qt = -(-shape.n_tok // 256)
    total = n_qt * shape.heads * shape.batch
    f = total % cu
    if total < cu or f == 0:
        return []
    best = min((-(-f * p // cu) / p, p) for p in (1, 2, 3, 4) if f * p <= 448)
    if best[1] == 1 or best[0] >= 1.0:
        return []
    return [(nid // (n_qt * shape.heads), (nid // n_qt) % shape.heads, nid % n_qt)
            for nid in range(total - f, total)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: s.name)
def test_attention_split_last_round(shape):
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = _split_tiles(shape, cu)
    if not tiles:
        pytest.skip(f"{cu} compute units leave no under-filled last round at this shape")
    inp = G.attention_inputs(shape, 2.0)
    B, N, H, d, HD = shape.batch, shape.n_tok, shape.heads, shape.head_dim, shape.hidden
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    desc = D.attn_desc(B, shape.n_vis, shape.n_txt, H, d, inp["txt_valid"])
    wsb = D.dit_joint_attention_workspace_bytes()
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    outs = []
    for use_ws in (False, True, True):
        out = torch.empty((B, N, HD), dtype=torch.bfloat16, device="cuda")
        l = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        D.dit_joint_attention(desc, q, k, v, HD, out, HD, l, workspace=ws if use_ws else None,
                              workspace_bytes=wsb if use_ws else 0)
        outs.append((out, l))
    torch.cuda.synchronize()
    (o0, l0), (o1, l1), (o2, l2) = outs
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "split attention rerun differs"
    in_split = np.zeros((B, N, H), bool)
    for b, h, qt in tiles:
        in_split[b, qt * 256:(qt + 1) * 256, h] = True
    g0 = bits_of(o0).reshape(B, N, H, d)
    g1 = bits_of(o1).reshape(B, N, H, d)
    np.testing.assert_array_equal(g0[~in_split], g1[~in_split])
    assert (g0[in_split] != g1[in_split]).any(), "the split path did not run"
    lse0, lse1 = l0.cpu().numpy().transpose(0, 2, 1), l1.cpu().numpy().transpose(0, 2, 1)
    np.testing.assert_array_equal(lse0[~in_split], lse1[~in_split])
    # oracle rows: the sampled set plus 40 rows of every split tile's query range
    rows = set(sample_rows(shape.n_vis, shape.n_txt, inp["txt_valid"], n_random=32, seed=shape.seed).tolist())
    rng = np.random.default_rng(shape.seed)
    for qt in sorted({t[2] for t in tiles}):
        lo, hi = qt * 256, min(N, (qt + 1) * 256)
        rows.update(int(r) for r in rng.integers(lo, hi, 40))
    rows = np.array(sorted(rows), np.int64)
    qo = _dec(inp["q"][:, rows]).reshape(B, len(rows), H, d)
    ko = _dec(inp["k"]).reshape(B, N, H, d)
    vo = _dec(inp["v"]).reshape(B, N, H, d)
    o, lo_ = O.joint_attention(qo, ko, vo, shape.n_vis, inp["txt_valid"])
    print(f"{shape.name}: {len(tiles)} split tiles, {int(in_split[:, rows].sum())} sampled "
          f"(row, head) pairs inside them", flush=True)
    assert_parity(host(o1)[:, rows], o.reshape(B, len(rows), HD), f"{shape.name} split out")
    assert_parity(host(l1)[:, :, rows], lo_, f"{shape.name} split lse", max_abs=1e-3, rel_l2=1e-5)


def test_attention_padding_is_ignored_bitwise():
    shape = ATTN_SHAPES[0]
    inp = G.attention_inputs(shape)
    out1, lse1 = _run_attention(shape, inp)
    inp2 = dict(inp)
    k2, v2 = inp["k"].copy(), inp["v"].copy()
    rng = np.random.default_rng(5)
    for b in range(shape.batch):
        lo = shape.n_vis + int(inp["txt_valid"][b])
        k2[b, lo:] = rng.integers(0, 65536, k2[b, lo:].shape, dtype=np.uint16)  # NaN/Inf included
        v2[b, lo:] = rng.integers(0, 65536, v2[b, lo:].shape, dtype=np.uint16)
    inp2["k"], inp2["v"] = k2, v2
    out2, lse2 = _run_attention(shape, inp2)
    np.testing.assert_array_equal(bits_of(out1), bits_of(out2))
    np.testing.assert_array_equal(lse1.cpu().numpy(), lse2.cpu().numpy())


def test_attention_mask_sensitivity():
    shape = ATTN_SHAPES[0]
    inp = G.attention_inputs(shape, 2.0)
    out1, _ = _run_attention(shape, inp)
    inp2 = dict(inp)
    inp2["txt_valid"] = np.array([30, 40], np.int32)
    out2, _ = _run_attention(shape, inp2)
    o2, _ = _oracle_attention(shape, inp2)
    assert_parity(host(out2), o2.reshape(host(out2).shape), "valid length 30")
    moved = np.abs(host(out1)[0] - host(out2)[0]).max()
    assert moved > 10 * 2e-2 / 4, f"changing the valid length moved the output only {moved}"


def test_attention_q_zero_is_mean_of_valid_values():
    shape = ATTN_SHAPES[1]
    inp = G.attention_inputs(shape)
    inp["q"] = np.zeros_like(inp["q"])
    out, lse = _run_attention(shape, inp)
    B, N, H, d = shape.batch, shape.n_tok, shape.heads, shape.head_dim
    v = _dec(inp["v"]).reshape(B, N, H, d)
    got = host(out).reshape(B, N, H, d)
    for b in range(B):
        nk = shape.n_vis + int(inp["txt_valid"][b])
        want = np.broadcast_to(v[b, :nk].mean(axis=0), (N, H, d))
        assert_parity(got[b], want, f"Q=0 row {b}")
        np.testing.assert_allclose(host(lse)[b], math.log(nk), rtol=1e-5)


def test_attention_single_valid_key_exact():
    shape = C.AttnShape("one_key", batch=1, n_vis=1, n_txt=70, heads=2, head_dim=64,
                        txt_valid=("fixed", (0,)), seed=44)
    inp = G.attention_inputs(shape)
    out, _ = _run_attention(shape, inp)
    want = np.broadcast_to(inp["v"][0, 0], (shape.n_tok, shape.hidden))
    np.testing.assert_array_equal(bits_of(out)[0], want)


def test_attention_deterministic():
    shape = ATTN_SHAPES[1]
    inp = G.attention_inputs(shape, 3.0)
    a, la = _run_attention(shape, inp)
    b, lb = _run_attention(shape, inp)
    np.testing.assert_array_equal(bits_of(a), bits_of(b))
    np.testing.assert_array_equal(la.cpu().numpy(), lb.cpu().numpy())


def test_attention_strided_qkv_buffer():
    """q, k, v as column blocks of one [B, N, 3*H*d] buffer (the block's layout)."""
    shape = ATTN_SHAPES[0]
    inp = G.attention_inputs(shape)
    B, N, HD = shape.batch, shape.n_tok, shape.hidden
    qkv = np.concatenate([inp["q"], inp["k"], inp["v"]], axis=-1)
    t = dev_bf16(qkv)
    out = torch.empty((B, N, HD + 64), dtype=torch.bfloat16, device="cuda")
    desc = D.attn_desc(B, shape.n_vis, shape.n_txt, shape.heads, shape.head_dim, inp["txt_valid"])
    D.dit_joint_attention(desc, t, t[..., HD:], t[..., 2 * HD:], 3 * HD, out, HD + 64)
    torch.cuda.synchronize()
    o, _ = _oracle_attention(shape, inp)
    assert_parity(host(out)[..., :HD], o.reshape(B, N, HD), "strided qkv")


# ------------------------------------------------------------------ sampler

@pytest.mark.parametrize("n,cfg", [(1001, True), (4096 * 64, True), (37, False)])
def test_euler_step(n, cfg):
    x0 = G.normal_bf16(50, (n,))
    vc = G.normal_bf16(51, (n,))
    vu = G.normal_bf16(52, (n,))
    x = dev_f32_from_bf16(x0)
    D.dit_euler_step(x, dev_bf16(vc), dev_bf16(vu) if cfg else None, n, 5.0, 0.7, 0.7 - 1 / 30)
    torch.cuda.synchronize()
    v = O.cfg_combine(_dec(vc), _dec(vu), 5.0) if cfg else _dec(vc)
    want = O.euler_update(_dec(x0), v, 0.7, 0.7 - 1 / 30)
    assert_parity(host(x), want, f"euler n={n}", max_abs=1e-5, rel_l2=1e-6)


def test_timestep_features():
    sig = O.sigma_schedule(30)[:-1]
    t = torch.tensor(sig, dtype=torch.float32, device="cuda")
    out = torch.empty((30, 256), dtype=torch.bfloat16, device="cuda")
    D.dit_timestep_features(t, 30, 256, 1000.0, out)
    torch.cuda.synchronize()
    want = np.stack([O.timestep_features(1000.0 * s, 256) for s in np.float32(sig)])
    # fp32 angles up to 1000 rad carry ~1e-4 absolute phase error
    assert_parity(host(out), want, "timestep features", max_abs=8e-3, rel_l2=5e-3)


def test_casts_roundtrip():
    a = G.normal_bf16(60, (33, 40))
    f = torch.full((33, 48), float("nan"), dtype=torch.float32, device="cuda")
    D.dit_cast_bf16_f32(dev_bf16(a), 40, 33, 40, f, 48)
    b = torch.zeros((33, 44), dtype=torch.bfloat16, device="cuda")
    D.dit_cast_f32_bf16(f, 48, 33, 40, b, 44)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(f)[:, :40], _dec(a))
    assert np.isnan(host(f)[:, 40:]).all()
    np.testing.assert_array_equal(bits_of(b)[:, :40], a)


@pytest.mark.parametrize("M,N,K", [(300, 200, 192), (33, 64, 64)])
def test_linear_residual_small_tiles(M, N, K):
    a, w, b = _gemm_case(300 + M, M, N, K)
    x0 = G.normal_bf16(14, (M, N))
    want = _dec(x0) + O.linear(_dec(a), _dec(w), _dec(b))
    x = dev_f32_from_bf16(x0)
    D.dit_linear(dev_bf16(a), K, dev_bf16(w), dev_bf16(b), M, N, K, D.EPI_RES_F32, x, N)
    torch.cuda.synchronize()
    assert_parity(host(x), want, f"residual {M}x{N}x{K}", max_abs=1e-4 * np.abs(want).max(),
                  rel_l2=1e-5)


@pytest.mark.parametrize("rows,hidden", [(300, 256), (7, 5120)])
def test_layernorm_without_modulation(rows, hidden):
    x = G.normal_bf16(22, (rows, hidden), 2.0, 0.3)
    want = O.adaln_modulate(_dec(x), np.zeros(hidden), np.zeros(hidden), 1e-6)
    out = torch.empty((rows, hidden), dtype=torch.bfloat16, device="cuda")
    D.dit_adaln_modulate(dev_f32_from_bf16(x), rows, hidden, rows, None, None, 0, 1e-6, out)
    torch.cuda.synchronize()
    assert_bf16_ulp(host(out), want, f"layernorm {rows}x{hidden}")
