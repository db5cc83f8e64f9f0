"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol include/dit.h declares, and rejects bad arguments on the host with the
documented status before anything is launched (the pointers passed here are
never dereferenced)."""

import ctypes
import os
import re

import pytest

import diffusion_transformer_denoising_dit_amd as D
from synthetic import configs as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20  # a 256-byte-aligned address that is never dereferenced


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "dit.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = D.lib()
    declared = _declared_functions()
    assert len(declared) >= 14
    for name in declared:
        assert hasattr(L, name), f"libdit.so does not export {name}"
    assert sorted(declared) == sorted(D.EXPORTED)
    assert "gfx950" in D.dit_version()


def test_status_strings():
    L = D.lib()
    for code, name in D._lib.STATUS.items():
        assert L.dit_status_string(code).decode() == name


def _expect(status, fn, *args, **kw):
    with pytest.raises(D.DitError) as e:
        fn(*args, **kw)
    assert e.value.status_name == status, str(e.value)
    return str(e.value)


def _attn(batch=1, n_vis=64, n_txt=16, heads=2, head_dim=64, valid=(4,)):
    return D.attn_desc(batch, n_vis, n_txt, heads, head_dim, list(valid))


def test_attention_argument_errors():
    f = D.dit_joint_attention
    hd = 128
    _expect("DIT_EINVAL", f, _attn(batch=0), FAKE, FAKE, FAKE, hd, FAKE * 2, hd, stream=0)
    _expect("DIT_EINVAL", f, _attn(batch=9, valid=[0] * 8), FAKE, FAKE, FAKE, hd, FAKE * 2, hd, stream=0)
    _expect("DIT_EUNSUPPORTED", f, _attn(head_dim=96), FAKE, FAKE, FAKE, 192, FAKE * 2, 192, stream=0)
    _expect("DIT_EINVAL", f, _attn(valid=(17,)), FAKE, FAKE, FAKE, hd, FAKE * 2, hd, stream=0)
    _expect("DIT_EINVAL", f, _attn(valid=(-1,)), FAKE, FAKE, FAKE, hd, FAKE * 2, hd, stream=0)
    _expect("DIT_EINVAL", f, _attn(n_vis=0, valid=(0,)), FAKE, FAKE, FAKE, hd, FAKE * 2, hd, stream=0)
    _expect("DIT_EINVAL", f, _attn(), None, FAKE, FAKE, hd, FAKE * 2, hd, stream=0)
    _expect("DIT_EINVAL", f, _attn(), FAKE, FAKE, FAKE, hd - 8, FAKE * 2, hd, stream=0)
    _expect("DIT_EINVAL", f, _attn(), FAKE, FAKE, FAKE, hd + 4, FAKE * 2, hd, stream=0)
    _expect("DIT_EUNSUPPORTED", f, _attn(), FAKE, FAKE, FAKE, (1 << 24) + 8, FAKE * 2, hd, stream=0)
    _expect("DIT_EINVAL", f, _attn(), FAKE + 2, FAKE, FAKE, hd, FAKE * 2, hd, stream=0)
    # out aliasing q
    _expect("DIT_EINVAL", f, _attn(), FAKE, FAKE * 4, FAKE * 4, hd, FAKE + 256, hd, stream=0)
    _expect("DIT_EINVAL", f, _attn(), FAKE, FAKE, FAKE, hd, FAKE * 2, hd, softmax_scale=-1.0, stream=0)
    # query tiles x heads x batch beyond the kernel's 1-D grid (2^30 tokens, 8 heads, 8 rows)
    _expect("DIT_EUNSUPPORTED", f, _attn(batch=8, n_vis=(1 << 30) - 16, heads=8, valid=[4] * 8),
            FAKE, FAKE, FAKE, 1024, FAKE * 2, 1024, stream=0)
    # optional workspace (the split of an under-filled last round): aligned,
    # at least dit_joint_attention_workspace_bytes(), overlapping nothing
    wsb = D.dit_joint_attention_workspace_bytes()
    assert wsb >= 448 * 256 * 129 * 4
    ws = FAKE * 8
    _expect("DIT_EINVAL", f, _attn(), FAKE, FAKE, FAKE, hd, FAKE * 2, hd, workspace=ws + 64,
            workspace_bytes=wsb, stream=0)
    msg = _expect("DIT_EWORKSPACE", f, _attn(), FAKE, FAKE, FAKE, hd, FAKE * 2, hd, workspace=ws,
                  workspace_bytes=wsb - 256, stream=0)
    assert str(wsb) in msg
    _expect("DIT_EINVAL", f, _attn(), FAKE, FAKE, FAKE, hd, FAKE * 2, hd, workspace=FAKE * 2 - 4096,
            workspace_bytes=wsb, stream=0)


def test_partial_attention_and_merge_argument_errors():
    f = D.dit_attention_partial
    hd = 128
    ok = dict(batch=1, n_q=16, n_k=8, heads=1, head_dim=128, k_valid=[8])

    def pd(**kw):
        a = dict(ok)
        a.update(kw)
        return D.partial_desc(a["batch"], a["n_q"], a["n_k"], a["heads"], a["head_dim"], a["k_valid"])

    args = (FAKE, hd, FAKE * 2, FAKE * 3, hd, FAKE * 4, hd, FAKE * 5)
    _expect("DIT_EINVAL", f, pd(batch=0), *args, stream=0)
    _expect("DIT_EINVAL", f, pd(n_k=0, k_valid=[0]), *args, stream=0)
    _expect("DIT_EINVAL", f, pd(k_valid=[9]), *args, stream=0)
    _expect("DIT_EINVAL", f, pd(k_valid=[-1]), *args, stream=0)
    _expect("DIT_EUNSUPPORTED", f, pd(head_dim=96), FAKE, 96, FAKE * 2, FAKE * 3, 96, FAKE * 4, 96,
            FAKE * 5, stream=0)
    _expect("DIT_EINVAL", f, pd(), FAKE, hd, FAKE * 2, FAKE * 3, hd, FAKE * 4, hd, None, stream=0)
    _expect("DIT_EINVAL", f, pd(), FAKE, hd, FAKE * 2, FAKE * 3, hd, FAKE * 4, hd - 4, FAKE * 5,
            stream=0)
    _expect("DIT_EINVAL", f, pd(), FAKE, hd, FAKE * 2, FAKE * 3, hd, FAKE + 64, hd, FAKE * 5,
            stream=0)  # out overlaps q
    _expect("DIT_EUNSUPPORTED", f, pd(), FAKE, hd, FAKE * 2, FAKE * 3, (1 << 24) + 8, FAKE * 4, hd,
            FAKE * 5, stream=0)
    # query tiles x heads x batch beyond the kernel's 1-D grid
    _expect("DIT_EUNSUPPORTED", f, pd(batch=8, n_q=1 << 30, heads=2, k_valid=[8] * 8), *args,
            stream=0)
    m = D.dit_attention_merge
    _expect("DIT_EINVAL", m, 1, 16, 1, 128, [], hd, [], FAKE, hd, stream=0)
    _expect("DIT_EINVAL", m, 1, 16, 1, 128, [FAKE] * 33, hd, [FAKE * 2] * 33, FAKE * 3, hd,
            stream=0)
    _expect("DIT_EUNSUPPORTED", m, 1, 16, 1, 96, [FAKE], 96, [FAKE * 2], FAKE * 3, 96, stream=0)
    _expect("DIT_EINVAL", m, 1, 16, 1, 128, [FAKE], hd, [None], FAKE * 3, hd, stream=0)
    _expect("DIT_EINVAL", m, 1, 16, 1, 128, [FAKE], hd, [FAKE * 2], FAKE + 16, hd, stream=0)
    _expect("DIT_EINVAL", m, 1, 16, 1, 128, [FAKE], hd - 4, [FAKE * 2], FAKE * 3, hd, stream=0)


def test_linear_argument_errors():
    f = D.dit_linear
    _expect("DIT_EUNSUPPORTED", f, FAKE, 96, FAKE * 2, None, 4, 8, 96, D.EPI_BF16, FAKE * 4, 8, stream=0)
    _expect("DIT_EUNSUPPORTED", f, FAKE, 64, FAKE * 2, None, 4, 12, 64, D.EPI_BF16, FAKE * 4, 16, stream=0)
    _expect("DIT_EINVAL", f, FAKE, 64, FAKE * 2, None, 4, 8, 64, 9, FAKE * 4, 8, stream=0)
    # rows beyond DIT_LINEAR_MAX_M = 65535 * 256 (the general kernel's grid)
    _expect("DIT_EUNSUPPORTED", f, FAKE, 64, FAKE * 2, None, 65535 * 256 + 1, 8, 64, D.EPI_BF16,
            FAKE * 4, 8, stream=0)
    _expect("DIT_EINVAL", f, FAKE, 32, FAKE * 2, None, 4, 8, 64, D.EPI_BF16, FAKE * 4, 8, stream=0)
    _expect("DIT_EINVAL", f, FAKE, 64, FAKE * 2, None, 4, 8, 64, D.EPI_GATED_RES_F32, FAKE * 4, 8, stream=0)
    _expect("DIT_EINVAL", f, FAKE, 64, FAKE * 2, None, 4, 8, 64, D.EPI_BF16, FAKE + 64, 8, stream=0)
    _expect("DIT_EINVAL", f, None, 64, FAKE * 2, None, 4, 8, 64, D.EPI_BF16, FAKE * 4, 8, stream=0)
    # the gated residual epilogue: out (fp32, 4 x 8 x 4 B = 128 B) may not overlap
    # A (4 x 64 bf16 = 512 B), the bias (16 B) or the gate rows it reads
    g = dict(gate=FAKE * 5, gate_stride=8, gate_rows=4)
    _expect("DIT_EINVAL", f, FAKE, 64, FAKE * 2, None, 4, 8, 64, D.EPI_GATED_RES_F32, FAKE + 256, 8,
            **g, stream=0)
    _expect("DIT_EINVAL", f, FAKE, 64, FAKE * 2, FAKE * 4 + 64, 4, 8, 64, D.EPI_GATED_RES_F32,
            FAKE * 4, 8, **g, stream=0)
    _expect("DIT_EINVAL", f, FAKE, 64, FAKE * 2, None, 4, 8, 64, D.EPI_GATED_RES_F32, FAKE * 5 - 64,
            8, **g, stream=0)
    _expect("DIT_EINVAL", f, FAKE, 64, FAKE * 2, FAKE * 4 + 16, 4, 8, 64, D.EPI_BF16, FAKE * 4, 8,
            stream=0)
    # the optional K-split scratch: 256-byte aligned, at least
    # dit_linear_workspace_bytes(), overlapping none of the operands or out
    wsb = D.dit_linear_workspace_bytes()
    assert wsb == 256 * 256 * 256 * 4
    far = FAKE * 64
    _expect("DIT_EINVAL", f, FAKE, 64, FAKE * 2, None, 4, 8, 64, D.EPI_BF16, FAKE * 4, 8,
            workspace=far + 16, workspace_bytes=wsb, stream=0)
    _expect("DIT_EWORKSPACE", f, FAKE, 64, FAKE * 2, None, 4, 8, 64, D.EPI_BF16, FAKE * 4, 8,
            workspace=far, workspace_bytes=wsb - 256, stream=0)
    for clash in (FAKE, FAKE * 2, FAKE * 4):  # A, W, out inside the workspace's range
        _expect("DIT_EINVAL", f, FAKE, 64, FAKE * 2, None, 4, 8, 64, D.EPI_BF16, FAKE * 4, 8,
                workspace=clash - 256, workspace_bytes=wsb, stream=0)
    _expect("DIT_EINVAL", f, FAKE, 64, FAKE * 2, None, 4, 8, 64, D.EPI_GATED_RES_F32, FAKE * 4, 8,
            **g, workspace=FAKE * 5 - 256, workspace_bytes=wsb, stream=0)
    # m == 0 is a no-op that succeeds without touching the GPU
    f(FAKE, 64, FAKE * 2, None, 0, 8, 64, D.EPI_BF16, FAKE * 4, 8, stream=0)


def _block(**over):
    s = C.C1
    d = D.block_desc(s, [20])
    for k, v in over.items():
        if k in ("batch", "n_vis", "n_txt", "heads", "head_dim"):
            setattr(d.attn, k, v)
        else:
            setattr(d, k, v)
    return d


def test_block_descriptor_errors_and_workspace():
    ws = D.dit_block_workspace_bytes(_block())
    s = C.C1
    M = s.batch * s.n_tok
    assert ws >= M * s.hidden * 2 + M * max(3 * s.hidden, s.mlp) * 2
    for over, status in [({"hidden": 320}, "DIT_EINVAL"), ({"mlp": 1000}, "DIT_EUNSUPPORTED"),
                         ({"grid_w": 15}, "DIT_EINVAL"), ({"rope_h": 31}, "DIT_EINVAL"),
                         ({"rope_h": 30}, "DIT_EINVAL"), ({"rope_theta": 0.0}, "DIT_EINVAL"),
                         ({"mod_stride": -4}, "DIT_EINVAL"),
                         ({"batch": 8, "n_vis": 2_100_000}, "DIT_EUNSUPPORTED")]:
        d = _block(**over)
        with pytest.raises(D.DitError) as e:
            D.dit_block_workspace_bytes(d)
        W = {n: FAKE for n in ("w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "w_up", "b_up",
                               "w_dn", "b_dn")}
        _expect(status, D.dit_block_forward, d, W, FAKE, FAKE * 64, FAKE * 1024, 1 << 30, stream=0)
    W = {n: FAKE for n in ("w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "w_up", "b_up", "w_dn",
                           "b_dn")}
    _expect("DIT_EWORKSPACE", D.dit_block_forward, _block(), W, FAKE, FAKE * 64, FAKE * 1024, ws - 1,
            stream=0)
    W2 = dict(W, w_o=None)
    _expect("DIT_EINVAL", D.dit_block_forward, _block(), W2, FAKE, FAKE * 64, FAKE * 1024, ws, stream=0)
    # x overlapping the workspace
    _expect("DIT_EINVAL", D.dit_block_forward, _block(), W, FAKE, FAKE * 64, FAKE * 64, ws, stream=0)


def test_other_entry_points_argument_errors():
    _expect("DIT_EINVAL", D.dit_euler_step, None, FAKE, None, 16, 5.0, 1.0, 0.9, stream=0)
    _expect("DIT_EINVAL", D.dit_euler_step, FAKE + 4, FAKE * 2, None, 16, 5.0, 1.0, 0.9, stream=0)
    _expect("DIT_EINVAL", D.dit_euler_step, FAKE, FAKE * 2, None, 16, float("nan"), 1.0, 0.9, stream=0)
    _expect("DIT_EINVAL", D.dit_euler_step, FAKE, FAKE + 8, None, 16, 5.0, 1.0, 0.9, stream=0)
    D.dit_euler_step(FAKE, FAKE * 2, None, 0, 5.0, 1.0, 0.9, stream=0)  # n == 0: no-op
    _expect("DIT_EUNSUPPORTED", D.dit_adaln_modulate, FAKE, 4, 100, 4, FAKE, FAKE, 0, 1e-6, FAKE * 2,
            stream=0)
    _expect("DIT_EINVAL", D.dit_adaln_modulate, FAKE, 4, 256, 0, FAKE, FAKE, 0, 1e-6, FAKE * 2, stream=0)
    _expect("DIT_EINVAL", D.dit_adaln_modulate, FAKE, 4, 256, 4, FAKE, FAKE, 0, 1e-6, FAKE + 512,
            stream=0)
    _expect("DIT_EINVAL", D.dit_timestep_features, FAKE, 30, 255, 1000.0, FAKE * 2, stream=0)
    _expect("DIT_EINVAL", D.dit_cast_f32_bf16, FAKE, 6, 4, 6, FAKE * 2, 8, stream=0)
    _expect("DIT_EINVAL", D.dit_qk_rmsnorm_rope, _block(), FAKE, 100, FAKE, FAKE, stream=0)
    assert D.lib().dit_last_error().decode() != ""


def _fake_model(shape):
    desc = D.model_desc(shape, [int(v) for v in (10, 3)][:shape.block.batch])
    glue = {n: (1 << 24) * (i + 1) for i, n in enumerate(
        ("t_w1", "t_b1", "t_w2", "t_b2", "in_w", "in_b", "fin_w", "fin_b", "out_w", "out_b", "text"))}
    blk = {n: (1 << 32) + (1 << 24) * i for i, n in enumerate(
        ("w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "w_up", "b_up", "w_dn", "b_dn"))}
    w = D.model_weights(glue, [blk] * shape.depth, [1 << 34] * shape.depth, [1 << 35] * shape.depth)
    return desc, w


def test_step_cache_argument_errors():
    f = D.dit_change_score
    wsb = D.dit_change_score_workspace_bytes()
    assert wsb >= 8
    A, B, S_, W = 1 << 36, 1 << 37, 1 << 38, 1 << 39
    _expect("DIT_EINVAL", f, A, B, 5, 16, 0, S_, W, wsb, stream=0)          # dtype
    _expect("DIT_EINVAL", f, A, B, D.DTYPE_BF16, 0, 0, S_, W, wsb, stream=0)  # n < 1
    _expect("DIT_EINVAL", f, A, B, D.DTYPE_BF16, 16, 2, S_, W, wsb, stream=0)
    _expect("DIT_EINVAL", f, None, B, D.DTYPE_BF16, 16, 0, S_, W, wsb, stream=0)
    _expect("DIT_EINVAL", f, A + 2, B, D.DTYPE_BF16, 16, 0, S_, W, wsb, stream=0)
    _expect("DIT_EWORKSPACE", f, A, B, D.DTYPE_BF16, 16, 0, S_, W, wsb - 4, stream=0)
    _expect("DIT_EINVAL", f, A, A + 16, D.DTYPE_F32, 16, 1, S_, W, wsb, stream=0)  # update overlap
    _expect("DIT_EINVAL", f, A, B, D.DTYPE_F32, 16, 0, A + 32, W, wsb, stream=0)  # score in cur

    from synthetic import configs as C_
    desc, w = _fake_model(C_.TINY_LOOP)
    wsb = D.dit_denoise_workspace_bytes(desc)
    L, P, Dv, S_, W = 1 << 40, 1 << 41, 1 << 42, 1 << 43, 1 << 44
    g = D.dit_denoise_step_cached
    args = (1.0, 0.9, 5.0)
    _expect("DIT_EINVAL", g, desc, w, L, *args, 2, 1, P, Dv, S_, W, wsb, stream=0)       # action
    _expect("DIT_EINVAL", g, desc, w, L, *args, D.STEP_SKIP, 0, P, Dv, S_, W, wsb, stream=0)
    _expect("DIT_EINVAL", g, desc, w, L, *args, D.STEP_FULL, 3, P, Dv, S_, W, wsb, stream=0)
    _expect("DIT_EINVAL", g, desc, w, L, *args, D.STEP_FULL, 1, None, Dv, S_, W, wsb, stream=0)
    _expect("DIT_EINVAL", g, desc, w, L, *args, D.STEP_FULL, 1, P, P + 64, S_, W, wsb, stream=0)
    _expect("DIT_EINVAL", g, desc, w, L, *args, D.STEP_FULL, 1, P + 8, Dv, S_, W, wsb, stream=0)
    _expect("DIT_EWORKSPACE", g, desc, w, L, *args, D.STEP_FULL, 1, P, Dv, S_, W, wsb - 256,
            stream=0)
    _expect("DIT_EINVAL", g, desc, w, L, 1.0, float("inf"), 5.0, D.STEP_FULL, 1, P, Dv, S_, W, wsb,
            stream=0)
    p = D.dit_cache_probe
    _expect("DIT_EINVAL", p, desc, w, L, 0.5, P, 2, S_, W, wsb, stream=0)
    _expect("DIT_EINVAL", p, desc, w, L, 0.5, None, 1, S_, W, wsb, stream=0)
    _expect("DIT_EINVAL", p, desc, w, L, 0.5, P + 2, 1, S_, W, wsb, stream=0)
    _expect("DIT_EINVAL", p, desc, w, L, 0.5, W + 256, 1, S_, W, wsb, stream=0)  # saved in workspace


def test_mmdit_block_argument_errors():
    desc = _block()
    nb = D.dit_double_block_workspace_bytes(desc)
    assert nb == D.dit_block_workspace_bytes(desc)
    wi = {n: (1 << 32) + (1 << 24) * i for i, n in enumerate(
        ("w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "w_up", "b_up", "w_dn", "b_dn"))}
    wt = {n: v + (1 << 31) for n, v in wi.items()}
    MI, MT, XI, XT, W = 1 << 36, 1 << 37, 1 << 38, 1 << 39, 1 << 40
    f = D.dit_double_block_forward
    f_ok = (desc, wi, wt, MI, MT, XI, XT, W, nb)
    bad_w = dict(wt, w_o=None)
    _expect("DIT_EINVAL", f, desc, wi, bad_w, MI, MT, XI, XT, W, nb, stream=0)
    _expect("DIT_EINVAL", f, desc, wi, wt, None, MT, XI, XT, W, nb, stream=0)
    _expect("DIT_EINVAL", f, desc, wi, wt, MI, MT, XI, None, W, nb, stream=0)
    _expect("DIT_EINVAL", f, desc, wi, wt, MI, MT, XI, XI + 64, W, nb, stream=0)  # streams overlap
    _expect("DIT_EWORKSPACE", f, desc, wi, wt, MI, MT, XI, XT, W, nb - 256, stream=0)
    assert len(f_ok) == 9
    g = D.dit_single_block_forward
    sn = D.dit_single_block_workspace_bytes(desc)
    sw = {n: (1 << 32) + (1 << 24) * i for i, n in enumerate(("w1", "b1", "g_q", "g_k", "w2", "b2"))}
    _expect("DIT_EINVAL", g, desc, dict(sw, w2=None), MI, XI, W, sn, stream=0)
    _expect("DIT_EINVAL", g, desc, dict(sw, b1=(1 << 32) + 2), MI, XI, W, sn, stream=0)
    _expect("DIT_EINVAL", g, desc, sw, MI, W + 256, W, sn, stream=0)  # x inside the workspace
    _expect("DIT_EWORKSPACE", g, desc, sw, MI, XI, W, sn - 256, stream=0)


def test_wan_block_argument_errors():
    desc = _block()
    nb = D.dit_wan_block_workspace_bytes(desc)
    w = {n: (1 << 32) + (1 << 24) * i for i, n in enumerate(D.WAN_WEIGHT_NAMES)}
    MOD, X, CTX, W = 1 << 36, 1 << 37, 1 << 38, 1 << 40
    f = D.dit_wan_block_forward
    _expect("DIT_EINVAL", f, desc, dict(w, w_ckv=None), MOD, X, CTX, W, nb, stream=0)
    _expect("DIT_EINVAL", f, desc, dict(w, g_cq=(1 << 32) + 8), MOD, X, CTX, W, nb, stream=0)
    _expect("DIT_EINVAL", f, desc, w, MOD, X, None, W, nb, stream=0)         # context needed
    _expect("DIT_EINVAL", f, desc, w, MOD, X, X + 64, W, nb, stream=0)      # ctx inside x
    _expect("DIT_EINVAL", f, desc, w, MOD, W + 512, CTX, W, nb, stream=0)   # x inside workspace
    _expect("DIT_EWORKSPACE", f, desc, w, MOD, X, CTX, W, nb - 256, stream=0)
