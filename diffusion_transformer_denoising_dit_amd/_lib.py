"""ctypes binding of ``libdit.so`` (the C ABI declared in include/dit.h).

Argument marshalling only: every function takes device pointers (plain ints or
anything with ``data_ptr()``, e.g. torch tensors), host descriptors and a
stream handle, calls the C entry point of the same name and raises
``DitError`` on a non-OK status.  No arithmetic of the method happens here,
and there is no fallback: if the library is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdit.so")

DIT_MAX_BATCH = 8
STATUS = {0: "DIT_OK", 1: "DIT_EINVAL", 2: "DIT_EUNSUPPORTED", 3: "DIT_EWORKSPACE", 4: "DIT_EHIP"}
EPI_BF16, EPI_GELU_BF16, EPI_SILU_BF16, EPI_F32, EPI_GATED_RES_F32, EPI_RES_F32 = range(6)

EXPORTED = (
    "dit_joint_attention", "dit_joint_attention_workspace_bytes", "dit_attention_partial",
    "dit_attention_merge", "dit_linear_workspace_bytes",
    "dit_linear", "dit_adaln_modulate", "dit_qk_rmsnorm_rope",
    "dit_block_workspace_bytes", "dit_block_forward", "dit_euler_step",
    "dit_timestep_features", "dit_cast_f32_bf16", "dit_cast_bf16_f32", "dit_debug_positions",
    "dit_denoise_workspace_bytes", "dit_denoise_step",
    "dit_change_score_workspace_bytes", "dit_change_score", "dit_change_score_noalloc",
    "dit_cache_probe",
    "dit_denoise_step_cached", "dit_cache_ctrl_init", "dit_cache_ctrl_decide",
    "dit_cache_ctrl_observe",
    "dit_double_block_workspace_bytes", "dit_double_block_forward",
    "dit_single_block_workspace_bytes", "dit_single_block_forward",
    "dit_wan_block_workspace_bytes", "dit_wan_block_forward",
    "dit_status_string", "dit_last_error", "dit_version",
)
DTYPE_BF16, DTYPE_F32 = 0, 1
STEP_FULL, STEP_SKIP = 0, 1
CACHE_OFF, CACHE_CADENCE, CACHE_ONLINE_DELTA, CACHE_TEACACHE = range(4)
CACHE_MAX_COEF = 8


class DitError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS.get(status, f"status {status}")
        super().__init__(f"{self.status_name}: {message}")


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_vis", ctypes.c_int32), ("n_txt", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("txt_valid", ctypes.c_int32 * DIT_MAX_BATCH)]


class PartialDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k_valid", ctypes.c_int32 * DIT_MAX_BATCH)]


class MergeDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("parts", ctypes.c_int32)]


class BlockDesc(ctypes.Structure):
    _fields_ = [("attn", AttnDesc), ("hidden", ctypes.c_int32), ("mlp", ctypes.c_int32),
                ("grid_t", ctypes.c_int32), ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("rope_t", ctypes.c_int32), ("rope_h", ctypes.c_int32), ("rope_w", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("ln_eps", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("mod_stride", ctypes.c_int64)]


_WEIGHT_NAMES = ("w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "w_up", "b_up", "w_dn", "b_dn")


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_NAMES]


class LinearArgs(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("lda", ctypes.c_int64), ("w", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("m", ctypes.c_int64), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("epilogue", ctypes.c_int32), ("out", ctypes.c_void_p),
                ("ldc", ctypes.c_int64), ("gate", ctypes.c_void_p), ("gate_stride", ctypes.c_int64),
                ("gate_rows", ctypes.c_int64), ("group_rows", ctypes.c_int64),
                ("a_group_stride", ctypes.c_int64), ("c_group_stride", ctypes.c_int64),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class ModelDesc(ctypes.Structure):
    _fields_ = [("block", BlockDesc), ("depth", ctypes.c_int32), ("latent_channels", ctypes.c_int32),
                ("freq_dim", ctypes.c_int32), ("cfg", ctypes.c_int32), ("t_scale", ctypes.c_float)]


_GLUE_NAMES = ("t_w1", "t_b1", "t_w2", "t_b2", "in_w", "in_b", "fin_w", "fin_b", "out_w", "out_b",
               "text")


class ModelWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _GLUE_NAMES] + [
        ("blocks", ctypes.POINTER(BlockWeights)),
        ("mod_w", ctypes.POINTER(ctypes.c_void_p)),
        ("mod_b", ctypes.POINTER(ctypes.c_void_p))]


class SingleBlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "b1", "g_q", "g_k", "w2", "b2")]


WAN_WEIGHT_NAMES = ("w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "w_cq", "b_cq", "w_ckv", "b_ckv",
                    "g_cq", "g_ck", "w_co", "b_co", "w_up", "b_up", "w_dn", "b_dn")


class WanBlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WAN_WEIGHT_NAMES]


class CachePolicy(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("n_steps", ctypes.c_int32), ("warmup", ctypes.c_int32),
                ("cooldown", ctypes.c_int32), ("cadence", ctypes.c_int32), ("n_coef", ctypes.c_int32),
                ("alpha", ctypes.c_double), ("threshold", ctypes.c_double),
                ("coef", ctypes.c_double * CACHE_MAX_COEF)]


class CacheCtrl(ctypes.Structure):
    _fields_ = [("policy", CachePolicy), ("next_step", ctypes.c_int32), ("n_full", ctypes.c_int32),
                ("last_skipped", ctypes.c_int32), ("skip_next", ctypes.c_int32),
                ("have_first", ctypes.c_int32), ("first_change", ctypes.c_double),
                ("acc", ctypes.c_double)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdit.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m diffusion_transformer_denoising_dit_amd.build` (needs ROCm hipcc)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        sig = {
            "dit_joint_attention": (st, [ctypes.POINTER(AttnDesc), vp, vp, vp, i64, vp, i64, vp, f32, vp,
                                         ctypes.c_size_t, vp]),
            "dit_joint_attention_workspace_bytes": (ctypes.c_size_t, []),
            "dit_attention_partial": (st, [ctypes.POINTER(PartialDesc), vp, i64, vp, vp, i64, vp, i64,
                                           vp, f32, vp]),
            "dit_attention_merge": (st, [ctypes.POINTER(MergeDesc), ctypes.POINTER(vp), i64,
                                         ctypes.POINTER(vp), vp, i64, vp, vp]),
            "dit_linear_workspace_bytes": (ctypes.c_size_t, []),
            "dit_linear": (st, [ctypes.POINTER(LinearArgs), vp]),
            "dit_adaln_modulate": (st, [vp, i64, i32, i64, vp, vp, i64, f32, vp, vp]),
            "dit_qk_rmsnorm_rope": (st, [ctypes.POINTER(BlockDesc), vp, i64, vp, vp, vp]),
            "dit_block_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(BlockDesc)]),
            "dit_block_forward": (st, [ctypes.POINTER(BlockDesc), ctypes.POINTER(BlockWeights), vp, vp,
                                       vp, ctypes.c_size_t, vp]),
            "dit_euler_step": (st, [vp, vp, vp, i64, f32, f32, f32, vp]),
            "dit_timestep_features": (st, [vp, i32, i32, f32, vp, vp]),
            "dit_cast_f32_bf16": (st, [vp, i64, i64, i32, vp, i64, vp]),
            "dit_cast_bf16_f32": (st, [vp, i64, i64, i32, vp, i64, vp]),
            "dit_debug_positions": (st, [ctypes.POINTER(BlockDesc), vp, vp]),
            "dit_denoise_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(ModelDesc)]),
            "dit_denoise_step": (st, [ctypes.POINTER(ModelDesc), ctypes.POINTER(ModelWeights), vp, f32,
                                      f32, f32, vp, ctypes.c_size_t, vp]),
            "dit_change_score_workspace_bytes": (ctypes.c_size_t, []),
            "dit_change_score": (st, [vp, vp, i32, i64, i32, vp, vp, ctypes.c_size_t, vp]),
            "dit_change_score_noalloc": (st, [vp, vp, i32, i64, i32, vp, vp]),
            "dit_cache_probe": (st, [ctypes.POINTER(ModelDesc), ctypes.POINTER(ModelWeights), vp, f32,
                                     vp, i32, vp, vp, ctypes.c_size_t, vp]),
            "dit_denoise_step_cached": (st, [ctypes.POINTER(ModelDesc), ctypes.POINTER(ModelWeights), vp,
                                             f32, f32, f32, i32, i32, vp, vp, vp, vp, ctypes.c_size_t,
                                             vp]),
            "dit_cache_ctrl_init": (st, [ctypes.POINTER(CacheCtrl), ctypes.POINTER(CachePolicy)]),
            "dit_cache_ctrl_decide": (st, [ctypes.POINTER(CacheCtrl), i32, f32,
                                           ctypes.POINTER(ctypes.c_int32)]),
            "dit_cache_ctrl_observe": (st, [ctypes.POINTER(CacheCtrl), f32]),
            "dit_double_block_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(BlockDesc)]),
            "dit_double_block_forward": (st, [ctypes.POINTER(BlockDesc), ctypes.POINTER(BlockWeights),
                                              ctypes.POINTER(BlockWeights), vp, vp, vp, vp, vp,
                                              ctypes.c_size_t, vp]),
            "dit_single_block_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(BlockDesc)]),
            "dit_single_block_forward": (st, [ctypes.POINTER(BlockDesc),
                                              ctypes.POINTER(SingleBlockWeights), vp, vp, vp,
                                              ctypes.c_size_t, vp]),
            "dit_wan_block_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(BlockDesc)]),
            "dit_wan_block_forward": (st, [ctypes.POINTER(BlockDesc), ctypes.POINTER(WanBlockWeights),
                                           vp, vp, vp, vp, ctypes.c_size_t, vp]),
            "dit_status_string": (ctypes.c_char_p, [st]),
            "dit_last_error": (ctypes.c_char_p, []),
            "dit_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != 0:
        raise DitError(status, lib().dit_last_error().decode())


def attn_desc(batch, n_vis, n_txt, heads, head_dim, txt_valid) -> AttnDesc:
    d = AttnDesc()
    d.batch, d.n_vis, d.n_txt, d.heads, d.head_dim = batch, n_vis, n_txt, heads, head_dim
    for i, L in enumerate(list(txt_valid)[:DIT_MAX_BATCH]):
        d.txt_valid[i] = int(L)
    return d


def block_desc(shape, txt_valid, mod_stride=None) -> BlockDesc:
    """Descriptor from a ``synthetic.BlockShape``-like object."""
    d = BlockDesc()
    d.attn = attn_desc(shape.batch, shape.n_vis, shape.n_txt, shape.heads, shape.head_dim, txt_valid)
    d.hidden, d.mlp = shape.hidden, shape.mlp
    d.grid_t, d.grid_h, d.grid_w = shape.grid
    d.rope_t, d.rope_h, d.rope_w = shape.rope
    d.rope_theta, d.ln_eps, d.rms_eps = shape.rope_theta, shape.ln_eps, shape.rms_eps
    d.mod_stride = 6 * shape.hidden if mod_stride is None else mod_stride
    return d


def dit_joint_attention(desc: AttnDesc, q, k, v, qkv_row_stride, out, out_row_stride,
                        lse=None, softmax_scale=0.0, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().dit_joint_attention(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), qkv_row_stride,
                                     _ptr(out), out_row_stride, _ptr(lse), softmax_scale,
                                     _ptr(workspace), workspace_bytes, _stream(stream)))


def dit_joint_attention_workspace_bytes() -> int:
    return int(lib().dit_joint_attention_workspace_bytes())


def partial_desc(batch, n_q, n_k, heads, head_dim, k_valid) -> PartialDesc:
    d = PartialDesc()
    d.batch, d.n_q, d.n_k, d.heads, d.head_dim = batch, n_q, n_k, heads, head_dim
    for i, L in enumerate(list(k_valid)[:DIT_MAX_BATCH]):
        d.k_valid[i] = int(L)
    return d


def dit_attention_partial(desc: PartialDesc, q, q_row_stride, k, v, kv_row_stride, out,
                          out_row_stride, lse, softmax_scale=0.0, stream=None):
    _check(lib().dit_attention_partial(ctypes.byref(desc), _ptr(q), q_row_stride, _ptr(k), _ptr(v),
                                       kv_row_stride, _ptr(out), out_row_stride, _ptr(lse),
                                       softmax_scale, _stream(stream)))


def dit_attention_merge(batch, n_q, heads, head_dim, outs, part_row_stride, lses, out,
                        out_row_stride, lse_out=None, stream=None):
    d = MergeDesc()
    d.batch, d.n_q, d.heads, d.head_dim, d.parts = batch, n_q, heads, head_dim, len(outs)
    po = (ctypes.c_void_p * max(1, len(outs)))(*[_ptr(t) for t in outs])
    pl = (ctypes.c_void_p * max(1, len(lses)))(*[_ptr(t) for t in lses])
    _check(lib().dit_attention_merge(ctypes.byref(d), po, part_row_stride, pl, _ptr(out),
                                     out_row_stride, _ptr(lse_out), _stream(stream)))


def dit_linear_workspace_bytes() -> int:
    return int(lib().dit_linear_workspace_bytes())


def dit_linear(a, lda, w, bias, m, n, k, epilogue, out, ldc, gate=None, gate_stride=0, gate_rows=1,
               group_rows=0, a_group_stride=0, c_group_stride=0, workspace=None, workspace_bytes=0,
               stream=None):
    args = LinearArgs(_ptr(a), lda, _ptr(w), _ptr(bias), m, n, k, epilogue, _ptr(out), ldc,
                      _ptr(gate), gate_stride, gate_rows, group_rows, a_group_stride, c_group_stride,
                      _ptr(workspace), workspace_bytes)
    _check(lib().dit_linear(ctypes.byref(args), _stream(stream)))


def dit_adaln_modulate(x, rows, hidden, rows_per_batch, shift, scale, mod_stride, eps, out,
                       stream=None):
    _check(lib().dit_adaln_modulate(_ptr(x), rows, hidden, rows_per_batch, _ptr(shift), _ptr(scale),
                                    mod_stride, eps, _ptr(out), _stream(stream)))


def dit_qk_rmsnorm_rope(desc: BlockDesc, qkv, row_stride, g_q, g_k, stream=None):
    _check(lib().dit_qk_rmsnorm_rope(ctypes.byref(desc), _ptr(qkv), row_stride, _ptr(g_q), _ptr(g_k),
                                     _stream(stream)))


def dit_block_workspace_bytes(desc: BlockDesc) -> int:
    n = lib().dit_block_workspace_bytes(ctypes.byref(desc))
    if n == 0:
        raise DitError(1, lib().dit_last_error().decode())
    return n


def block_weights(tensors: dict) -> BlockWeights:
    return BlockWeights(*[_ptr(tensors[n]) for n in _WEIGHT_NAMES])


def dit_block_forward(desc: BlockDesc, weights, mod, x, workspace, workspace_bytes, stream=None):
    w = weights if isinstance(weights, BlockWeights) else block_weights(weights)
    _check(lib().dit_block_forward(ctypes.byref(desc), ctypes.byref(w), _ptr(mod), _ptr(x),
                                   _ptr(workspace), workspace_bytes, _stream(stream)))


def dit_euler_step(x, v_cond, v_uncond, n, guidance, sigma, sigma_next, stream=None):
    _check(lib().dit_euler_step(_ptr(x), _ptr(v_cond), _ptr(v_uncond), n, guidance, sigma, sigma_next,
                                _stream(stream)))


def dit_timestep_features(sigma, n, dim, t_scale, out, stream=None):
    _check(lib().dit_timestep_features(_ptr(sigma), n, dim, t_scale, _ptr(out), _stream(stream)))


def dit_cast_f32_bf16(inp, ld_in, rows, cols, out, ld_out, stream=None):
    _check(lib().dit_cast_f32_bf16(_ptr(inp), ld_in, rows, cols, _ptr(out), ld_out, _stream(stream)))


def dit_cast_bf16_f32(inp, ld_in, rows, cols, out, ld_out, stream=None):
    _check(lib().dit_cast_bf16_f32(_ptr(inp), ld_in, rows, cols, _ptr(out), ld_out, _stream(stream)))


def dit_debug_positions(desc: BlockDesc, out, stream=None):
    _check(lib().dit_debug_positions(ctypes.byref(desc), _ptr(out), _stream(stream)))


def dit_version() -> str:
    return lib().dit_version().decode()


def model_desc(loop_shape, txt_valid, t_scale=1000.0) -> ModelDesc:
    """Descriptor from a ``synthetic.LoopShape``-like object."""
    m = ModelDesc()
    m.block = block_desc(loop_shape.block, txt_valid, 0)
    m.depth = loop_shape.depth
    m.latent_channels = loop_shape.latent_channels
    m.freq_dim = loop_shape.freq_dim
    m.cfg = 1 if loop_shape.cfg else 0
    m.t_scale = t_scale
    return m


def model_weights(glue: dict, blocks: list, mod_w: list, mod_b: list) -> ModelWeights:
    """glue: device tensors named as the C struct (t_w1 ... out_b, text);
    blocks: per-layer dicts of block weights; mod_w/mod_b: per-layer tensors.
    The returned struct keeps its host arrays alive as attributes."""
    mw = ModelWeights(*[_ptr(glue[n]) for n in _GLUE_NAMES])
    arr = (BlockWeights * len(blocks))(*[block_weights(b) for b in blocks])
    pw = (ctypes.c_void_p * len(mod_w))(*[_ptr(t) for t in mod_w])
    pb = (ctypes.c_void_p * len(mod_b))(*[_ptr(t) for t in mod_b])
    mw.blocks = ctypes.cast(arr, ctypes.POINTER(BlockWeights))
    mw.mod_w = ctypes.cast(pw, ctypes.POINTER(ctypes.c_void_p))
    mw.mod_b = ctypes.cast(pb, ctypes.POINTER(ctypes.c_void_p))
    mw._keep = (arr, pw, pb)
    return mw


def dit_denoise_workspace_bytes(desc: ModelDesc) -> int:
    n = lib().dit_denoise_workspace_bytes(ctypes.byref(desc))
    if n == 0:
        raise DitError(1, lib().dit_last_error().decode())
    return n


def dit_denoise_step(desc: ModelDesc, weights: ModelWeights, latent, sigma, sigma_next, guidance,
                     workspace, workspace_bytes, stream=None):
    _check(lib().dit_denoise_step(ctypes.byref(desc), ctypes.byref(weights), _ptr(latent), sigma,
                                  sigma_next, guidance, _ptr(workspace), workspace_bytes,
                                  _stream(stream)))


# ---------------------------------------------------------------------------
# step caching

def dit_change_score_workspace_bytes() -> int:
    return int(lib().dit_change_score_workspace_bytes())


def dit_change_score(cur, prev, dtype, n, update, score, workspace, workspace_bytes, stream=None):
    _check(lib().dit_change_score(_ptr(cur), _ptr(prev), dtype, n, int(update), _ptr(score),
                                  _ptr(workspace), workspace_bytes, _stream(stream)))


def dit_change_score_noalloc(cur, prev, dtype, n, update, score, stream=None):
    _check(lib().dit_change_score_noalloc(_ptr(cur), _ptr(prev), dtype, n, int(update), _ptr(score),
                                          _stream(stream)))


def dit_cache_probe(desc, weights, latent, sigma, saved, have_saved, score, workspace,
                    workspace_bytes, stream=None):
    _check(lib().dit_cache_probe(ctypes.byref(desc), ctypes.byref(weights), _ptr(latent), sigma,
                                 _ptr(saved), int(have_saved), _ptr(score), _ptr(workspace),
                                 workspace_bytes, _stream(stream)))


def dit_denoise_step_cached(desc, weights, latent, sigma, sigma_next, guidance, action, have_prev,
                            prev_v, delta_v, score, workspace, workspace_bytes, stream=None):
    _check(lib().dit_denoise_step_cached(ctypes.byref(desc), ctypes.byref(weights), _ptr(latent),
                                         sigma, sigma_next, guidance, action, int(have_prev),
                                         _ptr(prev_v), _ptr(delta_v), _ptr(score), _ptr(workspace),
                                         workspace_bytes, _stream(stream)))


def cache_policy(mode, n_steps, warmup=0, cooldown=0, cadence=2, alpha=0.6, threshold=0.0,
                 coef=(1.0, 0.0)) -> CachePolicy:
    p = CachePolicy()
    p.mode, p.n_steps, p.warmup, p.cooldown, p.cadence = mode, n_steps, warmup, cooldown, cadence
    p.alpha, p.threshold = alpha, threshold
    p.n_coef = len(coef)
    for i, c in enumerate(list(coef)[:CACHE_MAX_COEF]):
        p.coef[i] = c
    return p


class CacheController:
    """The library's host-side step-cache controller (dit_cache_ctrl_*)."""

    def __init__(self, policy: CachePolicy):
        self.state = CacheCtrl()
        _check(lib().dit_cache_ctrl_init(ctypes.byref(self.state), ctypes.byref(policy)))

    def decide(self, step, probe_score=float("inf")) -> int:
        a = ctypes.c_int32()
        _check(lib().dit_cache_ctrl_decide(ctypes.byref(self.state), step, probe_score,
                                           ctypes.byref(a)))
        return a.value

    def observe(self, output_change):
        _check(lib().dit_cache_ctrl_observe(ctypes.byref(self.state), output_change))


# ---------------------------------------------------------------------------
# MM-DiT blocks

def _ws_bytes(fn, desc) -> int:
    n = fn(ctypes.byref(desc))
    if n == 0:
        raise DitError(1, lib().dit_last_error().decode())
    return n


def dit_double_block_workspace_bytes(desc: BlockDesc) -> int:
    return _ws_bytes(lib().dit_double_block_workspace_bytes, desc)


def dit_double_block_forward(desc: BlockDesc, w_img, w_txt, mod_img, mod_txt, x_img, x_txt,
                             workspace, workspace_bytes, stream=None):
    wi = w_img if isinstance(w_img, BlockWeights) else block_weights(w_img)
    wt = w_txt if isinstance(w_txt, BlockWeights) else block_weights(w_txt)
    _check(lib().dit_double_block_forward(ctypes.byref(desc), ctypes.byref(wi), ctypes.byref(wt),
                                          _ptr(mod_img), _ptr(mod_txt), _ptr(x_img), _ptr(x_txt),
                                          _ptr(workspace), workspace_bytes, _stream(stream)))


def single_block_weights(tensors: dict) -> SingleBlockWeights:
    return SingleBlockWeights(*[_ptr(tensors[n]) for n in ("w1", "b1", "g_q", "g_k", "w2", "b2")])


def dit_single_block_workspace_bytes(desc: BlockDesc) -> int:
    return _ws_bytes(lib().dit_single_block_workspace_bytes, desc)


def dit_single_block_forward(desc: BlockDesc, weights, mod, x, workspace, workspace_bytes,
                             stream=None):
    w = weights if isinstance(weights, SingleBlockWeights) else single_block_weights(weights)
    _check(lib().dit_single_block_forward(ctypes.byref(desc), ctypes.byref(w), _ptr(mod), _ptr(x),
                                          _ptr(workspace), workspace_bytes, _stream(stream)))


# ---------------------------------------------------------------------------
# Wan-style block

def wan_block_weights(tensors: dict) -> WanBlockWeights:
    return WanBlockWeights(*[_ptr(tensors[n]) for n in WAN_WEIGHT_NAMES])


def dit_wan_block_workspace_bytes(desc: BlockDesc) -> int:
    return _ws_bytes(lib().dit_wan_block_workspace_bytes, desc)


def dit_wan_block_forward(desc: BlockDesc, weights, mod, x, ctx, workspace, workspace_bytes,
                          stream=None):
    w = weights if isinstance(weights, WanBlockWeights) else wan_block_weights(weights)
    _check(lib().dit_wan_block_forward(ctypes.byref(desc), ctypes.byref(w), _ptr(mod), _ptr(x),
                                       _ptr(ctx), _ptr(workspace), workspace_bytes, _stream(stream)))
