// C ABI of the DiT hot path: argument checks on the host, then launches.
// Every check runs before the first launch of a call, so a call that fails
// enqueues nothing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/dit.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

dit_status fail(dit_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dit_status ok() {
  g_err[0] = '\0';
  return DIT_OK;
}

dit_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DIT_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [a0, a0+an) and [b0, b0+bn) byte ranges overlap?
bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

// The attention kernel runs one 512-thread workgroup per (batch row, head,
// 256-query tile) on a 1-D grid whose size in threads must fit 32 bits.
dit_status check_attn_grid(int64_t n_q, int32_t heads, int32_t batch) {
  const int64_t n_wg = (n_q + 255) / 256 * heads * batch;
  if (n_wg * 512 > 0xffffffffLL)
    return fail(DIT_EUNSUPPORTED, "%lld attention workgroups (query tiles x heads x batch) exceed "
                "the 1-D grid limit of %lld", static_cast<long long>(n_wg), 0xffffffffLL / 512);
  return DIT_OK;
}

dit_status check_attn_desc(const dit_attn_desc* d) {
  if (!d) return fail(DIT_EINVAL, "attention descriptor is NULL");
  if (d->batch < 1 || d->batch > DIT_MAX_BATCH)
    return fail(DIT_EINVAL, "batch %d outside [1, %d]", d->batch, DIT_MAX_BATCH);
  if (d->n_vis < 0 || d->n_txt < 0)
    return fail(DIT_EINVAL, "negative token count (n_vis %d, n_txt %d)", d->n_vis, d->n_txt);
  if (static_cast<int64_t>(d->n_vis) + d->n_txt < 1 ||
      static_cast<int64_t>(d->n_vis) + d->n_txt > (1 << 30))
    return fail(DIT_EINVAL, "n_vis + n_txt = %lld outside [1, 2^30]",
                static_cast<long long>(d->n_vis) + d->n_txt);
  if (d->heads < 1 || d->heads > 65535) return fail(DIT_EINVAL, "heads %d outside [1, 65535]", d->heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(DIT_EUNSUPPORTED, "head_dim %d: only 64 and 128 are implemented", d->head_dim);
  for (int b = 0; b < d->batch; ++b) {
    if (d->txt_valid[b] < 0 || d->txt_valid[b] > d->n_txt)
      return fail(DIT_EINVAL, "txt_valid[%d] = %d outside [0, n_txt = %d]", b, d->txt_valid[b],
                  d->n_txt);
    if (d->n_vis + d->txt_valid[b] < 1)
      return fail(DIT_EINVAL, "batch row %d has no valid key (n_vis 0, txt_valid 0)", b);
  }
  return check_attn_grid(static_cast<int64_t>(d->n_vis) + d->n_txt, d->heads, d->batch);
}

dit_status check_block_desc(const dit_block_desc* d) {
  if (!d) return fail(DIT_EINVAL, "block descriptor is NULL");
  dit_status s = check_attn_desc(&d->attn);
  if (s != DIT_OK) return s;
  const dit_attn_desc& a = d->attn;
  const int64_t rows = static_cast<int64_t>(a.batch) * (static_cast<int64_t>(a.n_vis) + a.n_txt);
  if (rows > DIT_LINEAR_MAX_M)
    return fail(DIT_EUNSUPPORTED, "batch x tokens = %lld above %lld rows (the projections' limit)",
                static_cast<long long>(rows), static_cast<long long>(DIT_LINEAR_MAX_M));
  if (d->hidden != a.heads * a.head_dim)
    return fail(DIT_EINVAL, "hidden %d != heads %d * head_dim %d", d->hidden, a.heads, a.head_dim);
  if (d->hidden % 64 != 0 || d->hidden > 16384)
    return fail(DIT_EUNSUPPORTED, "hidden %d: must be a multiple of 64 and <= 16384", d->hidden);
  if (d->mlp < 64 || d->mlp % 64 != 0)
    return fail(DIT_EUNSUPPORTED, "mlp %d: must be a positive multiple of 64", d->mlp);
  if (d->grid_t < 1 || d->grid_h < 1 || d->grid_w < 1)
    return fail(DIT_EINVAL, "grid (%d, %d, %d) must be positive", d->grid_t, d->grid_h, d->grid_w);
  if (static_cast<int64_t>(d->grid_t) * d->grid_h * d->grid_w != a.n_vis)
    return fail(DIT_EINVAL, "grid %d x %d x %d != n_vis %d", d->grid_t, d->grid_h, d->grid_w,
                a.n_vis);
  if (d->rope_t < 0 || d->rope_h < 0 || d->rope_w < 0 || d->rope_t % 2 || d->rope_h % 2 ||
      d->rope_w % 2)
    return fail(DIT_EINVAL, "rope dims (%d, %d, %d) must be even and >= 0", d->rope_t, d->rope_h,
                d->rope_w);
  if (d->rope_t + d->rope_h + d->rope_w != a.head_dim)
    return fail(DIT_EINVAL, "rope dims sum %d != head_dim %d", d->rope_t + d->rope_h + d->rope_w,
                a.head_dim);
  if (!(d->rope_theta > 0.f) || !std::isfinite(d->rope_theta))
    return fail(DIT_EINVAL, "rope_theta must be finite and > 0");
  if (!(d->ln_eps >= 0.f) || !(d->rms_eps >= 0.f))
    return fail(DIT_EINVAL, "ln_eps and rms_eps must be >= 0");
  if (d->mod_stride < 0 || d->mod_stride % 4 != 0)
    return fail(DIT_EINVAL, "mod_stride %lld must be >= 0 and a multiple of 4",
                static_cast<long long>(d->mod_stride));
  return DIT_OK;
}

dit::RopeParams rope_params(const dit_block_desc* d, uint16_t* qkv, int64_t row_stride,
                            const uint16_t* gq, const uint16_t* gk) {
  dit::RopeParams p{};
  p.qkv = qkv;
  p.row_stride = row_stride;
  p.g_q = gq;
  p.g_k = gk;
  p.n_tok = d->attn.n_vis + d->attn.n_txt;
  p.rows = static_cast<int64_t>(d->attn.batch) * p.n_tok;
  p.n_vis = d->attn.n_vis;
  p.hidden = d->hidden;
  p.head_dim = d->attn.head_dim;
  p.grid_h = d->grid_h;
  p.grid_w = d->grid_w;
  p.rope_t = d->rope_t;
  p.rope_h = d->rope_h;
  p.rope_w = d->rope_w;
  p.theta = d->rope_theta;
  p.eps = d->rms_eps;
  return p;
}

// The attention kernel addresses the 64 rows of a key tile with 32-bit byte
// offsets from the tile's first row.
constexpr int64_t kMaxQkvRowStride = int64_t{1} << 24;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WsLayout {
  size_t h_off, big_off, split_off, total;
};

// Block workspace: h/o/h2, then qkv/the MLP hidden, then (for token counts
// that reach the large GEMM kernel) the scratch of its K-split last round.
WsLayout ws_layout(const dit_block_desc* d) {
  const size_t M = static_cast<size_t>(d->attn.batch) * (d->attn.n_vis + d->attn.n_txt);
  const size_t D = d->hidden, F = d->mlp;
  WsLayout w;
  w.h_off = 0;
  w.big_off = align256(M * D * 2);
  w.split_off = w.big_off + align256(M * (3 * D > F ? 3 * D : F) * 2);
  w.total = w.split_off + (M >= 1024 ? dit::kSplitWsBytes : 0);
  return w;
}

float* split_scratch(char* ws, const WsLayout& L) {
  return L.total > L.split_off ? reinterpret_cast<float*>(ws + L.split_off) : nullptr;
}

dit_status check_linear(const dit_linear_args* a) {
  if (!a) return fail(DIT_EINVAL, "linear args are NULL");
  if (a->m < 0 || a->n < 1 || a->k < 1)
    return fail(DIT_EINVAL, "bad GEMM shape m %lld n %d k %d", static_cast<long long>(a->m), a->n,
                a->k);
  if (a->m == 0) return DIT_OK;
  // One 256-row tile per grid row of the general kernel, at most 65535 of them.
  if (a->m > DIT_LINEAR_MAX_M)
    return fail(DIT_EUNSUPPORTED, "m %lld above %lld rows", static_cast<long long>(a->m),
                static_cast<long long>(DIT_LINEAR_MAX_M));
  if (!a->a || !a->w || !a->out) return fail(DIT_EINVAL, "NULL a, w or out");
  if (a->k % 64 != 0) return fail(DIT_EUNSUPPORTED, "k %d must be a multiple of 64", a->k);
  if (a->n % 8 != 0) return fail(DIT_EUNSUPPORTED, "n %d must be a multiple of 8", a->n);
  if (a->epilogue < DIT_EPI_BF16 || a->epilogue > DIT_EPI_RES_F32)
    return fail(DIT_EINVAL, "unknown epilogue %d", a->epilogue);
  if (a->lda < a->k || a->lda % 8 != 0)
    return fail(DIT_EINVAL, "lda %lld must be >= k and a multiple of 8", static_cast<long long>(a->lda));
  if (a->ldc < a->n || a->ldc % 8 != 0)
    return fail(DIT_EINVAL, "ldc %lld must be >= n and a multiple of 8", static_cast<long long>(a->ldc));
  if (a->group_rows < 0 || (a->group_rows > 0 && (a->a_group_stride < 0 || a->c_group_stride < 0 ||
                                                  a->a_group_stride % 8 || a->c_group_stride % 8)))
    return fail(DIT_EINVAL, "bad row grouping (group_rows %lld)", static_cast<long long>(a->group_rows));
  if (!aligned(a->a, 16) || !aligned(a->w, 16) || !aligned(a->out, 16) ||
      (a->bias && !aligned(a->bias, 16)))
    return fail(DIT_EINVAL, "a, w, bias and out must be 16-byte aligned");
  if (a->epilogue == DIT_EPI_GATED_RES_F32) {
    if (!a->gate || a->gate_rows < 1 || a->gate_stride < 0 || a->gate_stride % 4 != 0 ||
        !aligned(a->gate, 8))
      return fail(DIT_EINVAL, "gated epilogue needs gate (8-byte aligned), gate_rows >= 1 and a "
                              "gate_stride that is a multiple of 4");
  }
  // The output is written while other workgroups still read A, the bias and
  // the gate: it must not overlap any of them (bytes spanned, row grouping
  // and strides included).
  const int64_t span_rows = a->group_rows > 0 ? a->group_rows : a->m;
  const int64_t groups = a->group_rows > 0 ? (a->m + a->group_rows - 1) / a->group_rows : 1;
  const size_t a_bytes = static_cast<size_t>(((groups - 1) * (a->group_rows > 0 ? a->a_group_stride : 0)) +
                                             (span_rows - 1) * a->lda + a->k) * 2;
  const size_t esz = a->epilogue == DIT_EPI_F32 || a->epilogue == DIT_EPI_RES_F32 ||
                             a->epilogue == DIT_EPI_GATED_RES_F32 ? 4 : 2;
  const size_t c_bytes = static_cast<size_t>(((groups - 1) * (a->group_rows > 0 ? a->c_group_stride : 0)) +
                                             (span_rows - 1) * a->ldc + a->n) * esz;
  if (overlap(a->a, a_bytes, a->out, c_bytes))
    return fail(DIT_EINVAL, "out overlaps the A operand");
  if (a->bias && overlap(a->bias, static_cast<size_t>(a->n) * 2, a->out, c_bytes))
    return fail(DIT_EINVAL, "out overlaps the bias");
  size_t gate_bytes = 0;
  if (a->epilogue == DIT_EPI_GATED_RES_F32) {
    gate_bytes = static_cast<size_t>(((a->m - 1) / a->gate_rows) * a->gate_stride + a->n) * 2;
    if (overlap(a->gate, gate_bytes, a->out, c_bytes))
      return fail(DIT_EINVAL, "out overlaps the gate rows");
  }
  if (a->workspace) {
    if (!aligned(a->workspace, 256)) return fail(DIT_EINVAL, "workspace not 256-byte aligned");
    if (a->workspace_bytes < dit::kSplitWsBytes)
      return fail(DIT_EWORKSPACE, "workspace %zu bytes < %zu needed", a->workspace_bytes, dit::kSplitWsBytes);
    const size_t wb = dit::kSplitWsBytes;
    if (overlap(a->workspace, wb, a->a, a_bytes) || overlap(a->workspace, wb, a->out, c_bytes) ||
        overlap(a->workspace, wb, a->w, static_cast<size_t>(a->n) * a->k * 2) ||
        (a->bias && overlap(a->workspace, wb, a->bias, static_cast<size_t>(a->n) * 2)) ||
        (gate_bytes && overlap(a->workspace, wb, a->gate, gate_bytes)))
      return fail(DIT_EINVAL, "workspace overlaps an operand or the output");
  }
  return DIT_OK;
}

dit::GemmParams gemm_params(const dit_linear_args* a) {
  dit::GemmParams p{};
  p.a = a->a;
  p.lda = a->lda;
  p.w = a->w;
  p.bias = a->bias;
  p.m = a->m;
  p.n = a->n;
  p.k = a->k;
  p.out = a->out;
  p.ldc = a->ldc;
  p.gate = a->gate;
  p.gate_stride = a->gate_stride;
  p.gate_rows = a->gate_rows > 0 ? a->gate_rows : 1;
  p.group_rows = a->group_rows;
  p.a_group_stride = a->a_group_stride;
  p.c_group_stride = a->c_group_stride;
  p.split_ws = static_cast<float*>(a->workspace);
  return p;
}

// The eight launches of one block (argument checks already done).  hbuf holds
// h, then o, then h2; big holds qkv, then the MLP hidden.
hipError_t block_launch(const dit_block_desc* desc, const dit_block_weights* w, const uint16_t* mod,
                        int64_t ms, float* x, char* ws, hipStream_t stream, const char** what) {
  const int B = desc->attn.batch;
  const int64_t N = static_cast<int64_t>(desc->attn.n_vis) + desc->attn.n_txt;
  const int64_t M = B * N;
  const int D = desc->hidden, F = desc->mlp;
  const WsLayout L = ws_layout(desc);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(ws + L.h_off);   // h, then o, then h2
  uint16_t* big = reinterpret_cast<uint16_t*>(ws + L.big_off);  // qkv, then the MLP hidden
  float* split = split_scratch(ws, L);

  hipError_t e;
  // 1. h = adaLN(x; shift1, scale1)
  e = dit::launch_adaln(x, M, D, N, mod + 0 * D, mod + 1 * D, ms, desc->ln_eps, hbuf, stream);
  if (e != hipSuccess) { *what = "block: adaln 1"; return e; }
  // 2. qkv = h W_qkv^T + b_qkv
  dit::GemmParams g{};
  g.a = hbuf; g.lda = D; g.w = w->w_qkv; g.bias = w->b_qkv; g.m = M; g.n = 3 * D; g.k = D;
  g.out = big; g.ldc = 3 * D; g.gate_rows = 1; g.split_ws = split;
  e = dit::launch_gemm(g, DIT_EPI_BF16, stream);
  if (e != hipSuccess) { *what = "block: qkv gemm"; return e; }
  // 3. q, k <- RoPE(RMSNorm(.) * g)
  e = dit::launch_qk_rmsnorm_rope(rope_params(desc, big, 3 * D, w->g_q, w->g_k), stream);
  if (e != hipSuccess) { *what = "block: rmsnorm/rope"; return e; }
  // 4. o = joint attention
  dit::AttnParams ap{};
  ap.q = big; ap.k = big + D; ap.v = big + 2 * D;
  ap.q_stride = ap.kv_stride = 3 * D;
  ap.q_batch = ap.kv_batch = N * 3 * D;
  ap.out = hbuf; ap.out_stride = D; ap.out_f32 = 0; ap.lse = nullptr;
  ap.n_q = ap.n_k = static_cast<int>(N); ap.heads = desc->attn.heads; ap.head_dim = desc->attn.head_dim;
  ap.batch = B;
  for (int b = 0; b < DIT_MAX_BATCH; ++b)
    ap.n_valid[b] = b < B ? desc->attn.n_vis + desc->attn.txt_valid[b] : 0;
  ap.scale_log2 = 1.4426950408889634f / std::sqrt(static_cast<float>(desc->attn.head_dim));
  ap.tail_ws = split;
  e = dit::launch_attention(ap, stream);
  if (e != hipSuccess) { *what = "block: attention"; return e; }
  // 5. x += gate1 * (o W_o^T + b_o)
  g = dit::GemmParams{};
  g.a = hbuf; g.lda = D; g.w = w->w_o; g.bias = w->b_o; g.m = M; g.n = D; g.k = D;
  g.out = x; g.ldc = D; g.gate = mod + 2 * D; g.gate_stride = ms; g.gate_rows = N; g.split_ws = split;
  e = dit::launch_gemm(g, DIT_EPI_GATED_RES_F32, stream);
  if (e != hipSuccess) { *what = "block: out-proj gemm"; return e; }
  // 6. h2 = adaLN(x; shift2, scale2)
  e = dit::launch_adaln(x, M, D, N, mod + 3 * D, mod + 4 * D, ms, desc->ln_eps, hbuf, stream);
  if (e != hipSuccess) { *what = "block: adaln 2"; return e; }
  // 7. u = GELU(h2 W_up^T + b_up)
  g = dit::GemmParams{};
  g.a = hbuf; g.lda = D; g.w = w->w_up; g.bias = w->b_up; g.m = M; g.n = F; g.k = D;
  g.out = big; g.ldc = F; g.gate_rows = 1; g.split_ws = split;
  e = dit::launch_gemm(g, DIT_EPI_GELU_BF16, stream);
  if (e != hipSuccess) { *what = "block: mlp-up gemm"; return e; }
  // 8. x += gate2 * (u W_dn^T + b_dn)
  g = dit::GemmParams{};
  g.a = big; g.lda = F; g.w = w->w_dn; g.bias = w->b_dn; g.m = M; g.n = D; g.k = F;
  g.out = x; g.ldc = D; g.gate = mod + 5 * D; g.gate_stride = ms; g.gate_rows = N; g.split_ws = split;
  e = dit::launch_gemm(g, DIT_EPI_GATED_RES_F32, stream);
  if (e != hipSuccess) { *what = "block: mlp-down gemm"; return e; }
  return hipSuccess;
}


// Workspace of one denoising step: small conditioning buffers, the fp32
// residual stream x, the final-norm output, the velocity and the block's own
// workspace.
struct StepLayout {
  size_t feat, c, s, mod, fin, lat, x, hf, v, part, blk, total;
};

StepLayout step_layout(const dit_model_desc* m) {
  const dit_block_desc& b = m->block;
  const size_t B = b.attn.batch, N = static_cast<size_t>(b.attn.n_vis) + b.attn.n_txt;
  const size_t D = b.hidden, C = m->latent_channels, nv = b.attn.n_vis;
  const size_t Bl = m->cfg ? 1 : B;
  StepLayout L;
  size_t o = 0;
  L.feat = o; o += align256(static_cast<size_t>(m->freq_dim) * 2);
  L.c = o; o += align256(D * 2);
  L.s = o; o += align256(D * 2);
  L.mod = o; o += align256(static_cast<size_t>(m->depth) * 6 * D * 2);  // every layer's modulation
  L.fin = o; o += align256(2 * D * 2);
  L.lat = o; o += align256(Bl * nv * C * 2);
  L.x = o; o += align256(B * N * D * 4);
  L.hf = o; o += align256(B * N * D * 2);
  L.v = o; o += align256(B * nv * C * 2);
  L.part = o; o += align256(dit::kScorePartialBytes);
  L.blk = o; o += ws_layout(&b).total;
  L.total = o;
  return L;
}

dit_status check_model_desc(const dit_model_desc* m) {
  if (!m) return fail(DIT_EINVAL, "model descriptor is NULL");
  dit_block_desc b = m->block;
  b.mod_stride = 0;
  dit_status s = check_block_desc(&b);
  if (s != DIT_OK) return s;
  if (m->depth < 1 || m->depth > 4096) return fail(DIT_EINVAL, "depth %d outside [1, 4096]", m->depth);
  if (m->latent_channels < 64 || m->latent_channels % 64 != 0)
    return fail(DIT_EUNSUPPORTED, "latent_channels %d must be a positive multiple of 64",
                m->latent_channels);
  if (m->freq_dim < 64 || m->freq_dim % 64 != 0 || m->freq_dim > 4096)
    return fail(DIT_EUNSUPPORTED, "freq_dim %d must be a multiple of 64 in [64, 4096]", m->freq_dim);
  if (m->cfg != 0 && m->cfg != 1) return fail(DIT_EINVAL, "cfg must be 0 or 1");
  if (m->cfg && b.attn.batch != 2) return fail(DIT_EINVAL, "cfg needs batch == 2 (cond, uncond)");
  if (b.attn.n_vis < 1) return fail(DIT_EINVAL, "a denoising step needs visual tokens");
  if (!std::isfinite(m->t_scale)) return fail(DIT_EINVAL, "t_scale must be finite");
  return DIT_OK;
}

dit_status check_block_weights(const dit_block_weights* w) {
  if (!w) return fail(DIT_EINVAL, "block weights are NULL");
  const uint16_t* ptrs[] = {w->w_qkv, w->b_qkv, w->g_q, w->g_k, w->w_o,
                            w->b_o,   w->w_up,  w->b_up, w->w_dn, w->b_dn};
  for (const uint16_t* p : ptrs)
    if (!p || !aligned(p, 16)) return fail(DIT_EINVAL, "a weight pointer is NULL or not 16-byte aligned");
  return DIT_OK;
}

dit::GemmParams gemm(const uint16_t* a, int64_t lda, const uint16_t* w, const uint16_t* bias, int64_t m,
                     int n, int k, void* out, int64_t ldc, float* split = nullptr) {
  dit::GemmParams g{};
  g.a = a; g.lda = lda; g.w = w; g.bias = bias; g.m = m; g.n = n; g.k = k;
  g.out = out; g.ldc = ldc; g.gate_rows = 1; g.split_ws = split;
  return g;
}

}  // namespace

extern "C" {

const char* dit_version(void) { return "dit-mi355x 0.1 (gfx950)"; }

const char* dit_last_error(void) { return g_err; }

const char* dit_status_string(dit_status s) {
  switch (s) {
    case DIT_OK: return "DIT_OK";
    case DIT_EINVAL: return "DIT_EINVAL";
    case DIT_EUNSUPPORTED: return "DIT_EUNSUPPORTED";
    case DIT_EWORKSPACE: return "DIT_EWORKSPACE";
    case DIT_EHIP: return "DIT_EHIP";
  }
  return "unknown dit_status";
}

size_t dit_joint_attention_workspace_bytes(void) { return dit::kAttnTailWsBytes; }

dit_status dit_joint_attention(const dit_attn_desc* desc, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, int64_t qkv_row_stride, uint16_t* out,
                               int64_t out_row_stride, float* lse, float softmax_scale,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dit_status s = check_attn_desc(desc);
  if (s != DIT_OK) return s;
  if (!q || !k || !v || !out) return fail(DIT_EINVAL, "NULL q, k, v or out");
  const int64_t hd = static_cast<int64_t>(desc->heads) * desc->head_dim;
  if (qkv_row_stride < hd || qkv_row_stride % 8 != 0)
    return fail(DIT_EINVAL, "qkv_row_stride %lld must be >= heads*head_dim and a multiple of 8",
                static_cast<long long>(qkv_row_stride));
  if (qkv_row_stride > kMaxQkvRowStride)
    return fail(DIT_EUNSUPPORTED, "qkv_row_stride %lld above %lld (key tiles are addressed with "
                "32-bit byte offsets)", static_cast<long long>(qkv_row_stride),
                static_cast<long long>(kMaxQkvRowStride));
  if (out_row_stride < hd || out_row_stride % 8 != 0)
    return fail(DIT_EINVAL, "out_row_stride %lld must be >= heads*head_dim and a multiple of 8",
                static_cast<long long>(out_row_stride));
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      (lse && !aligned(lse, 4)))
    return fail(DIT_EINVAL, "q, k, v and out must be 16-byte aligned");
  if (!(softmax_scale >= 0.f) || !std::isfinite(softmax_scale))
    return fail(DIT_EINVAL, "softmax_scale must be finite and >= 0");
  const int64_t n_tok = static_cast<int64_t>(desc->n_vis) + desc->n_txt;
  const size_t in_bytes = static_cast<size_t>((desc->batch * n_tok - 1) * qkv_row_stride + hd) * 2;
  const size_t out_bytes = static_cast<size_t>((desc->batch * n_tok - 1) * out_row_stride + hd) * 2;
  if (overlap(out, out_bytes, q, in_bytes) || overlap(out, out_bytes, k, in_bytes) ||
      overlap(out, out_bytes, v, in_bytes))
    return fail(DIT_EINVAL, "out overlaps q, k or v");
  const size_t lse_bytes = lse ? static_cast<size_t>(desc->batch) * desc->heads * n_tok * 4 : 0;
  if (lse) {
    if (overlap(lse, lse_bytes, out, out_bytes) || overlap(lse, lse_bytes, q, in_bytes) ||
        overlap(lse, lse_bytes, k, in_bytes) || overlap(lse, lse_bytes, v, in_bytes))
      return fail(DIT_EINVAL, "lse overlaps q, k, v or out");
  }
  if (workspace) {
    if (!aligned(workspace, 256)) return fail(DIT_EINVAL, "workspace not 256-byte aligned");
    if (workspace_bytes < dit::kAttnTailWsBytes)
      return fail(DIT_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, dit::kAttnTailWsBytes);
    const size_t wb = dit::kAttnTailWsBytes;
    if (overlap(workspace, wb, q, in_bytes) || overlap(workspace, wb, k, in_bytes) ||
        overlap(workspace, wb, v, in_bytes) || overlap(workspace, wb, out, out_bytes) ||
        (lse && overlap(workspace, wb, lse, lse_bytes)))
      return fail(DIT_EINVAL, "workspace overlaps q, k, v, out or lse");
  }
  dit::AttnParams p{};
  p.tail_ws = static_cast<float*>(workspace);
  p.q = q;
  p.k = k;
  p.v = v;
  p.q_stride = p.kv_stride = qkv_row_stride;
  p.q_batch = p.kv_batch = n_tok * qkv_row_stride;
  p.out = out;
  p.out_stride = out_row_stride;
  p.lse = lse;
  p.n_q = p.n_k = static_cast<int>(n_tok);
  p.out_f32 = 0;
  p.heads = desc->heads;
  p.head_dim = desc->head_dim;
  p.batch = desc->batch;
  for (int b = 0; b < DIT_MAX_BATCH; ++b)
    p.n_valid[b] = b < desc->batch ? desc->n_vis + desc->txt_valid[b] : 0;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / std::sqrt(static_cast<float>(desc->head_dim));
  p.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(dit::launch_attention(p, stream), "attention launch");
}

dit_status dit_attention_partial(const dit_partial_desc* desc, const uint16_t* q,
                                 int64_t q_row_stride, const uint16_t* k, const uint16_t* v,
                                 int64_t kv_row_stride, float* out, int64_t out_row_stride,
                                 float* lse, float softmax_scale, hipStream_t stream) {
  if (!desc) return fail(DIT_EINVAL, "partial-attention descriptor is NULL");
  const dit_partial_desc& d = *desc;
  if (d.batch < 1 || d.batch > DIT_MAX_BATCH)
    return fail(DIT_EINVAL, "batch %d outside [1, %d]", d.batch, DIT_MAX_BATCH);
  if (d.n_q < 1 || d.n_k < 1 || d.n_q > (1 << 30) || d.n_k > (1 << 30))
    return fail(DIT_EINVAL, "n_q %d and n_k %d must be in [1, 2^30]", d.n_q, d.n_k);
  if (d.heads < 1 || d.heads > 65535) return fail(DIT_EINVAL, "heads %d outside [1, 65535]", d.heads);
  if (d.head_dim != 64 && d.head_dim != 128)
    return fail(DIT_EUNSUPPORTED, "head_dim %d: only 64 and 128 are implemented", d.head_dim);
  for (int b = 0; b < d.batch; ++b)
    if (d.k_valid[b] < 0 || d.k_valid[b] > d.n_k)
      return fail(DIT_EINVAL, "k_valid[%d] = %d outside [0, n_k = %d]", b, d.k_valid[b], d.n_k);
  if (dit_status st = check_attn_grid(d.n_q, d.heads, d.batch)) return st;
  if (!q || !k || !v || !out || !lse) return fail(DIT_EINVAL, "NULL q, k, v, out or lse");
  const int64_t hd = static_cast<int64_t>(d.heads) * d.head_dim;
  if (q_row_stride < hd || q_row_stride % 8 != 0 || kv_row_stride < hd || kv_row_stride % 8 != 0)
    return fail(DIT_EINVAL, "q/kv row strides must be >= heads*head_dim and multiples of 8");
  if (kv_row_stride > kMaxQkvRowStride)
    return fail(DIT_EUNSUPPORTED, "kv_row_stride %lld above %lld",
                static_cast<long long>(kv_row_stride), static_cast<long long>(kMaxQkvRowStride));
  if (out_row_stride < hd || out_row_stride % 4 != 0)
    return fail(DIT_EINVAL, "out_row_stride %lld must be >= heads*head_dim and a multiple of 4",
                static_cast<long long>(out_row_stride));
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return fail(DIT_EINVAL, "q, k, v and out must be 16-byte aligned, lse 4-byte");
  if (!(softmax_scale >= 0.f) || !std::isfinite(softmax_scale))
    return fail(DIT_EINVAL, "softmax_scale must be finite and >= 0");
  const size_t q_bytes = static_cast<size_t>((static_cast<int64_t>(d.batch) * d.n_q - 1) * q_row_stride + hd) * 2;
  const size_t kv_bytes = static_cast<size_t>((static_cast<int64_t>(d.batch) * d.n_k - 1) * kv_row_stride + hd) * 2;
  const size_t out_bytes = static_cast<size_t>((static_cast<int64_t>(d.batch) * d.n_q - 1) * out_row_stride + hd) * 4;
  const size_t lse_bytes = static_cast<size_t>(d.batch) * d.heads * d.n_q * 4;
  if (overlap(out, out_bytes, q, q_bytes) || overlap(out, out_bytes, k, kv_bytes) ||
      overlap(out, out_bytes, v, kv_bytes) || overlap(lse, lse_bytes, q, q_bytes) ||
      overlap(lse, lse_bytes, k, kv_bytes) || overlap(lse, lse_bytes, v, kv_bytes) ||
      overlap(lse, lse_bytes, out, out_bytes))
    return fail(DIT_EINVAL, "out or lse overlaps an input or each other");
  dit::AttnParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.q_stride = q_row_stride;
  p.kv_stride = kv_row_stride;
  p.q_batch = static_cast<int64_t>(d.n_q) * q_row_stride;
  p.kv_batch = static_cast<int64_t>(d.n_k) * kv_row_stride;
  p.out = out;
  p.out_stride = out_row_stride;
  p.out_f32 = 1;
  p.lse = lse;
  p.n_q = d.n_q;
  p.n_k = d.n_k;
  p.heads = d.heads;
  p.head_dim = d.head_dim;
  p.batch = d.batch;
  for (int b = 0; b < DIT_MAX_BATCH; ++b) p.n_valid[b] = b < d.batch ? d.k_valid[b] : 0;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.f / std::sqrt(static_cast<float>(d.head_dim));
  p.scale_log2 = scale * 1.4426950408889634f;
  return hip_status(dit::launch_attention(p, stream), "partial attention launch");
}

dit_status dit_attention_merge(const dit_merge_desc* desc, const float* const* outs,
                               int64_t part_row_stride, const float* const* lses, uint16_t* out,
                               int64_t out_row_stride, float* lse_out, hipStream_t stream) {
  if (!desc) return fail(DIT_EINVAL, "merge descriptor is NULL");
  const dit_merge_desc& d = *desc;
  if (d.parts < 1 || d.parts > DIT_MAX_PARTS)
    return fail(DIT_EINVAL, "parts %d outside [1, %d]", d.parts, DIT_MAX_PARTS);
  if (d.batch < 1 || d.batch > DIT_MAX_BATCH || d.n_q < 1 || d.heads < 1 || d.heads > 65535)
    return fail(DIT_EINVAL, "bad merge shape (batch %d, n_q %d, heads %d)", d.batch, d.n_q, d.heads);
  if (d.head_dim != 64 && d.head_dim != 128)
    return fail(DIT_EUNSUPPORTED, "head_dim %d: only 64 and 128 are implemented", d.head_dim);
  if (!outs || !lses || !out) return fail(DIT_EINVAL, "NULL outs, lses or out");
  const int64_t hd = static_cast<int64_t>(d.heads) * d.head_dim;
  if (part_row_stride < hd || part_row_stride % 4 != 0 || out_row_stride < hd || out_row_stride % 8 != 0)
    return fail(DIT_EINVAL, "part_row_stride (multiple of 4) and out_row_stride (multiple of 8) "
                            "must be >= heads*head_dim");
  const int64_t rows = static_cast<int64_t>(d.batch) * d.n_q;
  const size_t part_bytes = static_cast<size_t>((rows - 1) * part_row_stride + hd) * 4;
  const size_t lse_bytes = static_cast<size_t>(d.batch) * d.heads * d.n_q * 4;
  const size_t out_bytes = static_cast<size_t>((rows - 1) * out_row_stride + hd) * 2;
  if (!aligned(out, 16) || (lse_out && !aligned(lse_out, 4)))
    return fail(DIT_EINVAL, "out must be 16-byte aligned, lse_out 4-byte");
  dit::MergeParams p{};
  for (int i = 0; i < d.parts; ++i) {
    if (!outs[i] || !lses[i]) return fail(DIT_EINVAL, "NULL partial %d", i);
    if (!aligned(outs[i], 16) || !aligned(lses[i], 4))
      return fail(DIT_EINVAL, "partial %d: out must be 16-byte aligned, lse 4-byte", i);
    if (overlap(out, out_bytes, outs[i], part_bytes) || overlap(out, out_bytes, lses[i], lse_bytes) ||
        (lse_out && (overlap(lse_out, lse_bytes, outs[i], part_bytes) ||
                     overlap(lse_out, lse_bytes, lses[i], lse_bytes))))
      return fail(DIT_EINVAL, "an output overlaps partial %d", i);
    p.outs[i] = outs[i];
    p.lses[i] = lses[i];
  }
  if (lse_out && overlap(lse_out, lse_bytes, out, out_bytes))
    return fail(DIT_EINVAL, "lse_out overlaps out");
  p.parts = d.parts;
  p.part_stride = part_row_stride;
  p.out = out;
  p.out_stride = out_row_stride;
  p.lse_out = lse_out;
  p.batch = d.batch;
  p.n_q = d.n_q;
  p.heads = d.heads;
  p.head_dim = d.head_dim;
  return hip_status(dit::launch_attention_merge(p, stream), "attention merge launch");
}

size_t dit_linear_workspace_bytes(void) { return dit::kSplitWsBytes; }

dit_status dit_linear(const dit_linear_args* args, hipStream_t stream) {
  dit_status s = check_linear(args);
  if (s != DIT_OK) return s;
  if (args->m == 0) return ok();
  return hip_status(dit::launch_gemm(gemm_params(args), args->epilogue, stream), "gemm launch");
}

dit_status dit_adaln_modulate(const float* x, int64_t rows, int32_t hidden, int64_t rows_per_batch,
                              const uint16_t* shift, const uint16_t* scale, int64_t mod_stride,
                              float eps, uint16_t* out, hipStream_t stream) {
  if (rows < 0) return fail(DIT_EINVAL, "rows %lld < 0", static_cast<long long>(rows));
  if (rows == 0) return ok();
  if (!x || !out) return fail(DIT_EINVAL, "NULL x or out");
  if ((shift == nullptr) != (scale == nullptr))
    return fail(DIT_EINVAL, "shift and scale must both be given or both be NULL");
  if (hidden < 8 || hidden % 8 != 0 || hidden > 16384)
    return fail(DIT_EUNSUPPORTED, "hidden %d must be a multiple of 8 in [8, 16384]", hidden);
  if (rows_per_batch < 1) return fail(DIT_EINVAL, "rows_per_batch must be >= 1");
  if (mod_stride < 0 || mod_stride % 4 != 0)
    return fail(DIT_EINVAL, "mod_stride must be >= 0 and a multiple of 4");
  if (!(eps >= 0.f)) return fail(DIT_EINVAL, "eps must be >= 0");
  if (!aligned(x, 16) || !aligned(out, 8) || (shift && (!aligned(shift, 8) || !aligned(scale, 8))))
    return fail(DIT_EINVAL, "x must be 16-byte aligned; out, shift, scale 8-byte aligned");
  if (overlap(x, static_cast<size_t>(rows) * hidden * 4, out, static_cast<size_t>(rows) * hidden * 2))
    return fail(DIT_EINVAL, "out overlaps x");
  return hip_status(dit::launch_adaln(x, rows, hidden, rows_per_batch, shift, scale, mod_stride, eps,
                                      out, stream),
                    "adaln launch");
}

dit_status dit_qk_rmsnorm_rope(const dit_block_desc* desc, uint16_t* qkv, int64_t row_stride,
                               const uint16_t* g_q, const uint16_t* g_k, hipStream_t stream) {
  dit_status s = check_block_desc(desc);
  if (s != DIT_OK) return s;
  if (!qkv || !g_q || !g_k) return fail(DIT_EINVAL, "NULL qkv, g_q or g_k");
  if (row_stride < 2 * static_cast<int64_t>(desc->hidden) || row_stride % 8 != 0)
    return fail(DIT_EINVAL, "row_stride must be >= 2*hidden and a multiple of 8");
  if (!aligned(qkv, 16) || !aligned(g_q, 16) || !aligned(g_k, 16))
    return fail(DIT_EINVAL, "qkv, g_q and g_k must be 16-byte aligned");
  return hip_status(dit::launch_qk_rmsnorm_rope(rope_params(desc, qkv, row_stride, g_q, g_k), stream),
                    "rmsnorm/rope launch");
}

dit_status dit_debug_positions(const dit_block_desc* desc, int32_t* out, hipStream_t stream) {
  dit_status s = check_block_desc(desc);
  if (s != DIT_OK) return s;
  if (!out) return fail(DIT_EINVAL, "NULL out");
  return hip_status(dit::launch_positions(rope_params(desc, nullptr, 0, nullptr, nullptr), out, stream),
                    "positions launch");
}

size_t dit_block_workspace_bytes(const dit_block_desc* desc) {
  if (check_block_desc(desc) != DIT_OK) return 0;
  ok();
  return ws_layout(desc).total;
}

dit_status dit_block_forward(const dit_block_desc* desc, const dit_block_weights* w,
                             const uint16_t* mod, float* x, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  dit_status s = check_block_desc(desc);
  if (s != DIT_OK) return s;
  if (!w) return fail(DIT_EINVAL, "weights struct is NULL");
  const uint16_t* ptrs[] = {w->w_qkv, w->b_qkv, w->g_q, w->g_k, w->w_o,
                            w->b_o,   w->w_up,  w->b_up, w->w_dn, w->b_dn};
  for (const uint16_t* p : ptrs)
    if (!p || !aligned(p, 16)) return fail(DIT_EINVAL, "a weight pointer is NULL or not 16-byte aligned");
  if (!mod || !aligned(mod, 16)) return fail(DIT_EINVAL, "mod is NULL or not 16-byte aligned");
  if (!x || !aligned(x, 16)) return fail(DIT_EINVAL, "x is NULL or not 16-byte aligned");
  if (!workspace || !aligned(workspace, 256)) return fail(DIT_EINVAL, "workspace is NULL or not 256-byte aligned");
  const WsLayout L = ws_layout(desc);
  if (workspace_bytes < L.total)
    return fail(DIT_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, L.total);
  const int64_t M = static_cast<int64_t>(desc->attn.batch) * (desc->attn.n_vis + desc->attn.n_txt);
  if (overlap(x, static_cast<size_t>(M) * desc->hidden * 4, workspace, L.total))
    return fail(DIT_EINVAL, "x overlaps the workspace");
  const char* what = nullptr;
  const hipError_t e = block_launch(desc, w, mod, desc->mod_stride, x, static_cast<char*>(workspace),
                                    stream, &what);
  if (e != hipSuccess) return hip_status(e, what);
  return ok();
}

dit_status dit_euler_step(float* x, const uint16_t* v_cond, const uint16_t* v_uncond, int64_t n,
                          float guidance, float sigma, float sigma_next, hipStream_t stream) {
  if (n < 0) return fail(DIT_EINVAL, "n %lld < 0", static_cast<long long>(n));
  if (n == 0) return ok();
  if (!x || !v_cond) return fail(DIT_EINVAL, "NULL x or v_cond");
  if (!aligned(x, 16) || !aligned(v_cond, 8) || (v_uncond && !aligned(v_uncond, 8)))
    return fail(DIT_EINVAL, "x must be 16-byte aligned, v_cond/v_uncond 8-byte aligned");
  if (!std::isfinite(guidance) || !std::isfinite(sigma) || !std::isfinite(sigma_next))
    return fail(DIT_EINVAL, "guidance and sigmas must be finite");
  if (overlap(x, static_cast<size_t>(n) * 4, v_cond, static_cast<size_t>(n) * 2) ||
      (v_uncond && overlap(x, static_cast<size_t>(n) * 4, v_uncond, static_cast<size_t>(n) * 2)))
    return fail(DIT_EINVAL, "x overlaps a velocity buffer");
  return hip_status(dit::launch_euler(x, v_cond, v_uncond, n, guidance, sigma_next - sigma, stream),
                    "euler launch");
}

dit_status dit_timestep_features(const float* sigma, int32_t n, int32_t dim, float t_scale,
                                 uint16_t* out, hipStream_t stream) {
  if (n < 0) return fail(DIT_EINVAL, "n < 0");
  if (n == 0) return ok();
  if (!sigma || !out) return fail(DIT_EINVAL, "NULL sigma or out");
  if (dim < 2 || dim > 4096 || dim % 2) return fail(DIT_EINVAL, "dim %d must be even in [2, 4096]", dim);
  if (!std::isfinite(t_scale)) return fail(DIT_EINVAL, "t_scale must be finite");
  return hip_status(dit::launch_timestep_features(sigma, 0.f, n, dim, t_scale, out, stream),
                    "timestep launch");
}

dit_status dit_cast_f32_bf16(const float* in, int64_t ld_in, int64_t rows, int32_t cols,
                             uint16_t* out, int64_t ld_out, hipStream_t stream) {
  if (rows < 0 || cols < 0) return fail(DIT_EINVAL, "negative rows/cols");
  if (rows == 0 || cols == 0) return ok();
  if (!in || !out) return fail(DIT_EINVAL, "NULL in or out");
  if (cols % 4 || ld_in % 4 || ld_out % 4 || ld_in < cols || ld_out < cols)
    return fail(DIT_EINVAL, "cols and strides must be multiples of 4, strides >= cols");
  if (!aligned(in, 16) || !aligned(out, 8)) return fail(DIT_EINVAL, "in 16-byte, out 8-byte alignment");
  return hip_status(dit::launch_cast_f32_bf16(in, ld_in, rows, cols, out, ld_out, stream), "cast launch");
}

dit_status dit_cast_bf16_f32(const uint16_t* in, int64_t ld_in, int64_t rows, int32_t cols,
                             float* out, int64_t ld_out, hipStream_t stream) {
  if (rows < 0 || cols < 0) return fail(DIT_EINVAL, "negative rows/cols");
  if (rows == 0 || cols == 0) return ok();
  if (!in || !out) return fail(DIT_EINVAL, "NULL in or out");
  if (cols % 4 || ld_in % 4 || ld_out % 4 || ld_in < cols || ld_out < cols)
    return fail(DIT_EINVAL, "cols and strides must be multiples of 4, strides >= cols");
  if (!aligned(in, 8) || !aligned(out, 16)) return fail(DIT_EINVAL, "in 8-byte, out 16-byte alignment");
  return hip_status(dit::launch_cast_bf16_f32(in, ld_in, rows, cols, out, ld_out, stream), "cast launch");
}

// ---------------------------------------------------------------------------
// MM-DiT blocks ("ChunkFlow", Appendix B: double-stream and single-stream
// blocks).  Both are compositions of the DiT block's kernels; only the
// operand routing differs.

size_t dit_double_block_workspace_bytes(const dit_block_desc* desc) {
  if (check_block_desc(desc) != DIT_OK) return 0;
  ok();
  return ws_layout(desc).total;
}

dit_status dit_double_block_forward(const dit_block_desc* desc, const dit_block_weights* w_img,
                                    const dit_block_weights* w_txt, const uint16_t* mod_img,
                                    const uint16_t* mod_txt, float* x_img, float* x_txt,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dit_status st = check_block_desc(desc);
  if (st != DIT_OK) return st;
  if ((st = check_block_weights(w_img)) != DIT_OK) return st;
  if ((st = check_block_weights(w_txt)) != DIT_OK) return st;
  const int B = desc->attn.batch, S = desc->attn.n_vis, L = desc->attn.n_txt;
  const int D = desc->hidden, F = desc->mlp;
  const int64_t N = static_cast<int64_t>(S) + L;
  if (!mod_img || !aligned(mod_img, 16) || !mod_txt || !aligned(mod_txt, 16))
    return fail(DIT_EINVAL, "mod_img and mod_txt must be non-NULL and 16-byte aligned");
  if (!x_img || !aligned(x_img, 16) || (L > 0 && (!x_txt || !aligned(x_txt, 16))))
    return fail(DIT_EINVAL, "x_img and x_txt must be non-NULL and 16-byte aligned");
  if (!workspace || !aligned(workspace, 256)) return fail(DIT_EINVAL, "workspace is NULL or not 256-byte aligned");
  const WsLayout WL = ws_layout(desc);
  if (workspace_bytes < WL.total)
    return fail(DIT_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, WL.total);
  const size_t xi_bytes = static_cast<size_t>(B) * S * D * 4, xt_bytes = static_cast<size_t>(B) * L * D * 4;
  if (overlap(x_img, xi_bytes, workspace, WL.total) ||
      (L > 0 && (overlap(x_txt, xt_bytes, workspace, WL.total) || overlap(x_img, xi_bytes, x_txt, xt_bytes))))
    return fail(DIT_EINVAL, "x_img, x_txt and the workspace must not overlap");
  const int64_t ms = desc->mod_stride;
  char* ws = static_cast<char*>(workspace);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(ws + WL.h_off);   // h per stream, o (joint), h2 per stream
  uint16_t* big = reinterpret_cast<uint16_t*>(ws + WL.big_off);  // qkv (joint), MLP hidden per stream
  float* split = split_scratch(ws, WL);
  uint16_t* h_txt = hbuf + static_cast<int64_t>(B) * S * D;
  uint16_t* u_txt = big + static_cast<int64_t>(B) * S * F;
  struct Stream {
    const dit_block_weights* w;
    const uint16_t* mod;
    float* x;
    int rows;            // tokens of this stream per batch row
    int64_t first;       // its first token in the joint sequence
    uint16_t* h;         // its adaLN outputs, contiguous [B * rows, D]
    uint16_t* u;         // its MLP hidden, contiguous [B * rows, F]
  } streams[2] = {{w_img, mod_img, x_img, S, 0, hbuf, big},
                  {w_txt, mod_txt, x_txt, L, S, h_txt, u_txt}};
#define DIT_TRY(expr, what)                            \
  do {                                                 \
    const hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_status(e_, what); \
  } while (0)
  // per stream: h = adaLN(x; shift1, scale1); its q|k|v rows into the joint qkv buffer
  for (const Stream& t : streams) {
    if (t.rows == 0) continue;
    const int64_t M = static_cast<int64_t>(B) * t.rows;
    DIT_TRY(dit::launch_adaln(t.x, M, D, t.rows, t.mod, t.mod + D, ms, desc->ln_eps, t.h, stream),
            "double block: adaln 1");
    dit::GemmParams g = gemm(t.h, D, t.w->w_qkv, t.w->b_qkv, M, 3 * D, D, big + t.first * 3 * D, 3 * D);
    g.group_rows = t.rows;
    g.a_group_stride = static_cast<int64_t>(t.rows) * D;
    g.c_group_stride = N * 3 * D;
    g.split_ws = split;
    DIT_TRY(dit::launch_gemm(g, DIT_EPI_BF16, stream), "double block: qkv gemm");
  }
  // Q/K RMSNorm with each stream's gains + RoPE (image rows at their grid
  // position, text rows at 0), one launch per batch row and stream
  for (int b = 0; b < B; ++b)
    for (int si = 0; si < 2; ++si) {
      const Stream& t = streams[si];
      if (t.rows == 0) continue;
      dit::RopeParams rp = rope_params(desc, big + (b * N + t.first) * 3 * D, 3 * D, t.w->g_q, t.w->g_k);
      rp.rows = t.rows;
      if (si == 1) {  // text rows: token index i < n_tok = L, none visual
        rp.n_tok = L;
        rp.n_vis = 0;
      }
      DIT_TRY(dit::launch_qk_rmsnorm_rope(rp, stream), "double block: rmsnorm/rope");
    }
  // one joint attention over [image; valid text], o in the joint layout
  {
    dit::AttnParams ap{};
    ap.q = big; ap.k = big + D; ap.v = big + 2 * D;
    ap.q_stride = ap.kv_stride = 3 * D;
    ap.q_batch = ap.kv_batch = N * 3 * D;
    ap.out = hbuf; ap.out_stride = D; ap.out_f32 = 0; ap.lse = nullptr;
    ap.n_q = ap.n_k = static_cast<int>(N); ap.heads = desc->attn.heads; ap.head_dim = desc->attn.head_dim;
    ap.batch = B;
    for (int b = 0; b < DIT_MAX_BATCH; ++b) ap.n_valid[b] = b < B ? S + desc->attn.txt_valid[b] : 0;
    ap.scale_log2 = 1.4426950408889634f / std::sqrt(static_cast<float>(desc->attn.head_dim));
    ap.tail_ws = split;
    DIT_TRY(dit::launch_attention(ap, stream), "double block: attention");
  }
  // per stream: x += gate1 (o W_o^T + b_o)   (both read o before h2 reuses the buffer)
  for (const Stream& t : streams) {
    if (t.rows == 0) continue;
    dit::GemmParams g = gemm(hbuf + t.first * D, D, t.w->w_o, t.w->b_o, static_cast<int64_t>(B) * t.rows,
                             D, D, t.x, D);
    g.group_rows = t.rows;
    g.a_group_stride = N * D;
    g.c_group_stride = static_cast<int64_t>(t.rows) * D;
    g.gate = t.mod + 2 * D; g.gate_stride = ms; g.gate_rows = t.rows;
    g.split_ws = split;
    DIT_TRY(dit::launch_gemm(g, DIT_EPI_GATED_RES_F32, stream), "double block: out-proj gemm");
  }
  // per stream: x += gate2 (GELU(adaLN(x; shift2, scale2) W_up^T + b_up) W_dn^T + b_dn)
  for (const Stream& t : streams) {
    if (t.rows == 0) continue;
    const int64_t M = static_cast<int64_t>(B) * t.rows;
    DIT_TRY(dit::launch_adaln(t.x, M, D, t.rows, t.mod + 3 * D, t.mod + 4 * D, ms, desc->ln_eps, t.h, stream),
            "double block: adaln 2");
    dit::GemmParams gu = gemm(t.h, D, t.w->w_up, t.w->b_up, M, F, D, t.u, F);
    gu.split_ws = split;
    DIT_TRY(dit::launch_gemm(gu, DIT_EPI_GELU_BF16, stream), "double block: mlp-up gemm");
    dit::GemmParams g = gemm(t.u, F, t.w->w_dn, t.w->b_dn, M, D, F, t.x, D);
    g.gate = t.mod + 5 * D; g.gate_stride = ms; g.gate_rows = t.rows;
    g.split_ws = split;
    DIT_TRY(dit::launch_gemm(g, DIT_EPI_GATED_RES_F32, stream), "double block: mlp-down gemm");
  }
  return ok();
}

namespace {
struct SingleWs {
  size_t h, qkv, cat, split, total;
};
SingleWs single_ws(const dit_block_desc* d) {
  const size_t M = static_cast<size_t>(d->attn.batch) * (d->attn.n_vis + d->attn.n_txt);
  const size_t D = d->hidden, F = d->mlp;
  SingleWs w;
  w.h = 0;
  w.qkv = align256(M * D * 2);
  w.cat = w.qkv + align256(M * 3 * D * 2);
  w.split = w.cat + align256(M * (D + F) * 2);
  w.total = w.split + (M >= 1024 ? dit::kSplitWsBytes : 0);
  return w;
}
}  // namespace

size_t dit_single_block_workspace_bytes(const dit_block_desc* desc) {
  if (check_block_desc(desc) != DIT_OK) return 0;
  ok();
  return single_ws(desc).total;
}

dit_status dit_single_block_forward(const dit_block_desc* desc, const dit_single_block_weights* w,
                                    const uint16_t* mod, float* x, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  dit_status st = check_block_desc(desc);
  if (st != DIT_OK) return st;
  if (!w) return fail(DIT_EINVAL, "weights struct is NULL");
  const uint16_t* ptrs[] = {w->w1, w->b1, w->g_q, w->g_k, w->w2, w->b2};
  for (const uint16_t* p : ptrs)
    if (!p || !aligned(p, 16)) return fail(DIT_EINVAL, "a weight pointer is NULL or not 16-byte aligned");
  if (!mod || !aligned(mod, 16)) return fail(DIT_EINVAL, "mod is NULL or not 16-byte aligned");
  if (!x || !aligned(x, 16)) return fail(DIT_EINVAL, "x is NULL or not 16-byte aligned");
  if (!workspace || !aligned(workspace, 256)) return fail(DIT_EINVAL, "workspace is NULL or not 256-byte aligned");
  const SingleWs WL = single_ws(desc);
  if (workspace_bytes < WL.total)
    return fail(DIT_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, WL.total);
  const int B = desc->attn.batch, D = desc->hidden, F = desc->mlp;
  const int64_t N = static_cast<int64_t>(desc->attn.n_vis) + desc->attn.n_txt;
  const int64_t M = B * N;
  if (overlap(x, static_cast<size_t>(M) * D * 4, workspace, WL.total))
    return fail(DIT_EINVAL, "x overlaps the workspace");
  const int64_t ms = desc->mod_stride;
  char* ws = static_cast<char*>(workspace);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + WL.h);
  uint16_t* qkv = reinterpret_cast<uint16_t*>(ws + WL.qkv);
  uint16_t* cat = reinterpret_cast<uint16_t*>(ws + WL.cat);  // [o | GELU(up)], row stride D + F
  float* split = WL.total > WL.split ? reinterpret_cast<float*>(ws + WL.split) : nullptr;
  const int64_t ldcat = static_cast<int64_t>(D) + F;
  // h = adaLN(x; shift, scale)
  DIT_TRY(dit::launch_adaln(x, M, D, N, mod, mod + D, ms, desc->ln_eps, h, stream), "single block: adaln");
  // linear1: rows [0, 3D) of w1 -> q|k|v, rows [3D, 3D + F) -> GELU(up) into the right of cat
  DIT_TRY(dit::launch_gemm(gemm(h, D, w->w1, w->b1, M, 3 * D, D, qkv, 3 * D, split), DIT_EPI_BF16, stream),
          "single block: linear1 qkv");
  DIT_TRY(dit::launch_gemm(gemm(h, D, w->w1 + static_cast<int64_t>(3) * D * D, w->b1 + 3 * D, M, F, D,
                                cat + D, ldcat, split),
                           DIT_EPI_GELU_BF16, stream),
          "single block: linear1 mlp");
  DIT_TRY(dit::launch_qk_rmsnorm_rope(rope_params(desc, qkv, 3 * D, w->g_q, w->g_k), stream),
          "single block: rmsnorm/rope");
  {
    dit::AttnParams ap{};
    ap.q = qkv; ap.k = qkv + D; ap.v = qkv + 2 * D;
    ap.q_stride = ap.kv_stride = 3 * D;
    ap.q_batch = ap.kv_batch = N * 3 * D;
    ap.out = cat; ap.out_stride = ldcat; ap.out_f32 = 0; ap.lse = nullptr;
    ap.n_q = ap.n_k = static_cast<int>(N); ap.heads = desc->attn.heads; ap.head_dim = desc->attn.head_dim;
    ap.batch = B;
    for (int b = 0; b < DIT_MAX_BATCH; ++b)
      ap.n_valid[b] = b < B ? desc->attn.n_vis + desc->attn.txt_valid[b] : 0;
    ap.scale_log2 = 1.4426950408889634f / std::sqrt(static_cast<float>(desc->attn.head_dim));
    ap.tail_ws = split;
    DIT_TRY(dit::launch_attention(ap, stream), "single block: attention");
  }
  // linear2 on [o | GELU(up)], gated residual
  dit::GemmParams g = gemm(cat, ldcat, w->w2, w->b2, M, D, D + F, x, D, split);
  g.gate = mod + 2 * D; g.gate_stride = ms; g.gate_rows = N;
  DIT_TRY(dit::launch_gemm(g, DIT_EPI_GATED_RES_F32, stream), "single block: linear2");
#undef DIT_TRY
  return ok();
}

// ---------------------------------------------------------------------------
// Wan-style block ("ChunkFlow", Appendix B, equations (7)-(12)): self-
// attention over the video tokens, cross-attention to the text context, MLP.

namespace {
struct WanWs {
  size_t h, big, ckv, split, total;
};
WanWs wan_ws(const dit_block_desc* d) {
  const size_t B = d->attn.batch, S = d->attn.n_vis, L = d->attn.n_txt;
  const size_t D = d->hidden, F = d->mlp;
  WanWs w;
  w.h = 0;
  w.big = align256(B * S * D * 2);
  w.ckv = w.big + align256(B * S * (3 * D > F ? 3 * D : F) * 2);
  w.split = w.ckv + align256(B * L * 2 * D * 2);
  w.total = w.split + (B * S >= 1024 ? dit::kSplitWsBytes : 0);
  return w;
}

dit::AttnParams attn_params(const uint16_t* q, int64_t q_stride, int64_t q_batch, const uint16_t* k,
                            const uint16_t* v, int64_t kv_stride, int64_t kv_batch, uint16_t* out,
                            int64_t out_stride, int n_q, int n_k, const dit_attn_desc& a,
                            const int* n_valid, float* tail_ws) {
  dit::AttnParams ap{};
  ap.tail_ws = tail_ws;
  ap.q = q; ap.k = k; ap.v = v;
  ap.q_stride = q_stride; ap.kv_stride = kv_stride;
  ap.q_batch = q_batch; ap.kv_batch = kv_batch;
  ap.out = out; ap.out_stride = out_stride; ap.out_f32 = 0; ap.lse = nullptr;
  ap.n_q = n_q; ap.n_k = n_k; ap.heads = a.heads; ap.head_dim = a.head_dim; ap.batch = a.batch;
  for (int b = 0; b < DIT_MAX_BATCH; ++b) ap.n_valid[b] = b < a.batch ? n_valid[b] : 0;
  ap.scale_log2 = 1.4426950408889634f / std::sqrt(static_cast<float>(a.head_dim));
  return ap;
}
}  // namespace

size_t dit_wan_block_workspace_bytes(const dit_block_desc* desc) {
  if (check_block_desc(desc) != DIT_OK) return 0;
  ok();
  return wan_ws(desc).total;
}

dit_status dit_wan_block_forward(const dit_block_desc* desc, const dit_wan_block_weights* w,
                                 const uint16_t* mod, float* x, const uint16_t* ctx,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dit_status st = check_block_desc(desc);
  if (st != DIT_OK) return st;
  if (!w) return fail(DIT_EINVAL, "weights struct is NULL");
  const uint16_t* ptrs[] = {w->w_qkv, w->b_qkv, w->g_q,  w->g_k,  w->w_o,  w->b_o,
                            w->w_cq,  w->b_cq,  w->w_ckv, w->b_ckv, w->g_cq, w->g_ck,
                            w->w_co,  w->b_co,  w->w_up, w->b_up, w->w_dn, w->b_dn};
  for (const uint16_t* p : ptrs)
    if (!p || !aligned(p, 16)) return fail(DIT_EINVAL, "a weight pointer is NULL or not 16-byte aligned");
  const int B = desc->attn.batch, S = desc->attn.n_vis, L = desc->attn.n_txt;
  const int D = desc->hidden, F = desc->mlp;
  if (!mod || !aligned(mod, 16)) return fail(DIT_EINVAL, "mod is NULL or not 16-byte aligned");
  if (!x || !aligned(x, 16)) return fail(DIT_EINVAL, "x is NULL or not 16-byte aligned");
  if (L > 0 && (!ctx || !aligned(ctx, 16))) return fail(DIT_EINVAL, "ctx is NULL or not 16-byte aligned");
  if (!workspace || !aligned(workspace, 256)) return fail(DIT_EINVAL, "workspace is NULL or not 256-byte aligned");
  const WanWs WL = wan_ws(desc);
  if (workspace_bytes < WL.total)
    return fail(DIT_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, WL.total);
  const int64_t M = static_cast<int64_t>(B) * S;
  const size_t x_bytes = static_cast<size_t>(M) * D * 4;
  if (overlap(x, x_bytes, workspace, WL.total) ||
      (L > 0 && overlap(x, x_bytes, ctx, static_cast<size_t>(B) * L * D * 2)))
    return fail(DIT_EINVAL, "x overlaps the workspace or ctx");
  const int64_t ms = desc->mod_stride;
  char* ws = static_cast<char*>(workspace);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(ws + WL.h);  // h, o, LN(x1), cross o, h2
  uint16_t* big = reinterpret_cast<uint16_t*>(ws + WL.big);  // self q|k|v, cross q, MLP hidden
  uint16_t* ckv = reinterpret_cast<uint16_t*>(ws + WL.ckv);  // context k|v [B*L, 2D]
  float* split = WL.total > WL.split ? reinterpret_cast<float*>(ws + WL.split) : nullptr;
#define DIT_TRY(expr, what)                            \
  do {                                                 \
    const hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_status(e_, what); \
  } while (0)
  // self-attention over the video tokens
  DIT_TRY(dit::launch_adaln(x, M, D, S, mod, mod + D, ms, desc->ln_eps, hbuf, stream), "wan block: adaln 1");
  DIT_TRY(dit::launch_gemm(gemm(hbuf, D, w->w_qkv, w->b_qkv, M, 3 * D, D, big, 3 * D, split), DIT_EPI_BF16, stream),
          "wan block: qkv gemm");
  {
    dit::RopeParams rp = rope_params(desc, big, 3 * D, w->g_q, w->g_k);
    rp.n_tok = S;  // the sequence is the video tokens alone
    rp.rows = M;
    DIT_TRY(dit::launch_qk_rmsnorm_rope(rp, stream), "wan block: rmsnorm/rope");
  }
  {
    int nv[DIT_MAX_BATCH];
    for (int b = 0; b < DIT_MAX_BATCH; ++b) nv[b] = S;
    DIT_TRY(dit::launch_attention(attn_params(big, 3 * D, static_cast<int64_t>(S) * 3 * D, big + D, big + 2 * D,
                                              3 * D, static_cast<int64_t>(S) * 3 * D, hbuf, D, S, S,
                                              desc->attn, nv, split),
                                  stream),
            "wan block: self-attention");
  }
  {
    dit::GemmParams g = gemm(hbuf, D, w->w_o, w->b_o, M, D, D, x, D, split);
    g.gate = mod + 2 * D; g.gate_stride = ms; g.gate_rows = S;
    DIT_TRY(dit::launch_gemm(g, DIT_EPI_GATED_RES_F32, stream), "wan block: out-proj gemm");
  }
  // cross-attention: q from LN(x), k|v from the context, keys [0, txt_valid[b])
  DIT_TRY(dit::launch_adaln(x, M, D, S, nullptr, nullptr, 0, desc->ln_eps, hbuf, stream), "wan block: layernorm");
  DIT_TRY(dit::launch_gemm(gemm(hbuf, D, w->w_cq, w->b_cq, M, D, D, big, D, split), DIT_EPI_BF16, stream),
          "wan block: cross q gemm");
  {
    // RMSNorm over D with the cross gains; position 0 for every row makes the
    // rotation the identity
    dit::RopeParams rp = rope_params(desc, big, D, w->g_cq, w->g_cq);
    rp.q_only = 1; rp.n_tok = 1; rp.n_vis = 0; rp.rows = M;
    DIT_TRY(dit::launch_qk_rmsnorm_rope(rp, stream), "wan block: cross q rmsnorm");
  }
  if (L > 0) {
    DIT_TRY(dit::launch_gemm(gemm(ctx, D, w->w_ckv, w->b_ckv, static_cast<int64_t>(B) * L, 2 * D, D, ckv, 2 * D),
                             DIT_EPI_BF16, stream),
            "wan block: cross kv gemm");
    dit::RopeParams rp = rope_params(desc, ckv, 2 * D, w->g_ck, w->g_ck);
    rp.q_only = 1; rp.n_tok = 1; rp.n_vis = 0; rp.rows = static_cast<int64_t>(B) * L;
    DIT_TRY(dit::launch_qk_rmsnorm_rope(rp, stream), "wan block: cross k rmsnorm");
  }
  DIT_TRY(dit::launch_attention(attn_params(big, D, static_cast<int64_t>(S) * D, ckv, ckv + D, 2 * D,
                                            static_cast<int64_t>(L) * 2 * D, hbuf, D, S, L > 0 ? L : 1,
                                            desc->attn, desc->attn.txt_valid, split),
                                stream),
          "wan block: cross-attention");
  DIT_TRY(dit::launch_gemm(gemm(hbuf, D, w->w_co, w->b_co, M, D, D, x, D, split), DIT_EPI_RES_F32, stream),
          "wan block: cross out-proj gemm");
  // MLP
  DIT_TRY(dit::launch_adaln(x, M, D, S, mod + 3 * D, mod + 4 * D, ms, desc->ln_eps, hbuf, stream),
          "wan block: adaln 2");
  DIT_TRY(dit::launch_gemm(gemm(hbuf, D, w->w_up, w->b_up, M, F, D, big, F, split), DIT_EPI_GELU_BF16, stream),
          "wan block: mlp-up gemm");
  {
    dit::GemmParams g = gemm(big, F, w->w_dn, w->b_dn, M, D, F, x, D, split);
    g.gate = mod + 5 * D; g.gate_stride = ms; g.gate_rows = S;
    DIT_TRY(dit::launch_gemm(g, DIT_EPI_GATED_RES_F32, stream), "wan block: mlp-down gemm");
  }
#undef DIT_TRY
  return ok();
}

size_t dit_denoise_workspace_bytes(const dit_model_desc* desc) {
  if (check_model_desc(desc) != DIT_OK) return 0;
  ok();
  return step_layout(desc).total;
}

}  // extern "C"

namespace {

#define DIT_TRY(expr, what)                            \
  do {                                                 \
    const hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_status(e_, what); \
  } while (0)

// Argument checks shared by the denoising-step entry points: descriptor,
// weights, latent, scalars and workspace.
dit_status check_step_args(const dit_model_desc* desc, const dit_model_weights* w,
                           const float* latent, float sigma, float sigma_next, float guidance,
                           void* workspace, size_t workspace_bytes, StepLayout* L) {
  dit_status st = check_model_desc(desc);
  if (st != DIT_OK) return st;
  if (!w) return fail(DIT_EINVAL, "model weights are NULL");
  const uint16_t* glue[] = {w->t_w1, w->t_b1, w->t_w2, w->t_b2, w->in_w, w->in_b,
                            w->fin_w, w->fin_b, w->out_w, w->out_b, w->text};
  for (const uint16_t* p : glue)
    if (!p || !aligned(p, 16)) return fail(DIT_EINVAL, "a model weight is NULL or not 16-byte aligned");
  if (!w->blocks || !w->mod_w || !w->mod_b) return fail(DIT_EINVAL, "NULL per-layer arrays");
  for (int l = 0; l < desc->depth; ++l) {
    st = check_block_weights(&w->blocks[l]);
    if (st != DIT_OK) return st;
    if (!w->mod_w[l] || !w->mod_b[l] || !aligned(w->mod_w[l], 16) || !aligned(w->mod_b[l], 16))
      return fail(DIT_EINVAL, "modulation weights of layer %d are NULL or misaligned", l);
  }
  if (!latent || !aligned(latent, 16)) return fail(DIT_EINVAL, "latent is NULL or not 16-byte aligned");
  if (!std::isfinite(sigma) || !std::isfinite(sigma_next) || !std::isfinite(guidance))
    return fail(DIT_EINVAL, "sigma, sigma_next and guidance must be finite");
  if (!workspace || !aligned(workspace, 256)) return fail(DIT_EINVAL, "workspace is NULL or not 256-byte aligned");
  *L = step_layout(desc);
  if (workspace_bytes < L->total)
    return fail(DIT_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, L->total);
  const dit_block_desc& bd = desc->block;
  const size_t lat_bytes = static_cast<size_t>(desc->cfg ? 1 : bd.attn.batch) * bd.attn.n_vis *
                           desc->latent_channels * 4;
  if (overlap(latent, lat_bytes, workspace, L->total))
    return fail(DIT_EINVAL, "latent overlaps the workspace");
  return DIT_OK;
}

// Timestep conditioning s, the modulations of layers [0, mod_layers) (and,
// when that is every layer, the final one) and the first block's input
// tokens x:
//   f = sinusoidal(t_scale * sigma);  c = SiLU(f W1 + b1);  s = SiLU(c W2 + b2)
//   mod_l = s W_mod[l] + b_mod[l];  fin = s W_fin + b_fin
//   x[b] = [bf16(latent) W_in + b_in ; text[b]]
// The modulations are matrix-vector products bound by their weight reads;
// they run before the input projection, whose 4-byte-per-element store of x
// would otherwise leave the caches full of fresh lines whose write-back
// competes with those reads (at c3 the block modulation took 101 us inside
// the step after the input projection, against 54 us from a clean cache).
dit_status step_prologue(const dit_model_desc* desc, const dit_model_weights* w,
                         const float* latent, float sigma, const StepLayout& L, char* ws,
                         int mod_layers, hipStream_t stream) {
  const dit_block_desc& bd = desc->block;
  const int B = bd.attn.batch, nv = bd.attn.n_vis;
  const int64_t N = static_cast<int64_t>(nv) + bd.attn.n_txt;
  const int D = bd.hidden, C = desc->latent_channels, Fq = desc->freq_dim;
  const int Bl = desc->cfg ? 1 : B;
  uint16_t* feat = reinterpret_cast<uint16_t*>(ws + L.feat);
  uint16_t* cbuf = reinterpret_cast<uint16_t*>(ws + L.c);
  uint16_t* sbuf = reinterpret_cast<uint16_t*>(ws + L.s);
  uint16_t* lat = reinterpret_cast<uint16_t*>(ws + L.lat);
  float* x = reinterpret_cast<float*>(ws + L.x);
  DIT_TRY(dit::launch_timestep_features(nullptr, sigma, 1, Fq, desc->t_scale, feat, stream), "step: timestep");
  DIT_TRY(dit::launch_gemm(gemm(feat, Fq, w->t_w1, w->t_b1, 1, D, Fq, cbuf, D), DIT_EPI_SILU_BF16, stream),
          "step: t-mlp 1");
  DIT_TRY(dit::launch_gemm(gemm(cbuf, D, w->t_w2, w->t_b2, 1, D, D, sbuf, D), DIT_EPI_SILU_BF16, stream),
          "step: t-mlp 2");
  uint16_t* mod = reinterpret_cast<uint16_t*>(ws + L.mod);
  for (int l = 0; l < mod_layers; ++l)
    DIT_TRY(dit::launch_gemm(gemm(sbuf, D, w->mod_w[l], w->mod_b[l], 1, 6 * D, D,
                                  mod + static_cast<int64_t>(l) * 6 * D, 6 * D),
                             DIT_EPI_BF16, stream),
            "step: modulation");
  if (mod_layers == desc->depth)
    DIT_TRY(dit::launch_gemm(gemm(sbuf, D, w->fin_w, w->fin_b, 1, 2 * D, D,
                                  reinterpret_cast<uint16_t*>(ws + L.fin), 2 * D),
                             DIT_EPI_BF16, stream),
            "step: final modulation");
  DIT_TRY(dit::launch_cast_f32_bf16(latent, C, static_cast<int64_t>(Bl) * nv, C, lat, C, stream),
          "step: latent cast");
  {
    dit::GemmParams g = gemm(lat, C, w->in_w, w->in_b, static_cast<int64_t>(B) * nv, D, C, x, D);
    g.group_rows = nv;
    g.a_group_stride = desc->cfg ? 0 : static_cast<int64_t>(nv) * C;
    g.c_group_stride = N * D;
    DIT_TRY(dit::launch_gemm(g, DIT_EPI_F32, stream), "step: input projection");
  }
  for (int b = 0; b < B; ++b)
    DIT_TRY(dit::launch_cast_bf16_f32(w->text + static_cast<int64_t>(b) * bd.attn.n_txt * D, D,
                                      bd.attn.n_txt, D, x + (b * N + nv) * D, D, stream),
            "step: text rows");
  return DIT_OK;
}

// The block stack on x (modulations from the prologue), the final adaLN and
// the projection of the visual rows to the latent channels: v bf16
// [batch, n_vis, C] in the workspace.
dit_status step_denoiser(const dit_model_desc* desc, const dit_model_weights* w,
                         const StepLayout& L, char* ws, hipStream_t stream) {
  dit_block_desc bd = desc->block;
  bd.mod_stride = 0;  // one modulation vector per step, shared by every batch row
  const int B = bd.attn.batch, nv = bd.attn.n_vis;
  const int64_t N = static_cast<int64_t>(nv) + bd.attn.n_txt;
  const int D = bd.hidden, C = desc->latent_channels;
  uint16_t* mod = reinterpret_cast<uint16_t*>(ws + L.mod);
  uint16_t* fin = reinterpret_cast<uint16_t*>(ws + L.fin);
  float* x = reinterpret_cast<float*>(ws + L.x);
  uint16_t* hf = reinterpret_cast<uint16_t*>(ws + L.hf);
  uint16_t* v = reinterpret_cast<uint16_t*>(ws + L.v);
  char* blk = ws + L.blk;
  for (int l = 0; l < desc->depth; ++l) {
    const char* what = nullptr;
    const hipError_t e = block_launch(&bd, &w->blocks[l], mod + static_cast<int64_t>(l) * 6 * D, 0, x, blk,
                                      stream, &what);
    if (e != hipSuccess) return hip_status(e, what);
  }
  DIT_TRY(dit::launch_adaln(x, B * N, D, N, fin, fin + D, 0, bd.ln_eps, hf, stream), "step: final adaln");
  dit::GemmParams g = gemm(hf, D, w->out_w, w->out_b, static_cast<int64_t>(B) * nv, C, D, v, C);
  g.group_rows = nv;
  g.a_group_stride = N * D;
  g.c_group_stride = static_cast<int64_t>(nv) * C;
  DIT_TRY(dit::launch_gemm(g, DIT_EPI_BF16, stream), "step: output projection");
  return DIT_OK;
}

// Elements of the velocity the sampler uses (and of the latent).
int64_t step_velocity_elems(const dit_model_desc* desc) {
  const dit_block_desc& bd = desc->block;
  return static_cast<int64_t>(desc->cfg ? 1 : bd.attn.batch) * bd.attn.n_vis * desc->latent_channels;
}

// Host-side skip decision of a step-caching controller.  Every quantity is
// double and evaluated without contraction so that the decision does not
// depend on the compiler's choice of fused multiply-adds.
double cache_rescale(const dit_cache_policy& p, double r) {
#pragma clang fp contract(off)
  double y = 0.0;
  for (int i = 0; i < p.n_coef; ++i) y = y * r + p.coef[i];
  return y;
}

}  // namespace

extern "C" {

dit_status dit_denoise_step(const dit_model_desc* desc, const dit_model_weights* w, float* latent,
                            float sigma, float sigma_next, float guidance, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  StepLayout L;
  dit_status st = check_step_args(desc, w, latent, sigma, sigma_next, guidance, workspace,
                                  workspace_bytes, &L);
  if (st != DIT_OK) return st;
  char* ws = static_cast<char*>(workspace);
  if ((st = step_prologue(desc, w, latent, sigma, L, ws, desc->depth, stream)) != DIT_OK) return st;
  if ((st = step_denoiser(desc, w, L, ws, stream)) != DIT_OK) return st;
  // guidance + Euler on the fp32 latent
  const uint16_t* v = reinterpret_cast<const uint16_t*>(ws + L.v);
  const int64_t n = step_velocity_elems(desc);
  if (desc->cfg)
    DIT_TRY(dit::launch_euler(latent, v, v + n, n, guidance, sigma_next - sigma, stream), "step: euler");
  else
    DIT_TRY(dit::launch_euler(latent, v, nullptr, n, 1.f, sigma_next - sigma, stream), "step: euler");
  return ok();
}

size_t dit_change_score_workspace_bytes(void) { return dit::kScorePartialBytes; }

static_assert(DIT_CHANGE_SCORE_SCRATCH_BYTES == dit::kScorePartialBytes,
              "the documented scratch size is the kernels' partial-sum size");

// Checks shared by dit_change_score and dit_change_score_noalloc (the
// workspace ones only when a workspace is passed).
dit_status check_change_score(const void* cur, void* prev, int32_t dtype, int64_t n, int32_t update,
                              float* score, const void* workspace, size_t workspace_bytes,
                              bool has_workspace) {
  if (dtype != DIT_DTYPE_BF16 && dtype != DIT_DTYPE_F32)
    return fail(DIT_EINVAL, "dtype %d is neither DIT_DTYPE_BF16 nor DIT_DTYPE_F32", dtype);
  if (n < 1) return fail(DIT_EINVAL, "n %lld < 1", static_cast<long long>(n));
  if (n > DIT_CHANGE_SCORE_MAX_N)
    return fail(DIT_EINVAL, "n %lld > %lld", static_cast<long long>(n),
                static_cast<long long>(DIT_CHANGE_SCORE_MAX_N));
  if (update != 0 && update != 1) return fail(DIT_EINVAL, "update must be 0 or 1");
  if (!cur || !prev || !score || (has_workspace && !workspace))
    return fail(DIT_EINVAL, has_workspace ? "NULL cur, prev, score or workspace" : "NULL cur, prev or score");
  if (!aligned(cur, 16) || !aligned(prev, 16) || !aligned(score, 4) ||
      (has_workspace && !aligned(workspace, 16)))
    return fail(DIT_EINVAL, "cur, prev and workspace must be 16-byte aligned, score 4-byte");
  if (has_workspace && workspace_bytes < dit::kScorePartialBytes)
    return fail(DIT_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, dit::kScorePartialBytes);
  const size_t bytes = static_cast<size_t>(n) * (dtype == DIT_DTYPE_BF16 ? 2 : 4);
  if (update && overlap(cur, bytes, prev, bytes))
    return fail(DIT_EINVAL, "cur and prev overlap (prev is overwritten)");
  if (overlap(score, 4, cur, bytes) || overlap(score, 4, prev, bytes))
    return fail(DIT_EINVAL, "score overlaps an array");
  if (has_workspace && (overlap(workspace, dit::kScorePartialBytes, cur, bytes) ||
                        overlap(workspace, dit::kScorePartialBytes, prev, bytes) ||
                        overlap(workspace, dit::kScorePartialBytes, score, 4)))
    return fail(DIT_EINVAL, "workspace overlaps an array");
  return DIT_OK;
}

dit_status dit_change_score(const void* cur, void* prev, int32_t dtype, int64_t n, int32_t update,
                            float* score, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  dit_status st = check_change_score(cur, prev, dtype, n, update, score, workspace, workspace_bytes, true);
  if (st != DIT_OK) return st;
  return hip_status(dit::launch_change_score(cur, prev, dtype == DIT_DTYPE_BF16, n, update != 0,
                                             static_cast<float*>(workspace), score, stream),
                    "change-score launch");
}

dit_status dit_change_score_noalloc(const void* cur, void* prev, int32_t dtype, int64_t n,
                                    int32_t update, float* score, hipStream_t stream) {
  dit_status st = check_change_score(cur, prev, dtype, n, update, score, nullptr, 0, false);
  if (st != DIT_OK) return st;
  float* partials = nullptr;
  st = hip_status(dit::change_score_scratch(&partials), "change-score scratch address");
  if (st != DIT_OK) return st;
  return hip_status(dit::launch_change_score(cur, prev, dtype == DIT_DTYPE_BF16, n, update != 0,
                                             partials, score, stream),
                    "change-score launch");
}

dit_status dit_cache_probe(const dit_model_desc* desc, const dit_model_weights* w,
                           const float* latent, float sigma, uint16_t* saved, int32_t have_saved,
                           float* score, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  StepLayout L;
  dit_status st = check_step_args(desc, w, latent, sigma, sigma, 1.f, workspace, workspace_bytes, &L);
  if (st != DIT_OK) return st;
  if (have_saved != 0 && have_saved != 1) return fail(DIT_EINVAL, "have_saved must be 0 or 1");
  if (!saved || !score || !aligned(saved, 16) || !aligned(score, 4))
    return fail(DIT_EINVAL, "saved (16-byte aligned) and score must not be NULL");
  const dit_block_desc& bd = desc->block;
  const int64_t rows = static_cast<int64_t>(bd.attn.batch) * (static_cast<int64_t>(bd.attn.n_vis) + bd.attn.n_txt);
  const int D = bd.hidden;
  const size_t feat_bytes = static_cast<size_t>(rows) * D * 2;
  if (overlap(saved, feat_bytes, workspace, L.total) || overlap(score, 4, workspace, L.total) ||
      overlap(score, 4, saved, feat_bytes))
    return fail(DIT_EINVAL, "saved or score overlaps the workspace or each other");
  char* ws = static_cast<char*>(workspace);
  if ((st = step_prologue(desc, w, latent, sigma, L, ws, 1, stream)) != DIT_OK) return st;
  uint16_t* mod = reinterpret_cast<uint16_t*>(ws + L.mod);
  const float* x = reinterpret_cast<const float*>(ws + L.x);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.hf);
  float* part = reinterpret_cast<float*>(ws + L.part);
  const int64_t N = static_cast<int64_t>(bd.attn.n_vis) + bd.attn.n_txt;
  // block 0's first adaLN (its modulation from the prologue): h = LN(x) (1 + scale1) + shift1
  DIT_TRY(dit::launch_adaln(x, rows, D, N, mod, mod + D, 0, bd.ln_eps, h, stream), "probe: adaln");
  if (have_saved)
    DIT_TRY(dit::launch_change_score(h, saved, true, rows * D, true, part, score, stream), "probe: score");
  else {
    DIT_TRY(hipMemcpyAsync(saved, h, feat_bytes, hipMemcpyDeviceToDevice, stream), "probe: save");
    DIT_TRY(dit::launch_score_invalid(part, score, stream), "probe: score");
  }
  return ok();
}

dit_status dit_denoise_step_cached(const dit_model_desc* desc, const dit_model_weights* w,
                                   float* latent, float sigma, float sigma_next, float guidance,
                                   int32_t action, int32_t have_prev, float* prev_v,
                                   float* delta_v, float* score, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  StepLayout L;
  dit_status st = check_step_args(desc, w, latent, sigma, sigma_next, guidance, workspace,
                                  workspace_bytes, &L);
  if (st != DIT_OK) return st;
  if (action != DIT_STEP_FULL && action != DIT_STEP_SKIP)
    return fail(DIT_EINVAL, "action %d is neither DIT_STEP_FULL nor DIT_STEP_SKIP", action);
  if (have_prev != 0 && have_prev != 1) return fail(DIT_EINVAL, "have_prev must be 0 or 1");
  if (action == DIT_STEP_SKIP && !have_prev)
    return fail(DIT_EINVAL, "a cached step needs a previous output and a measured change");
  if (!prev_v || !delta_v || !aligned(prev_v, 16) || !aligned(delta_v, 16))
    return fail(DIT_EINVAL, "prev_v and delta_v must be non-NULL and 16-byte aligned");
  if (score && !aligned(score, 4)) return fail(DIT_EINVAL, "score must be 4-byte aligned");
  const int64_t n = step_velocity_elems(desc);
  const size_t vb = static_cast<size_t>(n) * 4;
  if (overlap(prev_v, vb, delta_v, vb) || overlap(prev_v, vb, latent, vb) ||
      overlap(delta_v, vb, latent, vb) || overlap(prev_v, vb, workspace, L.total) ||
      overlap(delta_v, vb, workspace, L.total) ||
      (score && (overlap(score, 4, workspace, L.total) || overlap(score, 4, prev_v, vb) ||
                 overlap(score, 4, delta_v, vb) || overlap(score, 4, latent, vb))))
    return fail(DIT_EINVAL, "latent, prev_v, delta_v, score and workspace must not overlap");
  char* ws = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(ws + L.part);
  const float dt = sigma_next - sigma;
  if (action == DIT_STEP_SKIP) {
    DIT_TRY(dit::launch_cached_velocity(latent, nullptr, nullptr, n, 1.f, dt, prev_v, delta_v, true,
                                        true, part, nullptr, stream),
            "cached step: estimate");
    return ok();
  }
  if ((st = step_prologue(desc, w, latent, sigma, L, ws, desc->depth, stream)) != DIT_OK) return st;
  if ((st = step_denoiser(desc, w, L, ws, stream)) != DIT_OK) return st;
  const uint16_t* v = reinterpret_cast<const uint16_t*>(ws + L.v);
  DIT_TRY(dit::launch_cached_velocity(latent, v, desc->cfg ? v + n : nullptr, n,
                                      desc->cfg ? guidance : 1.f, dt, prev_v, delta_v, false,
                                      have_prev != 0, part, score, stream),
          "cached step: full");
  return ok();
}

dit_status dit_cache_ctrl_init(dit_cache_ctrl* c, const dit_cache_policy* p) {
  if (!c || !p) return fail(DIT_EINVAL, "NULL controller or policy");
  if (p->mode < DIT_CACHE_OFF || p->mode > DIT_CACHE_TEACACHE)
    return fail(DIT_EINVAL, "unknown cache mode %d", p->mode);
  if (p->n_steps < 1) return fail(DIT_EINVAL, "n_steps %d < 1", p->n_steps);
  if (p->warmup < 0 || p->cooldown < 0) return fail(DIT_EINVAL, "negative warmup or cooldown");
  if (p->mode == DIT_CACHE_CADENCE && p->cadence < 1) return fail(DIT_EINVAL, "cadence %d < 1", p->cadence);
  if (p->mode == DIT_CACHE_ONLINE_DELTA && !(p->alpha >= 0.0 && std::isfinite(p->alpha)))
    return fail(DIT_EINVAL, "alpha must be finite and >= 0");
  if (p->mode == DIT_CACHE_TEACACHE) {
    if (!std::isfinite(p->threshold)) return fail(DIT_EINVAL, "threshold must be finite");
    if (p->n_coef < 1 || p->n_coef > DIT_CACHE_MAX_COEF)
      return fail(DIT_EINVAL, "n_coef %d outside [1, %d]", p->n_coef, DIT_CACHE_MAX_COEF);
    for (int i = 0; i < p->n_coef; ++i)
      if (!std::isfinite(p->coef[i])) return fail(DIT_EINVAL, "coefficient %d is not finite", i);
  }
  std::memset(c, 0, sizeof(*c));
  c->policy = *p;
  return ok();
}

dit_status dit_cache_ctrl_decide(dit_cache_ctrl* c, int32_t step, float probe_score, int32_t* action) {
  if (!c || !action) return fail(DIT_EINVAL, "NULL controller or action");
  if (step != c->next_step)
    return fail(DIT_EINVAL, "steps must be decided in order: expected %d, got %d", c->next_step, step);
  if (step >= c->policy.n_steps) return fail(DIT_EINVAL, "step %d past n_steps %d", step, c->policy.n_steps);
  const dit_cache_policy& p = c->policy;
  c->next_step = step + 1;
  const bool boundary = step < p.warmup || step >= p.n_steps - p.cooldown;
  const bool allowed = !boundary && c->n_full >= 2;
  bool skip = false;
  switch (p.mode) {
    case DIT_CACHE_OFF: break;
    case DIT_CACHE_CADENCE: skip = allowed && (step - p.warmup) % p.cadence != 0; break;
    case DIT_CACHE_ONLINE_DELTA: skip = allowed && !c->last_skipped && c->skip_next; break;
    case DIT_CACHE_TEACACHE:
      if (std::isfinite(probe_score)) {
        c->acc = c->acc + cache_rescale(p, static_cast<double>(probe_score));
        skip = allowed && c->acc < p.threshold;
      }
      break;
  }
  if (skip) {
    c->last_skipped = 1;
    c->skip_next = 0;
    *action = DIT_STEP_SKIP;
  } else {
    c->last_skipped = 0;
    c->acc = 0.0;
    ++c->n_full;
    *action = DIT_STEP_FULL;
  }
  return ok();
}

dit_status dit_cache_ctrl_observe(dit_cache_ctrl* c, float output_change) {
  if (!c) return fail(DIT_EINVAL, "NULL controller");
  if (c->policy.mode != DIT_CACHE_ONLINE_DELTA || !std::isfinite(output_change)) return ok();
  const double v = static_cast<double>(output_change);
  if (!c->have_first) {
    c->first_change = v;
    c->have_first = 1;
  }
  c->skip_next = v < c->policy.alpha * c->first_change;
  return ok();
}

#undef DIT_TRY

}  // extern "C"
