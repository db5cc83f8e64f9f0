/*
 * dit.h -- C ABI of the MI355X (gfx950) DiT denoiser hot path.
 *
 * One denoising step, as the pages state it: the denoiser takes the current
 * latent, the timestep and the text conditioning and predicts a velocity; the
 * sampler turns that velocity into a less noisy latent ("Difflet" paper,
 * section 1 Introduction and section 3 Model Pipelines).  Per-request
 * variation reaches the device only as a small runtime value -- the number of
 * valid text keys -- never as a mask ("Difflet", section 1 and section 4.2
 * Representing Attention Mask).
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer unless stated otherwise; every
 *    descriptor/struct pointer is a HOST pointer, read during the call only.
 *  - bf16 tensors are passed as uint16_t bit patterns (bfloat16, the top half
 *    of an IEEE binary32).  All tensors are row-major; strides are counted in
 *    elements, not bytes.
 *  - Ownership: the caller allocates and frees every buffer, workspace
 *    included.  The library allocates nothing and keeps no per-call state.
 *  - Asynchrony: every call only enqueues kernels on `stream` (0 = the null
 *    stream) and returns; results are ready when the stream reaches them.
 *  - Errors: arguments are checked on the host before anything is enqueued.
 *    A call that returns anything but DIT_OK has enqueued nothing (no partial
 *    work).  dit_last_error() then holds a thread-local message.  A failed
 *    launch returns DIT_EHIP.
 *  - Determinism: no atomics and no data-dependent reduction order; equal
 *    inputs give bitwise-equal outputs.
 *  - Unsupported layouts fail here, at the boundary, and are never silently
 *    rewritten ("Difflet Engineering Report", Backend operation boundary).
 */
#ifndef DIT_H_
#define DIT_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dit_status {
  DIT_OK = 0,
  DIT_EINVAL = 1,       /* bad argument: null pointer, shape, range, alias    */
  DIT_EUNSUPPORTED = 2, /* well-formed but outside what the kernels implement */
  DIT_EWORKSPACE = 3,   /* workspace smaller than dit_block_workspace_bytes() */
  DIT_EHIP = 4          /* a HIP launch or runtime call failed                */
} dit_status;

#define DIT_MAX_BATCH 8

/* Static description of a joint-attention call.
 * Token order of every batch row is [visual (n_vis); text (n_txt)].  Text
 * padding sits after the valid text tokens, so the valid keys of row b are the
 * single interval [0, n_vis + txt_valid[b]) ("Difflet", section 4.2
 * Representing Attention Mask; "Difflet Engineering Report", Attention CTE
 * routing and mask representation).
 *   batch      1 .. DIT_MAX_BATCH
 *   n_vis      >= 0 visual tokens; n_txt >= 0 text slots; n_vis + n_txt >= 1
 *   heads      >= 1, with ceil((n_vis + n_txt) / 256) * heads * batch at most
 *              8388607 (one 512-thread workgroup per 256-query tile, head and
 *              batch row on a 1-D grid; more is DIT_EUNSUPPORTED)
 *   head_dim   64 or 128
 *   txt_valid  host values in [0, n_txt] (entries past `batch` are ignored);
 *              n_vis + txt_valid[b] must be >= 1 so no row is empty. */
typedef struct dit_attn_desc {
  int32_t batch, n_vis, n_txt, heads, head_dim;
  int32_t txt_valid[DIT_MAX_BATCH];
} dit_attn_desc;

/* Joint attention ("Difflet", section 4: one softmax over the visual and text
 * keys of each query; section 4.2: padded text keys excluded by the interval
 * bound, fully padded key tiles never visited).
 *
 * For every batch row b, head h and query token i (all N = n_vis + n_txt
 * rows, padded text rows included):
 *   o[b,i,h,:] = sum_{j < n_vis+txt_valid[b]} softmax_j(scale * q.k_j) v_j
 *
 *   q, k, v  bf16, element [b, i, h, e] at  ptr + (b*N + i)*qkv_row_stride
 *            + h*head_dim + e   (e.g. three column blocks of one [B,N,3*H*d]
 *            buffer with qkv_row_stride = 3*H*d).  Must be 16-byte aligned
 *            and qkv_row_stride a multiple of 8, at most 2^24
 *            (DIT_EUNSUPPORTED above).
 *   out      bf16 [b, i, h, e] at  out + (b*N + i)*out_row_stride + h*head_dim
 *            + e;  out_row_stride >= heads*head_dim, multiple of 8.  Must not
 *            overlap q, k or v.
 *   lse      nullable; fp32 [batch, heads, N]: natural-log softmax
 *            denominator of each row (max included), for merging partials.
 *   softmax_scale  0 -> 1/sqrt(head_dim).
 *   workspace  optional device scratch (NULL, or >=
 *            dit_joint_attention_workspace_bytes() bytes, 256-byte aligned,
 *            not overlapping q, k, v, out or lse; else DIT_EWORKSPACE /
 *            DIT_EINVAL).  With it, when the 256-query tiles of all rows and
 *            heads fill the device's compute units at least once and leave a
 *            part-filled last round that a split finishes sooner, each tile
 *            of that round is split into 2-4 key ranges attended separately
 *            and merged by their log-denominators ("Difflet", section 4.3: the partial/merge
 *            arithmetic of ring attention): the same weighted sum, up to fp32
 *            and bf16 rounding of the partials (bitwise reproducible on one
 *            device; the split depends on its compute-unit count).  Its
 *            contents are overwritten and not read across calls.
 * Scores are accumulated in fp32 from bf16 inputs (MFMA), softmax statistics
 * are fp32, probabilities are rounded to bf16 for the value product.  They are
 * taken relative to a per-query reference that is the running maximum, or,
 * once a query's weights sum to 32 or more, lags it by at most 2 (log2
 * units); a key that sets a new maximum within that lag then gets a rounded
 * weight rather than exactly 1, which moves the output by at most 2^-12 of
 * the largest |v| per such key. */
size_t dit_joint_attention_workspace_bytes(void);
dit_status dit_joint_attention(const dit_attn_desc* desc, const uint16_t* q,
                               const uint16_t* k, const uint16_t* v,
                               int64_t qkv_row_stride, uint16_t* out,
                               int64_t out_row_stride, float* lse,
                               float softmax_scale, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Split joint attention ("Difflet", section 4.3, Ring for joint attention):
 * the key set of each query is cut into partitions -- the text keys with
 * bounds [0, L_text) and one partition per chunk of visual keys -- and each
 * partition is attended separately; partials are merged afterwards by
 * rescaling to a common maximum.  This is the building block of sequence-
 * parallel attention; on one GPU it lets a caller split a long key sequence.
 *
 * dit_attention_partial: for every batch row b, head h and query row i
 * (i < n_q), attention of q over the valid keys [0, k_valid[b]) of the
 * partition (k_valid[b] in [0, n_k]; 0 is an empty partition):
 *   out[b,i,h,:] = sum_j softmax_j(scale * q.k_j) v_j      (fp32, normalised)
 *   lse[b,h,i]   = log sum_j exp(scale * q.k_j)            (natural log)
 * An empty partition writes out = 0 and lse = -inf (the neutral element of
 * the merge).
 *   q    bf16, element (b, i, h, e) at q + (b*n_q + i)*q_row_stride + h*head_dim + e
 *   k, v bf16, element (b, j, h, e) at k + (b*n_k + j)*kv_row_stride + h*head_dim + e
 *   out  fp32, element (b, i, h, e) at out + (b*n_q + i)*out_row_stride + h*head_dim + e
 *   lse  fp32 [batch, heads, n_q], required.
 * Strides are multiples of 8 (q, k, v; kv_row_stride at most 2^24) and of 4
 * (out) and at least heads*head_dim; pointers 16-byte aligned (lse 4-byte).
 * out and lse must not overlap q, k, v or each other.  head_dim 64 or 128;
 * ceil(n_q / 256) * heads * batch at most 8388607 (else DIT_EUNSUPPORTED).
 * Arithmetic as in dit_joint_attention (the same softmax reference). */
#define DIT_MAX_PARTS 32
typedef struct dit_partial_desc {
  int32_t batch;      /* 1..DIT_MAX_BATCH */
  int32_t n_q;        /* query rows per batch row (>= 1) */
  int32_t n_k;        /* key rows of this partition per batch row (>= 1) */
  int32_t heads;
  int32_t head_dim;   /* 64 or 128 */
  int32_t k_valid[DIT_MAX_BATCH];  /* valid keys of batch row b: [0, k_valid[b]) */
} dit_partial_desc;

dit_status dit_attention_partial(const dit_partial_desc* desc, const uint16_t* q,
                                 int64_t q_row_stride, const uint16_t* k,
                                 const uint16_t* v, int64_t kv_row_stride, float* out,
                                 int64_t out_row_stride, float* lse, float softmax_scale,
                                 hipStream_t stream);

/* dit_attention_merge: joint normalisation of `parts` partials of the same
 * queries ("Difflet", section 4.3: rescale to a common maximum, add, divide):
 *   M        = max_p lse_p[b,h,i]
 *   w_p      = exp(lse_p[b,h,i] - M)
 *   out      = sum_p w_p out_p[b,i,h,:] / sum_p w_p     (bf16, RNE)
 *   lse_out  = M + log(sum_p w_p)                        (nullable, fp32)
 * (With out_p = acc_p / l_p and lse_p = m_p + log l_p this is the page's
 * (sum_p e^(m_p - M) acc_p) / (sum_p e^(m_p - M) l_p).)
 *   outs, lses  host arrays of `parts` device pointers laid out as the out
 *               and lse of dit_attention_partial (part_row_stride for all)
 *   out         bf16 (b, i, h, e) at out + (b*n_q + i)*out_row_stride + h*head_dim + e
 * parts in [1, DIT_MAX_PARTS].  A (b, h, i) whose partials all hold no
 * valid key (every lse_p = -inf) gets out = 0 and lse_out = -inf, the merge's
 * neutral element (what an empty partial itself returns).  Strides: part_row_stride a
 * multiple of 4, out_row_stride a multiple of 8, both >= heads*head_dim.
 * out must not overlap any input. */
typedef struct dit_merge_desc {
  int32_t batch, n_q, heads, head_dim, parts;
} dit_merge_desc;

dit_status dit_attention_merge(const dit_merge_desc* desc, const float* const* outs,
                               int64_t part_row_stride, const float* const* lses,
                               uint16_t* out, int64_t out_row_stride, float* lse_out,
                               hipStream_t stream);

/* Linear layer epilogues (the GEMM of "ChunkFlow" Appendix B equations (13)
 * and (16), with the work around it fused into the store). */
typedef enum dit_epilogue {
  DIT_EPI_BF16 = 0,        /* out(bf16) = acc + bias                         */
  DIT_EPI_GELU_BF16 = 1,   /* out(bf16) = GELU_erf(acc + bias)               */
  DIT_EPI_SILU_BF16 = 2,   /* out(bf16) = SiLU(acc + bias)                   */
  DIT_EPI_F32 = 3,         /* out(fp32) = acc + bias                         */
  DIT_EPI_GATED_RES_F32 = 4, /* out(fp32) += gate[g,:] * (acc + bias)        */
  DIT_EPI_RES_F32 = 5        /* out(fp32) += acc + bias                        */
} dit_epilogue;

/* y = A W^T + bias with an epilogue.
 *   a     bf16 [m, k]: row r at a + (r / group_rows)*a_group_stride
 *         + (r % group_rows)*lda.  With group_rows == 0 rows are a + r*lda.
 *   w     bf16 [n, k], contiguous (k contiguous): PyTorch Linear layout.
 *   bias  bf16 [n] or NULL.
 *   out   row r at out + (r / group_rows)*c_group_stride + (r % group_rows)*ldc;
 *         bf16 or fp32 by epilogue.  With DIT_EPI_GATED_RES_F32 and
 *         DIT_EPI_RES_F32 `out` is read and written (the residual stream).
 *         For every epilogue `out` must not overlap a, the bias or (gated)
 *         the gate rows it reads (DIT_EINVAL, nothing enqueued).
 *   gate  bf16, DIT_EPI_GATED_RES_F32 only: row r uses gate + (r / gate_rows)
 *         * gate_stride (gate_rows >= 1).
 *   workspace  optional device scratch (NULL, or >= dit_linear_workspace_bytes()
 *         bytes, 256-byte aligned, overlapping none of the other buffers;
 *         DIT_EINVAL / DIT_EWORKSPACE otherwise).  With it, when the last
 *         round of 256 x 256 output tiles would fill fewer than half of the
 *         GPU's compute units, those tiles are split along K over several
 *         workgroups and their fp32 partial sums added in K order by a second
 *         kernel (deterministic; the summation order differs from the
 *         unsplit path's).  Its contents are scratch: overwritten, not read
 *         across calls; calls that share it must be ordered on one stream.
 * Requires k % 64 == 0 and m <= DIT_LINEAR_MAX_M (DIT_EUNSUPPORTED otherwise),
 * lda/ldc/strides multiples of 8, pointers 16-byte aligned.  m, n >= 1
 * (m == 0 is a no-op). */
#define DIT_LINEAR_MAX_M (65535LL * 256)
typedef struct dit_linear_args {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* w;
  const uint16_t* bias;
  int64_t m;
  int32_t n, k;
  int32_t epilogue;
  void* out;
  int64_t ldc;
  const uint16_t* gate;
  int64_t gate_stride, gate_rows;
  int64_t group_rows, a_group_stride, c_group_stride;
  void* workspace;
  size_t workspace_bytes;
} dit_linear_args;

/* Bytes of the optional dit_linear workspace (64 MiB: 256 partial tiles). */
size_t dit_linear_workspace_bytes(void);
dit_status dit_linear(const dit_linear_args* args, hipStream_t stream);

/* Adaptive LayerNorm ("Difflet Engineering Report", Terms used in this
 * report: AdaLN): per row r of x (fp32 [rows, hidden], row stride `hidden`)
 *   out[r,:] = (x - mean) / sqrt(var + eps) * (1 + scale[b,:]) + shift[b,:]
 * with biased variance, no learned affine, b = r / rows_per_batch, and
 * shift/scale bf16 rows at shift + b*mod_stride, scale + b*mod_stride
 * (mod_stride may be 0 to share one vector); shift = scale = NULL is a plain
 * LayerNorm without affine.  out is bf16 [rows, hidden].
 * hidden % 8 == 0 and hidden <= 16384. */
dit_status dit_adaln_modulate(const float* x, int64_t rows, int32_t hidden,
                              int64_t rows_per_batch, const uint16_t* shift,
                              const uint16_t* scale, int64_t mod_stride,
                              float eps, uint16_t* out, hipStream_t stream);

/* Q/K RMSNorm over the full hidden width followed by axial RoPE, in place
 * ("Difflet Engineering Report", Wan attention head sharding and global RMS:
 * one sum of squares over the whole projection).  For every token row r of
 * qkv (bf16, row stride `row_stride`, q at column 0, k at column `hidden`):
 *   q <- RoPE(q / sqrt(mean(q^2) + eps) * g_q),  k likewise with g_k.
 * RoPE: head_dim splits into [rope_t | rope_h | rope_w] dims; pair (2j, 2j+1)
 * of axis a turns by pos_a * theta^(-2j / rope_a).  Token i of a batch row
 * (i = r mod (n_vis + n_txt)) is visual when i < n_vis = grid_t*grid_h*grid_w,
 * at t = i / (grid_h*grid_w), h = (i / grid_w) % grid_h, w = i % grid_w;
 * text tokens sit at (0,0,0), i.e. are not rotated.  Descriptor fields used:
 * attn.{batch,n_vis,n_txt,heads,head_dim}, hidden, grid_*, rope_*,
 * rope_theta, rms_eps. */
typedef struct dit_block_desc {
  dit_attn_desc attn;
  int32_t hidden;  /* == heads * head_dim, multiple of 64 */
  int32_t mlp;     /* MLP width, multiple of 64            */
  int32_t grid_t, grid_h, grid_w; /* n_vis == grid_t * grid_h * grid_w     */
  int32_t rope_t, rope_h, rope_w; /* even, rope_t+rope_h+rope_w == head_dim */
  float rope_theta, ln_eps, rms_eps;
  int64_t mod_stride; /* elements between batch rows of `mod`; 0 = shared */
} dit_block_desc;

dit_status dit_qk_rmsnorm_rope(const dit_block_desc* desc, uint16_t* qkv,
                               int64_t row_stride, const uint16_t* g_q,
                               const uint16_t* g_k, hipStream_t stream);

/* Weights of one block, bf16, [out, in] with `in` contiguous. */
typedef struct dit_block_weights {
  const uint16_t *w_qkv, *b_qkv; /* [3D, D], [3D] : q, k, v column blocks */
  const uint16_t *g_q, *g_k;     /* [D] RMSNorm gains                     */
  const uint16_t *w_o, *b_o;     /* [D, D], [D]                           */
  const uint16_t *w_up, *b_up;   /* [F, D], [F]                           */
  const uint16_t *w_dn, *b_dn;   /* [D, F], [D]                           */
} dit_block_weights;

/* Bytes of device workspace dit_block_forward needs for `desc` (0 on a bad
 * descriptor). */
size_t dit_block_workspace_bytes(const dit_block_desc* desc);

/* One DiT block, in place on the residual stream x (fp32 [B, N, D], N =
 * n_vis + n_txt, visual tokens first):
 *   h  = adaLN(x; shift1, scale1)
 *   q,k,v = h W_qkv^T + b_qkv;  q,k <- RoPE(RMSNorm_D(.) * g)
 *   o  = joint_attention(q, k, v; n_vis + txt_valid[b])
 *   x  = x + gate1 * (o W_o^T + b_o)
 *   h2 = adaLN(x; shift2, scale2)
 *   x  = x + gate2 * (GELU(h2 W_up^T + b_up) W_dn^T + b_dn)
 * mod: bf16 [B, 6, D] = (shift1, scale1, gate1, shift2, scale2, gate2) per
 * batch row, row stride desc->mod_stride (0 = one vector for all rows).
 * Activations h, qkv, o, h2 and the MLP hidden are bf16 in `workspace`
 * (>= dit_block_workspace_bytes(desc), 256-byte aligned); the residual stream
 * stays fp32.  For B * N >= 1024 the workspace also holds the 64 MiB of
 * scratch the GEMMs use to split an under-filled last round of tiles along K
 * (see dit_linear); the double, single and Wan blocks' workspaces do the
 * same. */
dit_status dit_block_forward(const dit_block_desc* desc,
                             const dit_block_weights* w, const uint16_t* mod,
                             float* x, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Classifier-free guidance and one flow-matching Euler step on the fp32
 * latent ("Difflet", section 3: the scheduler turns the predicted velocity
 * into a less noisy latent; "Difflet Engineering Report", Video output
 * corrections: scheduler state stays fp32):
 *   v = v_uncond + guidance * (v_cond - v_uncond)   (v = v_cond if v_uncond
 *                                                    is NULL)
 *   x = x + (sigma_next - sigma) * v
 * x fp32 [n]; v_cond, v_uncond bf16 [n]; n >= 0. */
dit_status dit_euler_step(float* x, const uint16_t* v_cond,
                          const uint16_t* v_uncond, int64_t n, float guidance,
                          float sigma, float sigma_next, hipStream_t stream);

/* Sinusoidal timestep features: for t = t_scale * sigma[s] and
 * f_j = 10000^(-j/(dim/2)), out[s, :] = [cos(t f), sin(t f)] (bf16 [n, dim]).
 * sigma: fp32 device [n]; dim even, 2..4096. */
dit_status dit_timestep_features(const float* sigma, int32_t n, int32_t dim,
                                 float t_scale, uint16_t* out,
                                 hipStream_t stream);

/* Strided casts used around the block stack (loop glue).
 * f32 -> bf16: out[r*ld_out + c] = bf16(in[r*ld_in + c]) for r < rows, c < cols
 * bf16 -> f32: the reverse.  cols % 4 == 0, ld_* % 4 == 0. */
dit_status dit_cast_f32_bf16(const float* in, int64_t ld_in, int64_t rows,
                             int32_t cols, uint16_t* out, int64_t ld_out,
                             hipStream_t stream);
dit_status dit_cast_bf16_f32(const uint16_t* in, int64_t ld_in, int64_t rows,
                             int32_t cols, float* out, int64_t ld_out,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * One denoising step of a DiT stack (loop glue + blocks + sampler).
 *
 * The denoiser predicts a velocity from the latent, the timestep and the text
 * conditioning; the scheduler moves the latent to the next noise level
 * ("Difflet", section 3; "19. Diffusion, Image, Video, and World Models",
 * Follow the diffusion pipeline).  Steps, in order, all on `stream`:
 *   f    = sinusoidal(t_scale * sigma, freq_dim)                (bf16 [1, F])
 *   c    = SiLU(f W_t1^T + b_t1);  s = SiLU(c W_t2^T + b_t2)    (bf16 [1, D])
 *   for l < depth:  mod_l = s W_mod[l]^T + b_mod[l]  (bf16 [6, D], shared by
 *                   every batch row);  (shift, scale) = s W_fin^T + b_fin
 *                   (all depend on s alone and are computed here, before
 *                   the input projection)
 *   x[b, :n_vis]  = bf16(latent[lb]) W_in^T + b_in              (fp32)
 *   x[b, n_vis:]  = text[b]                                     (fp32)
 *   for l < depth:  dit_block_forward(x; mod_l)
 *   h = adaLN(x; shift, scale)
 *   v[b] = h[b, :n_vis] W_out^T + b_out                         (bf16)
 *   latent += (sigma_next - sigma) * v        (cfg == 0: each row its own
 *             latent, lb = b), or with cfg == 1 (batch == 2, row 0
 *             conditional, row 1 unconditional, one latent, lb = 0):
 *   latent += (sigma_next - sigma) * (v[1] + guidance * (v[0] - v[1])).
 * Descriptor: block is as for dit_block_forward (block.mod_stride is
 * ignored); latent_channels % 8 == 0; freq_dim % 64 == 0.
 * latent: fp32 [cfg ? 1 : batch, n_vis, latent_channels], updated in place.
 * Workspace: >= dit_denoise_workspace_bytes(desc), 256-byte aligned. */
typedef struct dit_model_desc {
  dit_block_desc block;
  int32_t depth;
  int32_t latent_channels;
  int32_t freq_dim;
  int32_t cfg;
  float t_scale;
} dit_model_desc;

typedef struct dit_model_weights {
  const uint16_t *t_w1, *t_b1;       /* [D, freq_dim], [D]   */
  const uint16_t *t_w2, *t_b2;       /* [D, D], [D]          */
  const uint16_t *in_w, *in_b;       /* [D, C], [D]          */
  const uint16_t *fin_w, *fin_b;     /* [2D, D], [2D]: shift then scale */
  const uint16_t *out_w, *out_b;     /* [C, D], [C]          */
  const uint16_t* text;              /* [batch, n_txt, D] conditioning tokens */
  const dit_block_weights* blocks;   /* HOST array [depth] of device pointers */
  const uint16_t* const* mod_w;      /* HOST array [depth]: device [6D, D] */
  const uint16_t* const* mod_b;      /* HOST array [depth]: device [6D]    */
} dit_model_weights;

size_t dit_denoise_workspace_bytes(const dit_model_desc* desc);
dit_status dit_denoise_step(const dit_model_desc* desc, const dit_model_weights* w,
                            float* latent, float sigma, float sigma_next,
                            float guidance, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * MM-DiT blocks ("ChunkFlow", Appendix B, Per-Block Compute Model: DiT and
 * MM-DiT, equations (13)-(22)).  Same kernels as dit_block_forward, other
 * operand routing.  Descriptor as dit_block_forward (attn.n_vis = S image
 * tokens on the grid, attn.n_txt = L text slots with txt_valid[b] valid,
 * mod_stride = elements between the batch rows of a modulation tensor, 0 to
 * share one).  x streams fp32, updated in place; weights bf16 [out, in].
 *
 * Double-stream block: the image stream x_img [B, S, D] and the text stream
 * x_txt [B, L, D] each have their own weights (w_img, w_txt: the DiT block's
 * set) and modulation (mod_img, mod_txt: [B, 6, D], shift1, scale1, gate1,
 * shift2, scale2, gate2).  Per stream: h = adaLN(x; shift1, scale1),
 * q|k|v = h W_qkv^T + b_qkv, q^ = RoPE(RMSNorm_D(q) g_q), k^ likewise (the
 * stream's own gains; image tokens at their grid position, text at 0).  One
 * joint attention over [image; text] with keys [0, S + txt_valid[b]); then
 * per stream x += gate1 (o W_o^T + b_o) and
 * x += gate2 (GELU(adaLN(x; shift2, scale2) W_up^T + b_up) W_dn^T + b_dn).
 * Workspace >= dit_double_block_workspace_bytes (= the DiT block's for the
 * same descriptor), 256-byte aligned.  x_txt may be NULL when L == 0. */
size_t dit_double_block_workspace_bytes(const dit_block_desc* desc);
dit_status dit_double_block_forward(const dit_block_desc* desc,
                                    const dit_block_weights* w_img,
                                    const dit_block_weights* w_txt,
                                    const uint16_t* mod_img, const uint16_t* mod_txt,
                                    float* x_img, float* x_txt, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Single-stream block on the joint stream x [B, S + L, D] (image tokens
 * first): mod [B, 3, D] = (shift, scale, gate);
 *   h = adaLN(x; shift, scale)
 *   [q | k | v | up] = h w1^T + b1            w1 [3D + F, D], b1 [3D + F]
 *   q^, k^ = RoPE(RMSNorm_D(q) g_q), RoPE(RMSNorm_D(k) g_k)
 *   o = joint attention, keys [0, S + txt_valid[b])
 *   x += gate ([o | GELU(up)] w2^T + b2)      w2 [D, D + F], b2 [D]
 * Workspace >= dit_single_block_workspace_bytes, 256-byte aligned. */
typedef struct dit_single_block_weights {
  const uint16_t *w1, *b1, *g_q, *g_k, *w2, *b2;
} dit_single_block_weights;
size_t dit_single_block_workspace_bytes(const dit_block_desc* desc);
dit_status dit_single_block_forward(const dit_block_desc* desc,
                                    const dit_single_block_weights* w,
                                    const uint16_t* mod, float* x, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Wan-style block ("ChunkFlow", Appendix B, equations (7)-(12)): self-
 * attention over the video tokens, cross-attention to the text context, MLP.
 * Descriptor as dit_block_forward, read as: attn.n_vis = S video tokens on
 * the grid (the self-attention sequence), attn.n_txt = L context slots of
 * which txt_valid[b] are valid (the cross-attention keys [0, txt_valid[b])).
 *   x    fp32 [B, S, D], in place;  ctx bf16 [B, L, D] (may be NULL if L == 0)
 *   mod  bf16 [B, 6, D] (shift1, scale1, gate1, shift2, scale2, gate2), batch
 *        rows mod_stride apart (0 = shared)
 *   h  = adaLN(x; shift1, scale1);  q|k|v = h W_qkv^T + b_qkv;
 *   q^, k^ = RoPE(RMSNorm_D(.) g_q / g_k) at the grid positions;
 *   x += gate1 (SelfAttn(q^, k^, v) W_o^T + b_o)
 *   c  = LN(x) (no affine);  qc = RMSNorm_D(c W_cq^T + b_cq) g_cq;
 *   kc|vc = ctx W_ckv^T + b_ckv (w_ckv [2D, D]: key rows, then value rows);
 *   kc = RMSNorm_D(kc) g_ck;  x += CrossAttn(qc, kc, vc) W_co^T + b_co
 *        (no RoPE; a row with no valid context token attends to nothing: 0)
 *   x += gate2 (GELU(adaLN(x; shift2, scale2) W_up^T + b_up) W_dn^T + b_dn)
 * Workspace >= dit_wan_block_workspace_bytes, 256-byte aligned. */
typedef struct dit_wan_block_weights {
  const uint16_t *w_qkv, *b_qkv, *g_q, *g_k, *w_o, *b_o;
  const uint16_t *w_cq, *b_cq, *w_ckv, *b_ckv, *g_cq, *g_ck, *w_co, *b_co;
  const uint16_t *w_up, *b_up, *w_dn, *b_dn;
} dit_wan_block_weights;
size_t dit_wan_block_workspace_bytes(const dit_block_desc* desc);
dit_status dit_wan_block_forward(const dit_block_desc* desc, const dit_wan_block_weights* w,
                                 const uint16_t* mod, float* x, const uint16_t* ctx,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Step caching ("Difflet", section 5 Adaptive Step Caching on Trainium;
 * "Difflet Engineering Report", DiT caching: adaptive TeaCache, online delta,
 * and fixed cadence; "19. Diffusion, Image, Video, and World Models", Inside
 * TeaCache's skip decision).
 *
 * Nearby steps give similar denoiser outputs, so some full denoiser calls are
 * replaced by an estimate.  The device side keeps two fp32 arrays the size of
 * the velocity -- prev_v (the previously used velocity, possibly an estimate)
 * and delta_v (the most recently measured change) -- and reports one fp32
 * change score per call; the decision to skip is taken on the host by a
 * controller (dit_cache_ctrl_*) from those scores.  The relative L1 change of
 * cur against prev is sum|cur - prev| / sum|prev| (0 if both sums are 0,
 * +inf if only the reference sum is 0). */

typedef enum dit_dtype { DIT_DTYPE_BF16 = 0, DIT_DTYPE_F32 = 1 } dit_dtype;

/* Relative L1 change of cur against prev (n >= 1 elements of `dtype`),
 * written to *score (fp32, device).  With update = 1, prev <- cur in the same
 * pass (cur and prev must not overlap then).  The sum is deterministic: a
 * fixed partition of the elements that depends on n alone, fp32 partial sums,
 * a final sum in double.  cur, prev and workspace 16-byte aligned; workspace
 * >= dit_change_score_workspace_bytes() (partial sums; caller-owned).
 * 1 <= n <= DIT_CHANGE_SCORE_MAX_N. */
#define DIT_CHANGE_SCORE_MAX_N (INT64_C(1) << 40)
size_t dit_change_score_workspace_bytes(void);
dit_status dit_change_score(const void* cur, void* prev, int32_t dtype, int64_t n,
                            int32_t update, float* score, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* dit_change_score without a workspace, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, result and errors as
 * dit_change_score; the partial sums (DIT_CHANGE_SCORE_SCRATCH_BYTES = 8 KiB,
 * enough for any n up to DIT_CHANGE_SCORE_MAX_N) live in a static device
 * array of the library, one per GPU, held until the process ends; its
 * address is looked up on the first call on each device.  No allocation of
 * any kind.  All calls on one GPU share that array: calls whose executions
 * overlap on one GPU (e.g. on two streams) race and must be ordered by the
 * caller.  n > DIT_CHANGE_SCORE_MAX_N -> DIT_EINVAL. */
#define DIT_CHANGE_SCORE_SCRATCH_BYTES 8192
dit_status dit_change_score_noalloc(const void* cur, void* prev, int32_t dtype, int64_t n,
                                    int32_t update, float* score, hipStream_t stream);

/* The probe of calibrated adaptive caching: the change of block 0's modulated
 * input between this call and the previous one.  Runs the step's timestep
 * conditioning and input tokens (as dit_denoise_step), layer 0's modulation
 * and its first adaLN, h = LN(x) (1 + scale1) + shift1 for every token
 * (bf16 [batch, n_vis + n_txt, hidden]); then *score = relative L1 change of
 * h against `saved` and saved <- h.  have_saved = 0 (no previous features)
 * copies h into saved and writes *score = +inf, which forces a full step in
 * any threshold controller.  Only layer 0's block and modulation weights are
 * read.  Workspace as dit_denoise_step. */
dit_status dit_cache_probe(const dit_model_desc* desc, const dit_model_weights* w,
                           const float* latent, float sigma, uint16_t* saved,
                           int32_t have_saved, float* score, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* One denoising step under step caching.  With v the guided velocity of the
 * step (v_uncond + g (v_cond - v_uncond) with cfg, else the prediction):
 *   DIT_STEP_FULL: run the denoiser exactly as dit_denoise_step; if have_prev,
 *                  delta_v = v - prev_v and *score = relative L1 change of v
 *                  against prev_v (else *score = +inf); prev_v = v;
 *                  latent += (sigma_next - sigma) v
 *   DIT_STEP_SKIP: no denoiser call; v = prev_v + delta_v; prev_v = v;
 *                  latent += (sigma_next - sigma) v   (needs have_prev = 1:
 *                  two completed full steps; *score untouched)
 * prev_v, delta_v: fp32 [cfg ? 1 : batch, n_vis, latent_channels], 16-byte
 * aligned, caller-owned state of one generation; score nullable. */
typedef enum dit_step_action { DIT_STEP_FULL = 0, DIT_STEP_SKIP = 1 } dit_step_action;
dit_status dit_denoise_step_cached(const dit_model_desc* desc, const dit_model_weights* w,
                                   float* latent, float sigma, float sigma_next,
                                   float guidance, int32_t action, int32_t have_prev,
                                   float* prev_v, float* delta_v, float* score,
                                   void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* The host controller (no device work, no allocation; the struct is caller
 * state for one generation).  Steps are decided in order 0 .. n_steps-1.
 * Step i is always computed when i < warmup, i >= n_steps - cooldown, or
 * fewer than two full steps have completed.  Otherwise:
 *   DIT_CACHE_OFF           never skips;
 *   DIT_CACHE_CADENCE       skips unless (i - warmup) is a multiple of cadence;
 *   DIT_CACHE_ONLINE_DELTA  skips when the last full step's output change
 *                           (dit_cache_ctrl_observe) was below alpha times the
 *                           first output change of the generation and the
 *                           step before was not skipped;
 *   DIT_CACHE_TEACACHE      adds poly(probe_score) (coefficients coef[0..n_coef),
 *                           highest degree first) to an accumulator and skips
 *                           while it stays below threshold; every full step
 *                           resets it; a non-finite probe score computes.
 * Arithmetic is double, without fused multiply-adds. */
typedef enum dit_cache_mode {
  DIT_CACHE_OFF = 0,
  DIT_CACHE_CADENCE = 1,
  DIT_CACHE_ONLINE_DELTA = 2,
  DIT_CACHE_TEACACHE = 3
} dit_cache_mode;
#define DIT_CACHE_MAX_COEF 8
typedef struct dit_cache_policy {
  int32_t mode, n_steps, warmup, cooldown, cadence;
  int32_t n_coef;
  double alpha, threshold;
  double coef[DIT_CACHE_MAX_COEF];
} dit_cache_policy;
typedef struct dit_cache_ctrl {
  dit_cache_policy policy;
  int32_t next_step, n_full, last_skipped, skip_next, have_first;
  double first_change, acc;
} dit_cache_ctrl;
dit_status dit_cache_ctrl_init(dit_cache_ctrl* c, const dit_cache_policy* p);
/* *action = DIT_STEP_FULL or DIT_STEP_SKIP for `step`; probe_score is read
 * in DIT_CACHE_TEACACHE mode only (pass the probe's score of this step). */
dit_status dit_cache_ctrl_decide(dit_cache_ctrl* c, int32_t step, float probe_score,
                                 int32_t* action);
/* After a full step: the output change it measured (online-delta only;
 * non-finite values are ignored). */
dit_status dit_cache_ctrl_observe(dit_cache_ctrl* c, float output_change);

/* Debug: the integer (t, h, w) position of every token of one batch row,
 * int32 [n_vis + n_txt, 3] (device), from the same device code RoPE uses. */
dit_status dit_debug_positions(const dit_block_desc* desc, int32_t* out,
                               hipStream_t stream);

const char* dit_status_string(dit_status s);
const char* dit_last_error(void); /* thread-local; "" after DIT_OK */
const char* dit_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H_ */
