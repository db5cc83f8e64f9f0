// Internal launchers of the gfx950 kernels (host side).  Arguments are
// already validated by the C ABI layer in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

struct GemmParams {
  const uint16_t* a;
  int64_t lda;
  const uint16_t* w;
  const uint16_t* bias;
  int64_t m;
  int n, k;
  void* out;
  int64_t ldc;
  const uint16_t* gate;
  int64_t gate_stride, gate_rows;
  int64_t group_rows, a_group_stride, c_group_stride;
  // Optional fp32 scratch for splitting the last, partly filled round of
  // large-GEMM tiles along K (null: no split).  kSplitWsBytes at least.
  float* split_ws;
};
// Scratch for the K-split tail of the large GEMM: up to kMaxSplitParts
// partial 256 x 256 fp32 tiles.
constexpr int kMaxSplitParts = 256;
constexpr size_t kSplitWsBytes = static_cast<size_t>(kMaxSplitParts) * 256 * 256 * 4;
hipError_t launch_gemm(const GemmParams& p, int epilogue, hipStream_t s);
// Compute units of the current device (cached per device; 0 if unknown):
// the launchers size their last-round splits by it.
int compute_units();

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t q_stride;   // elements between query tokens
  int64_t kv_stride;  // elements between key / value tokens
  int64_t q_batch;    // elements between batch rows of q
  int64_t kv_batch;   // elements between batch rows of k and v
  void* out;          // bf16, or fp32 if out_f32: row (b, i) at out + (b*n_q + i)*out_stride
  int64_t out_stride;
  int out_f32;
  float* lse;         // nullable, fp32 [batch, heads, n_q]
  int n_q, n_k, heads, head_dim, batch;
  int n_valid[8];     // valid keys of batch row b: [0, n_valid[b]), n_valid[b] <= n_k
  float scale_log2;   // softmax scale * log2(e)
  // Optional scratch (nullable, bf16 output only) for the split of an
  // under-filled last round of query tiles along the keys; at least
  // kAttnTailWsBytes, 256-byte aligned.
  float* tail_ws;
  // Set by launch_attention: workgroups [0, wg_main) take whole key ranges;
  // each of the remaining query tiles is split into tail_parts key ranges
  // whose fp32 partials (tail_o, tail_lse) a second kernel merges.
  int wg_main, tail_parts;
  float* tail_o;
  float* tail_lse;
};
// Scratch of the split last round: at most kAttnMaxTailTiles partial tiles
// of 256 query rows, head_dim <= 128 fp32 values and one log-denominator each.
constexpr int kAttnMaxTailParts = 4;
constexpr int kAttnMaxTailTiles = 448;
constexpr size_t kAttnTailWsBytes = static_cast<size_t>(kAttnMaxTailTiles) * 256 * (128 + 1) * 4;
static_assert(kAttnTailWsBytes <= kSplitWsBytes, "the block workspaces' split scratch serves both");
hipError_t launch_attention(const AttnParams& p, hipStream_t s);

struct MergeParams {
  const float* outs[32];
  const float* lses[32];
  int parts;
  int64_t part_stride;  // fp32 elements between rows of a partial output
  uint16_t* out;
  int64_t out_stride;
  float* lse_out;       // nullable
  int batch, n_q, heads, head_dim;
};
hipError_t launch_attention_merge(const MergeParams& p, hipStream_t s);

hipError_t launch_adaln(const float* x, int64_t rows, int hidden, int64_t rows_per_batch,
                        const uint16_t* shift, const uint16_t* scale, int64_t mod_stride,
                        float eps, uint16_t* out, hipStream_t s);

struct RopeParams {
  uint16_t* qkv;
  int64_t row_stride;
  const uint16_t* g_q;
  const uint16_t* g_k;
  int64_t rows;
  int n_tok, n_vis, hidden, head_dim;
  int grid_h, grid_w;
  int rope_t, rope_h, rope_w;
  float theta, eps;
  int q_only;  // normalise only the q half (columns [0, hidden)) of each row
};
hipError_t launch_qk_rmsnorm_rope(const RopeParams& p, hipStream_t s);
hipError_t launch_positions(const RopeParams& p, int32_t* out, hipStream_t s);

hipError_t launch_euler(float* x, const uint16_t* vc, const uint16_t* vu, int64_t n, float g,
                        float dt, hipStream_t s);

// Step caching.  Streaming passes use at most kScoreBlocks workgroups, each
// leaving two fp32 partial sums in `partials` (kScorePartialBytes).
constexpr int kScoreBlocks = 1024;
constexpr size_t kScorePartialBytes = 2 * kScoreBlocks * sizeof(float);
// score = sum|cur - prev| / sum|prev| (bf16 or fp32 arrays of n elements);
// with update, prev <- cur in the same pass.
hipError_t launch_change_score(const void* cur, void* prev, bool bf16, int64_t n, bool update,
                               float* partials, float* score, hipStream_t s);
// Device address of the library's own partial-sum array on the current
// device (kScorePartialBytes; shared by every call on that device).
hipError_t change_score_scratch(float** out);
// score = +inf (nothing to compare with).
hipError_t launch_score_invalid(float* partials, float* score, hipStream_t s);
// Full step (skip false): v = guided velocity, delta = v - prev and the change
// score when have_prev, prev = v, x += dt v.  Skip: v = prev + delta,
// prev = v, x += dt v.  score may be null (not computed).
hipError_t launch_cached_velocity(float* x, const uint16_t* vc, const uint16_t* vu, int64_t n,
                                  float g, float dt, float* prev, float* delta, bool skip,
                                  bool have_prev, float* partials, float* score, hipStream_t s);
hipError_t launch_timestep_features(const float* sigma, float sigma0, int n, int dim,
                                    float t_scale, uint16_t* out, hipStream_t s);
hipError_t launch_cast_f32_bf16(const float* in, int64_t ld_in, int64_t rows, int cols,
                                uint16_t* out, int64_t ld_out, hipStream_t s);
hipError_t launch_cast_bf16_f32(const uint16_t* in, int64_t ld_in, int64_t rows, int cols,
                                float* out, int64_t ld_out, hipStream_t s);

}  // namespace dit
