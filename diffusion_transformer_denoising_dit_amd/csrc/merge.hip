// Merge of split joint-attention partials ("Difflet", section 4.3): each
// partial was normalised by its own softmax denominator, so the partials are
// weighted by exp(lse_p - M) (M the largest lse), added and divided by the
// sum of the weights.  Memory-bound: every output element reads one fp32
// element of each partial; a thread handles 4 consecutive features of one
// (batch row, query, head) with 16-byte reads and an 8-byte bf16 store.
#include "common.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
  const int quads = p.head_dim / 4;                        // threads per (row, head)
  const int64_t per_row = static_cast<int64_t>(p.heads) * quads;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= static_cast<int64_t>(p.batch) * p.n_q * per_row) return;
  const int64_t row = t / per_row;                         // b * n_q + i
  const int h = static_cast<int>((t % per_row) / quads);
  const int e0 = static_cast<int>(t % quads) * 4;
  const int64_t b = row / p.n_q, i = row % p.n_q;
  const int64_t lse_idx = (b * p.heads + h) * p.n_q + i;
  const int64_t col = static_cast<int64_t>(h) * p.head_dim + e0;

  float m = -INFINITY;
  for (int q = 0; q < p.parts; ++q) m = fmaxf(m, p.lses[q][lse_idx]);
  if (m == -INFINITY) {
    // every partial is empty (no valid key in any partition): the empty sum,
    // weighted output 0 and log-denominator -inf, as an empty partial gives
    const u32x2 z = {0u, 0u};
    *reinterpret_cast<u32x2*>(p.out + row * p.out_stride + col) = z;
    if (p.lse_out && e0 == 0) p.lse_out[lse_idx] = -INFINITY;
    return;
  }
  float den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < p.parts; ++q) {
    const float w = expf(p.lses[q][lse_idx] - m);
    const f32x4 o = *reinterpret_cast<const f32x4*>(p.outs[q] + row * p.part_stride + col);
    den += w;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, o[e], acc[e]);
  }
  const float inv = 1.f / den;
  u32x2 w2;
  w2[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w2[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(p.out + row * p.out_stride + col) = w2;
  if (p.lse_out && e0 == 0) p.lse_out[lse_idx] = m + logf(den);
}

}  // namespace

hipError_t launch_attention_merge(const MergeParams& p, hipStream_t s) {
  const int64_t threads = static_cast<int64_t>(p.batch) * p.n_q * p.heads * (p.head_dim / 4);
  if (threads == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((threads + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dit
