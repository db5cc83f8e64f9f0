// Joint attention over [visual; text] tokens on bf16 MFMA (gfx950).
//
// Each query attends to the visual and the valid text keys of its batch row
// under one softmax ("Difflet", section 4).  Padded text keys sit after the
// valid ones, so the valid keys are the interval [0, n_vis + L_b) and only two
// numbers per row decide the mask ("Difflet", section 4.2 Representing
// Attention Mask): key tiles past the bound are never visited, and only the
// one tile that straddles it is masked.
//
// The design point of the Trainium kernel the pages describe (128-query tiles,
// scores kept on chip, probabilities transposed before the value product) is
// kept; its mechanics are re-done for CDNA4:
//  * a workgroup of 4 waves owns 128 queries of one (batch row, head); each
//    wave owns 32 queries whose Q fragments stay in registers;
//  * scores are produced transposed, S^T = K Q^T, with K as the MFMA A operand
//    (32x32x16, bf16 in, fp32 out).  Every lane then holds 16 scores of ONE
//    query, so the softmax row statistics need a single cross-lane exchange
//    (lane l <-> l^32) and no transpose of P is needed: the fp32 scores, once
//    exponentiated and rounded to bf16, are already laid out as the B operand
//    of O^T = V^T P^T.  The key order inside each 16-key MFMA step is permuted
//    identically in both operands, which leaves the sum unchanged;
//  * K tiles are staged row-major and V tiles transposed (V^T, d-major) in LDS,
//    64 keys at a time, with the next tile prefetched into registers while the
//    current one is multiplied;
//  * the softmax runs in the log2 domain: scores are scaled by
//    scale*log2(e) and exponentiated with v_exp_f32; the running max and sum
//    are fp32; the output is divided by the sum once at the end.
#include "common.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int kBM = 128;  // queries per workgroup (32 per wave)
constexpr int kBN = 64;   // keys per tile
constexpr int kThreads = 256;
constexpr int kVtLd = kBN + 4;  // V^T row (keys) padded: 136 B rows -> conflict-free 8 B reads

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnParams p) {
  constexpr int kKLd = D + 8;        // K row padded by 16 B
  constexpr int kCpr = D / 8;        // 16-byte chunks per K/V row
  constexpr int kRowsPerPass = kThreads / kCpr;
  constexpr int kKPasses = kBN / kRowsPerPass;
  constexpr int kVPasses = kCpr * kBN / kThreads;
  constexpr int kDB = D / 32;        // 32-wide d blocks of O^T
  constexpr int kKS = D / 16;        // 16-wide k steps of Q K^T

  __shared__ __attribute__((aligned(16))) uint16_t sK[kBN * kKLd];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * kVtLd];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int hi = lane / 32;
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int n_tok = p.n_tok;
  const int n_valid = p.n_valid[b];
  const int64_t base = static_cast<int64_t>(b) * n_tok * p.qkv_stride + h * D;

  // Q fragments: lane holds Q[q][16*ks + 8*hi .. +7] for its query q.
  const int q_row = blockIdx.x * kBM + wave * 32 + lane % 32;
  const int q_ld = q_row < n_tok ? q_row : n_tok - 1;
  bf16x8 qf[kKS];
  {
    const uint16_t* src = p.q + base + static_cast<int64_t>(q_ld) * p.qkv_stride + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
  }

  // K load mapping: consecutive threads read consecutive chunks of one row.
  const int kc = tid % kCpr;
  const int kr = tid / kCpr;
  // V load mapping: a wave covers 64 keys of one chunk, so the transposed
  // 2-byte LDS writes of a wave land on one contiguous V^T row segment.
  const int vk = tid % kBN;
  const int vc = tid / kBN;

  u32x4 rk[kKPasses], rv[kVPasses];
  auto fetch = [&](int j0) {
#pragma unroll
    for (int i = 0; i < kKPasses; ++i) {
      int key = j0 + kr + i * kRowsPerPass;
      key = key < n_tok ? key : n_tok - 1;
      rk[i] = *reinterpret_cast<const u32x4*>(p.k + base + static_cast<int64_t>(key) * p.qkv_stride + kc * 8);
    }
#pragma unroll
    for (int i = 0; i < kVPasses; ++i) {
      int key = j0 + vk;
      key = key < n_tok ? key : n_tok - 1;
      rv[i] = *reinterpret_cast<const u32x4*>(p.v + base + static_cast<int64_t>(key) * p.qkv_stride + (vc + i * (kThreads / kBN)) * 8);
    }
  };

  f32x16 o[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m_run = -INFINITY;  // running max of scaled (log2-domain) scores
  float l_run = 0.f;        // this lane's partial sum of exponentials

  const int n_tiles = (n_valid + kBN - 1) / kBN;  // fully padded tiles are skipped
  const float c = p.scale_log2;
  fetch(0);

  for (int jt = 0; jt < n_tiles; ++jt) {
    const int j0 = jt * kBN;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kKPasses; ++i)
      *reinterpret_cast<u32x4*>(&sK[(kr + i * kRowsPerPass) * kKLd + kc * 8]) = rk[i];
    {
      // V rows past the valid bound are written as zeros, so whatever the
      // padded slots hold (even Inf/NaN) cannot reach the output.
      const bool vvalid = j0 + vk < n_valid;
#pragma unroll
      for (int i = 0; i < kVPasses; ++i) {
        const int d0 = (vc + i * (kThreads / kBN)) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = vvalid ? rv[i][e] : 0u;
          sVt[(d0 + 2 * e) * kVtLd + vk] = static_cast<uint16_t>(w & 0xffffu);
          sVt[(d0 + 2 * e + 1) * kVtLd + vk] = static_cast<uint16_t>(w >> 16);
        }
      }
    }
    __syncthreads();
    if (jt + 1 < n_tiles) fetch(j0 + kBN);

    // S^T for two 32-key halves: s[t][4*g + e] is the score of
    // key j0 + 32*t + 8*g + 4*hi + e against this lane's query.
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[t][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            &sK[(32 * t + lane % 32) * kKLd + 16 * ks + 8 * hi]);
        s[t] = mfma32x32x16(kf, qf[ks], s[t]);
      }
    }

    // scale into the log2 domain; mask the tile that straddles the bound
    const bool boundary = j0 + kBN > n_valid;
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[t][r] * c;
        if (boundary) {
          const int key = j0 + 32 * t + 8 * (r / 4) + 4 * hi + (r % 4);
          v = key < n_valid ? v : -INFINITY;
        }
        s[t][r] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(s[t][r] - m_new);
        s[t][r] = e;
        ls += e;
      }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int i = 0; i < kDB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[i][e] *= alpha;

    // O^T += V^T P^T over four 16-key steps.  Step u covers keys
    // j0 + 16*u + [0, 16); its 16 k-slots are, for lane half hi,
    // keys 4*hi + {0..3} then 8 + 4*hi + {0..3} -- the order in which the
    // score accumulator already holds them.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = u / 2;
      const int g0 = 2 * (u % 2);
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[e] = static_cast<__bf16>(s[t][4 * g0 + e]);
        pf[4 + e] = static_cast<__bf16>(s[t][4 * (g0 + 1) + e]);
      }
      const int kb = 16 * u + 4 * hi;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const uint16_t* vrow = &sVt[(32 * db + lane % 32) * kVtLd];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + kb);
        const u32x2 hi8 = *reinterpret_cast<const u32x2*>(vrow + kb + 8);
        u32x4 vv;
        vv[0] = lo[0]; vv[1] = lo[1]; vv[2] = hi8[0]; vv[3] = hi8[1];
        o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8, vv), pf, o[db]);
      }
    }
  }

  // Combine the two lane halves' partial sums, normalise, store.
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (q_row < n_tok) {
    const float inv = 1.f / l_tot;
    uint16_t* dst = p.out + (static_cast<int64_t>(b) * n_tok + q_row) * p.out_stride + h * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
        w[1] = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(dst + 32 * db + 8 * g + 4 * hi) = w;
      }
    if (p.lse && hi == 0)
      p.lse[(static_cast<int64_t>(b) * p.heads + h) * n_tok + q_row] =
          m_run * 0.69314718055994531f + logf(l_tot);
  }
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  dim3 grid((p.n_tok + kBM - 1) / kBM, p.heads, p.batch);
  dim3 block(kThreads);
  if (p.head_dim == 128)
    hipLaunchKernelGGL(attn_kernel<128>, grid, block, 0, s, p);
  else if (p.head_dim == 64)
    hipLaunchKernelGGL(attn_kernel<64>, grid, block, 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dit
