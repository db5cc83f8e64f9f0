// Bandwidth-bound per-token kernels of the DiT block (gfx950):
//  * adaLN: LayerNorm of the fp32 residual stream with timestep modulation,
//    written as the bf16 input of the next GEMM ("Difflet Engineering
//    Report", Terms used in this report: AdaLN);
//  * Q/K RMSNorm over the full hidden width plus axial RoPE, in place on the
//    QKV buffer ("Difflet Engineering Report", Wan attention head sharding
//    and global RMS: one sum of squares over the whole projection).
// One workgroup per token row; every thread keeps its slice of the row in
// registers between the reduction and the write, so each element is read once
// and written once with 16-byte accesses.
#include "common.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int kThreads = 256;

template <int NV>  // float4 vectors per thread: hidden <= 1024 * NV
__global__ __launch_bounds__(kThreads) void adaln_kernel(const float* __restrict__ x, int hidden,
                                                         int64_t rows_per_batch,
                                                         const uint16_t* __restrict__ shift,
                                                         const uint16_t* __restrict__ scale,
                                                         int64_t mod_stride, float eps,
                                                         uint16_t* __restrict__ out) {
  __shared__ float red[kThreads / kWave];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvec = hidden / 4;
  const float* row = x + r * hidden;
  f32x4 v[NV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + i * kThreads;
    if (c < nvec) {
      v[i] = *reinterpret_cast<const f32x4*>(row + 4 * c);
      s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
    }
  }
  const float mean = block_sum<kThreads>(s, red) / hidden;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + i * kThreads;
    if (c < nvec) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = v[i][e] - mean;
        q += d * d;
      }
    }
  }
  const float var = block_sum<kThreads>(q, red) / hidden;
  const float rstd = 1.f / sqrtf(var + eps);
  const int64_t b = r / rows_per_batch;
  const bool modulated = shift != nullptr;  // else a plain LayerNorm (shift = scale = 0)
  const uint16_t* sh = shift + b * mod_stride;
  const uint16_t* sc = scale + b * mod_stride;
  uint16_t* orow = out + r * hidden;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + i * kThreads;
    if (c < nvec) {
      u32x2 s2 = {0u, 0u}, c2 = {0u, 0u};
      if (modulated) {
        s2 = *reinterpret_cast<const u32x2*>(sh + 4 * c);
        c2 = *reinterpret_cast<const u32x2*>(sc + 4 * c);
      }
      const float shf[4] = {__uint_as_float(s2[0] << 16), __uint_as_float(s2[0] & 0xffff0000u),
                            __uint_as_float(s2[1] << 16), __uint_as_float(s2[1] & 0xffff0000u)};
      const float scf[4] = {__uint_as_float(c2[0] << 16), __uint_as_float(c2[0] & 0xffff0000u),
                            __uint_as_float(c2[1] << 16), __uint_as_float(c2[1] & 0xffff0000u)};
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (v[i][e] - mean) * rstd * (1.f + scf[e]) + shf[e];
      u32x2 w;
      w[0] = pack_bf16x2(y[0], y[1]);
      w[1] = pack_bf16x2(y[2], y[3]);
      *reinterpret_cast<u32x2*>(orow + 4 * c) = w;
    }
  }
}

// Integer (t, h, w) position of token i of a batch row; text tokens at 0.
__device__ __forceinline__ void token_pos(int i, int n_vis, int gh, int gw, int* pos) {
  if (i < n_vis) {
    pos[0] = i / (gh * gw);
    pos[1] = (i / gw) % gh;
    pos[2] = i % gw;
  } else {
    pos[0] = pos[1] = pos[2] = 0;
  }
}

template <int NV>  // 16-byte chunks per thread over the q and k halves: 2*hidden <= 2048*NV
__global__ __launch_bounds__(kThreads) void qk_rmsnorm_rope_kernel(RopeParams p) {
  __shared__ float red[kThreads / kWave];
  __shared__ float cs[2 * 128];  // cos, sin of each rotation pair of a head (head_dim <= 256)
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int half = p.head_dim / 2;

  if (tid < half) {
    int pos[3];
    token_pos(static_cast<int>(r % p.n_tok), p.n_vis, p.grid_h, p.grid_w, pos);
    // pair tid of a head: which axis block it lies in and its index there
    int axis, j, da;
    const int e2 = 2 * tid;
    if (e2 < p.rope_t) {
      axis = 0; j = tid; da = p.rope_t;
    } else if (e2 < p.rope_t + p.rope_h) {
      axis = 1; j = tid - p.rope_t / 2; da = p.rope_h;
    } else {
      axis = 2; j = tid - (p.rope_t + p.rope_h) / 2; da = p.rope_w;
    }
    const float inv_freq = powf(p.theta, -2.f * static_cast<float>(j) / static_cast<float>(da));
    const float ang = static_cast<float>(pos[axis]) * inv_freq;
    float sn, cn;
    sincosf(ang, &sn, &cn);
    cs[2 * tid] = cn;
    cs[2 * tid + 1] = sn;
  }

  const int nq = p.hidden / 8;  // chunks in the q half; the k half follows
  const int nc = p.q_only ? nq : 2 * nq;
  uint16_t* row = p.qkv + r * p.row_stride;
  u32x4 v[NV];
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + i * kThreads;
    if (c < nc) {
      const int col = c < nq ? 8 * c : p.hidden + 8 * (c - nq);
      v[i] = *reinterpret_cast<const u32x4*>(row + col);
      float f[8];
      unpack8(v[i], f);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a += f[e] * f[e];
      if (c < nq) sq += a; else sk += a;
    }
  }
  const float tq = block_sum<kThreads>(sq, red);
  const float tk = block_sum<kThreads>(sk, red);  // also orders the cs[] writes before use
  const float rq = 1.f / sqrtf(tq / p.hidden + p.eps);
  const float rk = 1.f / sqrtf(tk / p.hidden + p.eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + i * kThreads;
    if (c < nc) {
      const bool isq = c < nq;
      const int cin = isq ? 8 * c : 8 * (c - nq);  // column within the q or k half
      const uint16_t* g = (isq ? p.g_q : p.g_k) + cin;
      const float rs = isq ? rq : rk;
      float f[8], gf[8];
      unpack8(v[i], f);
      unpack8(*reinterpret_cast<const u32x4*>(g), gf);
      const int pair0 = (cin % p.head_dim) / 2;
      float y[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = f[2 * e] * rs * gf[2 * e];
        const float x1 = f[2 * e + 1] * rs * gf[2 * e + 1];
        const float cn = cs[2 * (pair0 + e)], sn = cs[2 * (pair0 + e) + 1];
        y[2 * e] = x0 * cn - x1 * sn;
        y[2 * e + 1] = x0 * sn + x1 * cn;
      }
      const int col = isq ? cin : p.hidden + cin;
      *reinterpret_cast<u32x4*>(row + col) = pack8(y);
    }
  }
}

__global__ void positions_kernel(RopeParams p, int32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.n_tok) return;
  int pos[3];
  token_pos(i, p.n_vis, p.grid_h, p.grid_w, pos);
  out[3 * i] = pos[0];
  out[3 * i + 1] = pos[1];
  out[3 * i + 2] = pos[2];
}

}  // namespace

hipError_t launch_adaln(const float* x, int64_t rows, int hidden, int64_t rows_per_batch,
                        const uint16_t* shift, const uint16_t* scale, int64_t mod_stride,
                        float eps, uint16_t* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int nv = (hidden / 4 + kThreads - 1) / kThreads;
  dim3 grid(static_cast<unsigned>(rows));
#define DIT_ADALN(NV_)                                                                  \
  case NV_:                                                                             \
    hipLaunchKernelGGL(adaln_kernel<NV_>, grid, dim3(kThreads), 0, s, x, hidden,        \
                       rows_per_batch, shift, scale, mod_stride, eps, out);             \
    break;
  switch (nv) {
    DIT_ADALN(1) DIT_ADALN(2) DIT_ADALN(3) DIT_ADALN(4) DIT_ADALN(5) DIT_ADALN(6)
    DIT_ADALN(7) DIT_ADALN(8) DIT_ADALN(9) DIT_ADALN(10) DIT_ADALN(11) DIT_ADALN(12)
    DIT_ADALN(13) DIT_ADALN(14) DIT_ADALN(15) DIT_ADALN(16)
    default: return hipErrorInvalidValue;
  }
#undef DIT_ADALN
  return hipGetLastError();
}

hipError_t launch_qk_rmsnorm_rope(const RopeParams& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  const int nv = (2 * (p.hidden / 8) + kThreads - 1) / kThreads;
  dim3 grid(static_cast<unsigned>(p.rows));
#define DIT_ROPE(NV_)                                                                       \
  case NV_:                                                                                 \
    hipLaunchKernelGGL(qk_rmsnorm_rope_kernel<NV_>, grid, dim3(kThreads), 0, s, p);         \
    break;
  switch (nv) {
    DIT_ROPE(1) DIT_ROPE(2) DIT_ROPE(3) DIT_ROPE(4) DIT_ROPE(5) DIT_ROPE(6) DIT_ROPE(7)
    DIT_ROPE(8) DIT_ROPE(9) DIT_ROPE(10) DIT_ROPE(11) DIT_ROPE(12) DIT_ROPE(13)
    DIT_ROPE(14) DIT_ROPE(15) DIT_ROPE(16)
    default: return hipErrorInvalidValue;
  }
#undef DIT_ROPE
  return hipGetLastError();
}

hipError_t launch_positions(const RopeParams& p, int32_t* out, hipStream_t s) {
  if (p.n_tok == 0) return hipSuccess;
  hipLaunchKernelGGL(positions_kernel, dim3((p.n_tok + 255) / 256), dim3(256), 0, s, p, out);
  return hipGetLastError();
}

}  // namespace dit
