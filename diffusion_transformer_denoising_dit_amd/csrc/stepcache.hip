// Step-caching kernels (gfx950): the relative L1 change score of two arrays
// ("19. Diffusion, Image, Video, and World Models", Inside TeaCache's skip
// decision: mean|cur - prev| / mean|prev|), optionally replacing the saved
// array by the current one in the same pass ("Difflet", section 5: the probe
// compares and updates its saved features within one call and returns one
// scalar), and the sampler side of the output estimator ("Difflet", section
// 5: a full step measures its output's change against the previously used
// output and saves both; a cached step moves the latent with previous output
// plus saved change).
//
// All of it is HBM-bound streaming.  Sums are deterministic: a fixed grid of
// at most kScoreBlocks workgroups, each thread owning a fixed set of 8-element
// chunks, a fixed reduction tree inside the workgroup, per-workgroup partials
// in a small workspace and one final workgroup adding them in double.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum of (a, b) over the workgroup; the result is valid in thread 0.
__device__ __forceinline__ void block_sum2(float& a, float& b) {
  __shared__ float red[2][kThreads / kWave];
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) {
    red[0][w] = a;
    red[1][w] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a = red[0][0];
    b = red[1][0];
#pragma unroll
    for (int i = 1; i < kThreads / kWave; ++i) {
      a += red[0][i];
      b += red[1][i];
    }
  }
}

template <bool kBf16>
__device__ __forceinline__ void load8(const void* p, int64_t i, float* f) {
  if constexpr (kBf16) {
    unpack8(*reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p) + i), f);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = a[e];
      f[4 + e] = b[e];
    }
  }
}

template <bool kBf16>
__device__ __forceinline__ void store8(void* p, int64_t i, const float* f) {
  if constexpr (kBf16) {
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p) + i) = pack8(f);
  } else {
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = f[e];
      b[e] = f[4 + e];
    }
    *reinterpret_cast<f32x4*>(static_cast<float*>(p) + i) = a;
    *reinterpret_cast<f32x4*>(static_cast<float*>(p) + i + 4) = b;
  }
}

template <bool kBf16>
__device__ __forceinline__ float load1(const void* p, int64_t i) {
  if constexpr (kBf16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// Per-workgroup sums of |cur - prev| and |prev|; with kUpdate, prev <- cur
// (each element is read and then written by the same thread).  Chunk c of 8
// elements belongs to thread c mod (grid * kThreads); the n mod 8 tail
// elements to the first threads of workgroup 0.
template <bool kBf16, bool kUpdate>
__global__ __launch_bounds__(kThreads) void change_partials_kernel(const void* __restrict__ cur,
                                                                   void* __restrict__ prev,
                                                                   int64_t n,
                                                                   float* __restrict__ partials) {
  float num = 0.f, den = 0.f;
  const int64_t n8 = n / 8;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; c < n8; c += stride) {
    float a[8], p[8];
    load8<kBf16>(cur, 8 * c, a);
    load8<kBf16>(prev, 8 * c, p);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      num += fabsf(a[e] - p[e]);
      den += fabsf(p[e]);
    }
    if constexpr (kUpdate) store8<kBf16>(prev, 8 * c, a);
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 8 * n8) {
    const int64_t i = 8 * n8 + threadIdx.x;
    const float a = load1<kBf16>(cur, i), p = load1<kBf16>(prev, i);
    num += fabsf(a - p);
    den += fabsf(p);
    if constexpr (kUpdate) {
      if constexpr (kBf16) static_cast<uint16_t*>(prev)[i] = static_cast<const uint16_t*>(cur)[i];
      else static_cast<float*>(prev)[i] = a;
    }
  }
  block_sum2(num, den);
  if (threadIdx.x == 0) {
    partials[2 * blockIdx.x] = num;
    partials[2 * blockIdx.x + 1] = den;
  }
}

// score = sum num / sum den over the partials (double, fixed order); a zero
// denominator gives 0 when the numerator is 0 too, else +inf.  valid == 0
// writes +inf (nothing to compare with).
__global__ __launch_bounds__(kThreads) void change_final_kernel(const float* __restrict__ partials,
                                                                int n_parts, int valid,
                                                                float* __restrict__ score) {
  __shared__ double red[2][kThreads];
  double a = 0.0, b = 0.0;
  for (int i = threadIdx.x; i < n_parts; i += kThreads) {
    a += partials[2 * i];
    b += partials[2 * i + 1];
  }
  red[0][threadIdx.x] = a;
  red[1][threadIdx.x] = b;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      red[0][threadIdx.x] += red[0][threadIdx.x + s];
      red[1][threadIdx.x] += red[1][threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double num = red[0][0], den = red[1][0];
    float r;
    if (!valid) r = INFINITY;
    else if (den == 0.0) r = num == 0.0 ? 0.f : INFINITY;
    else r = static_cast<float>(num / den);
    score[0] = r;
  }
}

// The sampler side of the output estimator on n fp32 elements.
//   full (kSkip false): v = vu + g (vc - vu) (v = vc without guidance);
//     with have_prev: delta = v - prev and the sums of |v - prev|, |prev|;
//     prev = v;  x += dt v
//   skip (kSkip true):  v = prev + delta;  prev = v;  x += dt v
// Four elements per thread and chunk; chunk c belongs to thread
// c mod (grid * kThreads), the n mod 4 tail to workgroup 0.
template <bool kSkip>
__device__ __forceinline__ void velocity_elem(float& xv, float c, float u, bool has_u, float g,
                                              float dt, float& pv, float& dv, bool have_prev,
                                              float& num, float& den) {
  float v;
  if constexpr (kSkip) {
    v = pv + dv;
  } else {
    v = has_u ? u + g * (c - u) : c;
    if (have_prev) {
      const float d = v - pv;
      num += fabsf(d);
      den += fabsf(pv);
      dv = d;
    }
  }
  pv = v;
  xv += dt * v;
}

template <bool kSkip>
__global__ __launch_bounds__(kThreads) void cached_velocity_kernel(
    float* __restrict__ x, const uint16_t* __restrict__ vc, const uint16_t* __restrict__ vu,
    int64_t n, float g, float dt, float* __restrict__ prev, float* __restrict__ delta,
    int have_prev, float* __restrict__ partials) {
  float num = 0.f, den = 0.f;
  const bool has_u = vu != nullptr;
  const int64_t n4 = n / 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; c < n4; c += stride) {
    const int64_t i = 4 * c;
    const f32x4 x4 = *reinterpret_cast<const f32x4*>(x + i);
    const f32x4 p4 = *reinterpret_cast<const f32x4*>(prev + i);
    float xv[4], pv[4], dv[4] = {0.f, 0.f, 0.f, 0.f};
    float cv[4] = {0.f, 0.f, 0.f, 0.f}, uv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xv[e] = x4[e];
      pv[e] = p4[e];
    }
    if constexpr (kSkip) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(delta + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) dv[e] = d4[e];
    } else {
      const u32x2 c2 = *reinterpret_cast<const u32x2*>(vc + i);
      cv[0] = __uint_as_float(c2[0] << 16);
      cv[1] = __uint_as_float(c2[0] & 0xffff0000u);
      cv[2] = __uint_as_float(c2[1] << 16);
      cv[3] = __uint_as_float(c2[1] & 0xffff0000u);
      if (has_u) {
        const u32x2 u2 = *reinterpret_cast<const u32x2*>(vu + i);
        uv[0] = __uint_as_float(u2[0] << 16);
        uv[1] = __uint_as_float(u2[0] & 0xffff0000u);
        uv[2] = __uint_as_float(u2[1] << 16);
        uv[3] = __uint_as_float(u2[1] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      velocity_elem<kSkip>(xv[e], cv[e], uv[e], has_u, g, dt, pv[e], dv[e], have_prev, num, den);
    f32x4 xo, po, dout;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xo[e] = xv[e];
      po[e] = pv[e];
      dout[e] = dv[e];
    }
    *reinterpret_cast<f32x4*>(x + i) = xo;
    *reinterpret_cast<f32x4*>(prev + i) = po;
    if constexpr (!kSkip) {
      if (have_prev) *reinterpret_cast<f32x4*>(delta + i) = dout;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 4 * n4) {
    const int64_t i = 4 * n4 + threadIdx.x;
    float xv = x[i], pv = prev[i], dv = kSkip ? delta[i] : 0.f;
    const float cv = kSkip ? 0.f : bf16_to_f32(vc[i]);
    const float uv = (!kSkip && has_u) ? bf16_to_f32(vu[i]) : 0.f;
    velocity_elem<kSkip>(xv, cv, uv, has_u, g, dt, pv, dv, have_prev, num, den);
    x[i] = xv;
    prev[i] = pv;
    if (!kSkip && have_prev) delta[i] = dv;
  }
  if constexpr (!kSkip) {
    block_sum2(num, den);
    if (threadIdx.x == 0 && partials) {
      partials[2 * blockIdx.x] = num;
      partials[2 * blockIdx.x + 1] = den;
    }
  }
}

// Workgroups of a streaming pass over n elements in chunks of `per`: enough
// to cover every chunk once up to kScoreBlocks, a function of n alone.
int stream_blocks(int64_t n, int per) {
  const int64_t chunks = (n + per - 1) / per;
  const int64_t b = (chunks + kThreads - 1) / kThreads;
  return static_cast<int>(b < 1 ? 1 : (b > kScoreBlocks ? kScoreBlocks : b));
}

}  // namespace

hipError_t launch_change_score(const void* cur, void* prev, bool bf16, int64_t n, bool update,
                               float* partials, float* score, hipStream_t s) {
  const int blocks = stream_blocks(n, 8);
  if (bf16 && update)
    hipLaunchKernelGGL((change_partials_kernel<true, true>), dim3(blocks), dim3(kThreads), 0, s, cur, prev, n, partials);
  else if (bf16)
    hipLaunchKernelGGL((change_partials_kernel<true, false>), dim3(blocks), dim3(kThreads), 0, s, cur, prev, n, partials);
  else if (update)
    hipLaunchKernelGGL((change_partials_kernel<false, true>), dim3(blocks), dim3(kThreads), 0, s, cur, prev, n, partials);
  else
    hipLaunchKernelGGL((change_partials_kernel<false, false>), dim3(blocks), dim3(kThreads), 0, s, cur, prev, n, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(change_final_kernel, dim3(1), dim3(kThreads), 0, s, partials, blocks, 1, score);
  return hipGetLastError();
}

// Partial sums of the change score for callers that cannot allocate: a
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host that name
// is a stand-in, not a device address); it passes the address
// hipGetSymbolAddress returns for the current device, looked up once per
// device on its first use and kept.  Every call on one GPU shares that
// GPU's array: calls that overlap in time on one GPU race.
static __device__ __align__(256) float scratch[2 * kScoreBlocks];
static_assert(sizeof(scratch) == kScorePartialBytes, "scratch holds one pass's partial sums");

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t change_score_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_score_invalid(float* partials, float* score, hipStream_t s) {
  hipLaunchKernelGGL(change_final_kernel, dim3(1), dim3(kThreads), 0, s, partials, 0, 0, score);
  return hipGetLastError();
}

hipError_t launch_cached_velocity(float* x, const uint16_t* vc, const uint16_t* vu, int64_t n,
                                  float g, float dt, float* prev, float* delta, bool skip,
                                  bool have_prev, float* partials, float* score, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = stream_blocks(n, 4);
  if (skip) {
    hipLaunchKernelGGL(cached_velocity_kernel<true>, dim3(blocks), dim3(kThreads), 0, s, x, vc, vu,
                       n, g, dt, prev, delta, 1, nullptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(cached_velocity_kernel<false>, dim3(blocks), dim3(kThreads), 0, s, x, vc, vu,
                     n, g, dt, prev, delta, have_prev ? 1 : 0, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !score) return e;
  hipLaunchKernelGGL(change_final_kernel, dim3(1), dim3(kThreads), 0, s, partials,
                     have_prev ? blocks : 0, have_prev ? 1 : 0, score);
  return hipGetLastError();
}

}  // namespace dit
