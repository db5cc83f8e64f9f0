// Sampler-side kernels (gfx950): classifier-free guidance fused with the
// flow-matching Euler update on the fp32 latent, sinusoidal timestep
// features, and the strided casts that move tokens between the fp32 latent /
// residual stream and bf16 GEMM operands.
#include "common.h"
#include "kernels.h"

namespace dit {
namespace {

// x += dt * (vu + g (vc - vu)); vu == nullptr means no guidance (v = vc).
// Four elements per thread: 16-byte x and 8-byte v accesses.
__global__ void euler_kernel(float* __restrict__ x, const uint16_t* __restrict__ vc,
                             const uint16_t* __restrict__ vu, int64_t n, float g, float dt) {
  const int64_t i0 = 4 * (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
  if (i0 >= n) return;
  if (i0 + 3 < n) {
    f32x4 xv = *reinterpret_cast<const f32x4*>(x + i0);
    const u32x2 c2 = *reinterpret_cast<const u32x2*>(vc + i0);
    float c[4] = {__uint_as_float(c2[0] << 16), __uint_as_float(c2[0] & 0xffff0000u),
                  __uint_as_float(c2[1] << 16), __uint_as_float(c2[1] & 0xffff0000u)};
    if (vu) {
      const u32x2 u2 = *reinterpret_cast<const u32x2*>(vu + i0);
      const float u[4] = {__uint_as_float(u2[0] << 16), __uint_as_float(u2[0] & 0xffff0000u),
                          __uint_as_float(u2[1] << 16), __uint_as_float(u2[1] & 0xffff0000u)};
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = u[e] + g * (c[e] - u[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) xv[e] += dt * c[e];
    *reinterpret_cast<f32x4*>(x + i0) = xv;
  } else {
    for (int64_t i = i0; i < n; ++i) {
      float v = bf16_to_f32(vc[i]);
      if (vu) {
        const float u = bf16_to_f32(vu[i]);
        v = u + g * (v - u);
      }
      x[i] += dt * v;
    }
  }
}

// sigma == nullptr: a single row for the scalar sigma0.
__global__ void timestep_kernel(const float* __restrict__ sigma, float sigma0, int n, int dim,
                                float t_scale, uint16_t* __restrict__ out) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * dim) return;
  const int s = idx / dim, j = idx % dim;
  const int half = dim / 2;
  const int jj = j < half ? j : j - half;
  const float f = expf(-9.210340371976184f * static_cast<float>(jj) / static_cast<float>(half));
  const float a = t_scale * (sigma ? sigma[s] : sigma0) * f;
  out[idx] = f32_to_bf16(j < half ? cosf(a) : sinf(a));
}

__global__ void cast_f32_bf16_kernel(const float* __restrict__ in, int64_t ld_in, int64_t rows,
                                     int cols, uint16_t* __restrict__ out, int64_t ld_out) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int per_row = cols / 4;
  if (q >= rows * per_row) return;
  const int64_t r = q / per_row;
  const int c = 4 * static_cast<int>(q % per_row);
  const f32x4 v = *reinterpret_cast<const f32x4*>(in + r * ld_in + c);
  u32x2 w;
  w[0] = pack_bf16x2(v[0], v[1]);
  w[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(out + r * ld_out + c) = w;
}

__global__ void cast_bf16_f32_kernel(const uint16_t* __restrict__ in, int64_t ld_in, int64_t rows,
                                     int cols, float* __restrict__ out, int64_t ld_out) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int per_row = cols / 4;
  if (q >= rows * per_row) return;
  const int64_t r = q / per_row;
  const int c = 4 * static_cast<int>(q % per_row);
  const u32x2 w = *reinterpret_cast<const u32x2*>(in + r * ld_in + c);
  f32x4 v;
  v[0] = __uint_as_float(w[0] << 16);
  v[1] = __uint_as_float(w[0] & 0xffff0000u);
  v[2] = __uint_as_float(w[1] << 16);
  v[3] = __uint_as_float(w[1] & 0xffff0000u);
  *reinterpret_cast<f32x4*>(out + r * ld_out + c) = v;
}

inline unsigned blocks_for(int64_t work, int threads) {
  return static_cast<unsigned>((work + threads - 1) / threads);
}

}  // namespace

hipError_t launch_euler(float* x, const uint16_t* vc, const uint16_t* vu, int64_t n, float g,
                        float dt, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(euler_kernel, dim3(blocks_for((n + 3) / 4, 256)), dim3(256), 0, s, x, vc, vu,
                     n, g, dt);
  return hipGetLastError();
}

hipError_t launch_timestep_features(const float* sigma, float sigma0, int n, int dim,
                                    float t_scale, uint16_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(timestep_kernel, dim3(blocks_for(static_cast<int64_t>(n) * dim, 256)),
                     dim3(256), 0, s, sigma, sigma0, n, dim, t_scale, out);
  return hipGetLastError();
}

hipError_t launch_cast_f32_bf16(const float* in, int64_t ld_in, int64_t rows, int cols,
                                uint16_t* out, int64_t ld_out, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  hipLaunchKernelGGL(cast_f32_bf16_kernel, dim3(blocks_for(rows * (cols / 4), 256)), dim3(256), 0,
                     s, in, ld_in, rows, cols, out, ld_out);
  return hipGetLastError();
}

hipError_t launch_cast_bf16_f32(const uint16_t* in, int64_t ld_in, int64_t rows, int cols,
                                float* out, int64_t ld_out, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  hipLaunchKernelGGL(cast_bf16_f32_kernel, dim3(blocks_for(rows * (cols / 4), 256)), dim3(256), 0,
                     s, in, ld_in, rows, cols, out, ld_out);
  return hipGetLastError();
}

}  // namespace dit
