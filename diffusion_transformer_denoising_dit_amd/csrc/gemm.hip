// Linear layers of the DiT block on bf16 MFMA (gfx950): y = A W^T + bias with
// the surrounding elementwise work fused into the store -- GELU, SiLU, or the
// gated residual x += gate * y on the fp32 residual stream.  These are the
// projection and MLP terms of "ChunkFlow" Appendix B, equations (13) and (16).
//
// Tiling: a workgroup of 4 waves computes a 128 (W rows, n) x 256 (A rows, m)
// tile of C^T; each wave owns 64 x 128 = 2 x 4 MFMA 32x32 tiles.  The MFMA is
// fed W as its A operand and the activations as its B operand, so each lane
// ends up holding 4 consecutive output features of one token row: bias, gate
// and residual loads and the stores are 8- or 16-byte vectors.  K is staged
// through LDS 64 at a time (rows padded by 16 bytes so the 16-byte operand
// reads of a wave fall in distinct banks); the next K slice is fetched into
// registers while the current one is multiplied.
#include "common.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int kTN = 128;  // W rows (output features) per workgroup
constexpr int kTM = 256;  // A rows (tokens) per workgroup
constexpr int kBK = 64;
constexpr int kLd = kBK + 8;  // padded LDS row (elements)
constexpr int kThreads = 256;
constexpr int kAChunks = kTM * kBK / 8 / kThreads;  // 16-byte chunks per thread: 8
constexpr int kWChunks = kTN * kBK / 8 / kThreads;  // 4

enum { EPI_BF16 = 0, EPI_GELU = 1, EPI_SILU = 2, EPI_F32 = 3, EPI_GATED = 4 };

__device__ __forceinline__ int64_t a_row_offset(const GemmParams& p, int64_t r) {
  return p.group_rows > 0 ? (r / p.group_rows) * p.a_group_stride + (r % p.group_rows) * p.lda
                          : r * p.lda;
}
__device__ __forceinline__ int64_t c_row_offset(const GemmParams& p, int64_t r) {
  return p.group_rows > 0 ? (r / p.group_rows) * p.c_group_stride + (r % p.group_rows) * p.ldc
                          : r * p.ldc;
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[kTM * kLd];
  __shared__ __attribute__((aligned(16))) uint16_t sW[kTN * kLd];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wn = wave & 1;   // wave's 64-row half of the W tile
  const int wm = wave >> 1;  // wave's 128-row half of the A tile
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kTM;
  const int n0 = blockIdx.x * kTN;

  // global -> register staging: chunk column and the rows this thread loads
  const int cc = tid % 8;
  const int rr = tid / 8;  // 0..31
  const uint16_t* a_src[kAChunks];
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    int64_t r = m0 + rr + 32 * i;
    if (r > p.m - 1) r = p.m - 1;  // clamp: rows past m are computed, never stored
    a_src[i] = p.a + a_row_offset(p, r) + cc * 8;
  }
  const uint16_t* w_src[kWChunks];
#pragma unroll
  for (int i = 0; i < kWChunks; ++i) {
    int r = n0 + rr + 32 * i;
    if (r > p.n - 1) r = p.n - 1;
    w_src[i] = p.w + static_cast<int64_t>(r) * p.k + cc * 8;
  }

  u32x4 ra[kAChunks], rw[kWChunks];
  auto fetch = [&](int kt) {
    const int64_t ko = static_cast<int64_t>(kt) * kBK;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + ko);
#pragma unroll
    for (int i = 0; i < kWChunks; ++i) rw[i] = *reinterpret_cast<const u32x4*>(w_src[i] + ko);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int kTiles = p.k / kBK;
  fetch(0);
  const int fr = lane % 32;       // operand row within a 32-row MFMA tile
  const int fk = 8 * (lane / 32);  // operand k offset within a 16-wide k step

  for (int kt = 0; kt < kTiles; ++kt) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kAChunks; ++i)
      *reinterpret_cast<u32x4*>(&sA[(rr + 32 * i) * kLd + cc * 8]) = ra[i];
#pragma unroll
    for (int i = 0; i < kWChunks; ++i)
      *reinterpret_cast<u32x4*>(&sW[(rr + 32 * i) * kLd + cc * 8]) = rw[i];
    __syncthreads();
    if (kt + 1 < kTiles) fetch(kt + 1);

#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 wf[2], af[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        wf[i] = *reinterpret_cast<const bf16x8*>(
            &sW[(wn * 64 + i * 32 + fr) * kLd + ks * 16 + fk]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        af[j] = *reinterpret_cast<const bf16x8*>(
            &sA[(wm * 128 + j * 32 + fr) * kLd + ks * 16 + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(wf[i], af[j], acc[i][j]);
    }
  }

  // Epilogue.  acc[i][j][4*g + e] is C[m, n] with
  //   m = m0 + wm*128 + j*32 + lane%32,  n = n0 + wn*64 + i*32 + 8*g + 4*(lane/32) + e.
  const int hi = lane / 32;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = m0 + wm * 128 + j * 32 + (lane % 32);
    if (m >= p.m) continue;
    const int64_t crow = c_row_offset(p, m);
    const uint16_t* grow = nullptr;
    if (EPI == EPI_GATED) grow = p.gate + (m / p.gate_rows) * p.gate_stride;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 64 + i * 32 + 8 * g + 4 * hi;
        if (n >= p.n) continue;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * g + e];
        if (p.bias) {
          const u32x2 bb = *reinterpret_cast<const u32x2*>(p.bias + n);
          y[0] += __uint_as_float(bb[0] << 16);
          y[1] += __uint_as_float(bb[0] & 0xffff0000u);
          y[2] += __uint_as_float(bb[1] << 16);
          y[3] += __uint_as_float(bb[1] & 0xffff0000u);
        }
        if (EPI == EPI_GELU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = 0.5f * y[e] * (1.f + erff(y[e] * 0.70710678118654752f));
        } else if (EPI == EPI_SILU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = y[e] / (1.f + expf(-y[e]));
        }
        if (EPI == EPI_F32 || EPI == EPI_GATED) {
          float* dst = static_cast<float*>(p.out) + crow + n;
          f32x4 o;
          if (EPI == EPI_GATED) {
            o = *reinterpret_cast<const f32x4*>(dst);
            const u32x2 gg = *reinterpret_cast<const u32x2*>(grow + n);
            o[0] += __uint_as_float(gg[0] << 16) * y[0];
            o[1] += __uint_as_float(gg[0] & 0xffff0000u) * y[1];
            o[2] += __uint_as_float(gg[1] << 16) * y[2];
            o[3] += __uint_as_float(gg[1] & 0xffff0000u) * y[3];
          } else {
            o[0] = y[0]; o[1] = y[1]; o[2] = y[2]; o[3] = y[3];
          }
          *reinterpret_cast<f32x4*>(dst) = o;
        } else {
          uint16_t* dst = static_cast<uint16_t*>(p.out) + crow + n;
          u32x2 o;
          o[0] = pack_bf16x2(y[0], y[1]);
          o[1] = pack_bf16x2(y[2], y[3]);
          *reinterpret_cast<u32x2*>(dst) = o;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, int epilogue, hipStream_t s) {
  if (p.m == 0) return hipSuccess;
  dim3 grid((p.n + kTN - 1) / kTN, static_cast<unsigned>((p.m + kTM - 1) / kTM));
  dim3 block(kThreads);
  switch (epilogue) {
    case EPI_BF16: hipLaunchKernelGGL(gemm_kernel<EPI_BF16>, grid, block, 0, s, p); break;
    case EPI_GELU: hipLaunchKernelGGL(gemm_kernel<EPI_GELU>, grid, block, 0, s, p); break;
    case EPI_SILU: hipLaunchKernelGGL(gemm_kernel<EPI_SILU>, grid, block, 0, s, p); break;
    case EPI_F32: hipLaunchKernelGGL(gemm_kernel<EPI_F32>, grid, block, 0, s, p); break;
    case EPI_GATED: hipLaunchKernelGGL(gemm_kernel<EPI_GATED>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dit
