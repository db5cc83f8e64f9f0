// Linear layers of the DiT block on bf16 MFMA (gfx950): y = A W^T + bias with
// the surrounding elementwise work fused into the store -- GELU, SiLU, or the
// gated residual x += gate * y on the fp32 residual stream.  These are the
// projection and MLP terms of "ChunkFlow" Appendix B, equations (13) and (16).
//
// In both kernels the MFMA is fed W as its A operand and the activations as
// its B operand, so each lane ends up holding 4 consecutive output features
// of one token row: bias, gate and residual loads and the stores are 8- or
// 16-byte vectors.
//
// Large GEMMs (the block's projections and MLP): a workgroup of 8 waves (two
// per SIMD) computes a 256 (tokens) x 256 (features) tile, each wave 128 x 64
// = 8 x 4 MFMA 16x16x32 tiles with the accumulators in registers.  The
// 16x16x32 shape does the same work per cycle as 32x32x16 but draws less
// power: under sustained load on every CU the shader clock settles ~12 %
// higher with it (1.88 against 1.68 GHz, register operands, same flops).
// A 256 x 256 tile moves 64 bytes of operands from L2 per 2 x 256 x 256
// flops, half of what a 128 x 256 tile needs, which keeps L2 below its
// bandwidth at full MFMA rate.  K slices of 64 stream from HBM/L2 straight
// into a 160 KB LDS ring with global_load_lds_dwordx4; each operand row of a slice
// is one full 128-byte line, stored unpadded with its 16-byte chunks
// XOR-swizzled by row so the operand reads of a wave hit distinct bank
// groups.  The two waves of a SIMD take turns: one multiplies a whole slice
// from registers while the other reads its next fragments from LDS (see the
// kernel).  Workgroups are ordered XCD by XCD (the dispatcher deals workgroup
// ids round-robin over the 8 XCDs, each with its own L2) and, inside an XCD,
// in groups of 8 token tiles that sweep all feature tiles, so the
// workgroups running together on one XCD share operand slices in its L2.
//
// Small GEMMs (input/output projection, the MM-DiT text stream, anything below
// the large kernel's shape): a workgroup of 4 waves computes a 128 (features)
// x 256 (tokens) tile, each wave 64 x 128; K is staged through padded LDS 64
// at a time, the next slice fetched into registers while the current one is
// multiplied.  Matrix-vector products (at most 8 token rows: the timestep MLP
// and the modulation projections) stream W once without tiles.
#include <algorithm>
#include <atomic>
#include <type_traits>

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

enum { EPI_BF16 = 0, EPI_GELU = 1, EPI_SILU = 2, EPI_F32 = 3, EPI_GATED = 4, EPI_RES = 5 };

// GELU in its exact form x * Phi(x) = x (1 + erf(x / sqrt 2)) / 2, with erf
// from the rational approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (after Hastings): for z >= 0,
// erf(z) = 1 - q(t) exp(-z^2), t = 1 / (1 + p z), q a degree-5 polynomial in
// t with no constant term, |error| <= 1.5e-7.  1 + erf(x / sqrt 2) is then
// 2 - q e for x >= 0 and q e for x < 0 (no cancellation in the negative
// tail).  About 12 branch-free VALU instructions per value; against exact
// GELU the fp32 result is within 5e-7 absolute, far below the bf16 rounding
// of the stored output.
__device__ __forceinline__ float gelu(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.f));
  float q = fmaf(t, 1.061405429f, -1.453152027f);
  q = fmaf(t, q, 1.421413741f);
  q = fmaf(t, q, -0.284496736f);
  q = fmaf(t, q, 0.254829592f);
  q *= t;
  const float qe = q * __builtin_amdgcn_exp2f(-(z * z) * 1.4426950408889634f);
  return 0.5f * x * (x >= 0.f ? 2.f - qe : qe);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int64_t a_row_offset(const GemmParams& p, int64_t r) {
  return p.group_rows > 0 ? (r / p.group_rows) * p.a_group_stride + (r % p.group_rows) * p.lda
                          : r * p.lda;
}
__device__ __forceinline__ int64_t c_row_offset(const GemmParams& p, int64_t r) {
  return p.group_rows > 0 ? (r / p.group_rows) * p.c_group_stride + (r % p.group_rows) * p.ldc
                          : r * p.ldc;
}

// Features n..n+3 of token row m (output row offset crow) from y[0..3], the
// bias already added: apply the epilogue and store (8-byte bf16 or 16-byte
// fp32 accesses).
template <int EPI>
__device__ __forceinline__ void store_row(const GemmParams& p, int64_t m, int64_t crow, int n, float (&y)[4]) {
  if (EPI == EPI_GELU) {
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = gelu(y[e]);
  } else if (EPI == EPI_SILU) {
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = y[e] / (1.f + expf(-y[e]));
  }
  if (EPI == EPI_F32 || EPI == EPI_GATED || EPI == EPI_RES) {
    float* dst = static_cast<float*>(p.out) + crow + n;
    f32x4 o;
    if (EPI == EPI_RES) {
      o = *reinterpret_cast<const f32x4*>(dst);
      o[0] += y[0]; o[1] += y[1]; o[2] += y[2]; o[3] += y[3];
    } else if (EPI == EPI_GATED) {
      const uint16_t* grow = p.gate + (m / p.gate_rows) * p.gate_stride;
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

// y[0..3] = acc for output features n..n+3 of token row m: add the bias, apply
// the epilogue and store.
template <int EPI>
__device__ __forceinline__ void store_epilogue(const GemmParams& p, int64_t m, int n, float (&y)[4]) {
  if (p.bias) {
    const u32x2 bb = *reinterpret_cast<const u32x2*>(p.bias + n);
    y[0] += __uint_as_float(bb[0] << 16);
    y[1] += __uint_as_float(bb[0] & 0xffff0000u);
    y[2] += __uint_as_float(bb[1] << 16);
    y[3] += __uint_as_float(bb[1] & 0xffff0000u);
  }
  store_row<EPI>(p, m, c_row_offset(p, m), n, y);
}

// The epilogue of one wave's 128 (tokens) x 64 (features) block of a
// 256 x 256 tile, acc[i][j][e] = C[m, n] with m = m_base + 16j + lane%16 and
// n = n_base + 16i + 4*(lane/16) + e.  The loads it needs are issued in
// batches before their uses -- the bias of all 4 feature groups once, then
// per kEpiRows 16-row blocks the residual (and gate) values of all of them
// (the operand registers of the main loop are free by now) -- so a batch
// costs one memory round trip rather than one per group.  p.n is a
// multiple of 8, so a lane's 4 features are all in range or all out.
template <int EPI, bool kChecked>
__device__ __forceinline__ void tile_epilogue_impl(const GemmParams& p, const f32x4 (&acc)[4][8],
                                                   int64_t m_base, int n_base, int lane) {
  constexpr bool kResid = EPI == EPI_GATED || EPI == EPI_RES;
  // 16-row blocks per batch (of 8); the gated residual's gate values would
  // not fit beside 4 blocks' residuals without spilling
  constexpr int kEpiRows = EPI == EPI_GATED ? 2 : 4;
  const int nq = 4 * (lane / 16);
  u32x2 bias[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) bias[i] = u32x2{0u, 0u};
  if (p.bias) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n_base + i * 16 + nq;
      if (!kChecked || n < p.n) bias[i] = *reinterpret_cast<const u32x2*>(p.bias + n);
    }
  }
#pragma unroll
  for (int jp = 0; jp < 8 / kEpiRows; ++jp) {
    int64_t crow[kEpiRows];
    bool row_ok[kEpiRows];
    f32x4 xr[kEpiRows][4];
    u32x2 gt[kEpiRows][4];
#pragma unroll
    for (int h = 0; h < kEpiRows; ++h) {
      const int64_t m = m_base + (kEpiRows * jp + h) * 16 + (lane % 16);
      row_ok[h] = !kChecked || m < p.m;
      crow[h] = c_row_offset(p, row_ok[h] ? m : 0);
      if constexpr (kResid) {
        const uint16_t* grow =
            EPI == EPI_GATED ? p.gate + ((row_ok[h] ? m : 0) / p.gate_rows) * p.gate_stride : nullptr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = n_base + i * 16 + nq;
          if (row_ok[h] && (!kChecked || n < p.n)) {
            xr[h][i] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.out) + crow[h] + n);
            if constexpr (EPI == EPI_GATED) gt[h][i] = *reinterpret_cast<const u32x2*>(grow + n);
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kEpiRows; ++h) {
      if (!row_ok[h]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n_base + i * 16 + nq;
        if (kChecked && n >= p.n) continue;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[i][kEpiRows * jp + h][e];
        y[0] += __uint_as_float(bias[i][0] << 16);
        y[1] += __uint_as_float(bias[i][0] & 0xffff0000u);
        y[2] += __uint_as_float(bias[i][1] << 16);
        y[3] += __uint_as_float(bias[i][1] & 0xffff0000u);
        if constexpr (EPI == EPI_GELU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = gelu(y[e]);
        } else if constexpr (EPI == EPI_SILU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = y[e] / (1.f + expf(-y[e]));
        }
        if constexpr (EPI == EPI_F32 || kResid) {
          f32x4 o;
          if constexpr (EPI == EPI_RES) {
            o = xr[h][i];
            o[0] += y[0]; o[1] += y[1]; o[2] += y[2]; o[3] += y[3];
          } else if constexpr (EPI == EPI_GATED) {
            o = xr[h][i];
            o[0] += __uint_as_float(gt[h][i][0] << 16) * y[0];
            o[1] += __uint_as_float(gt[h][i][0] & 0xffff0000u) * y[1];
            o[2] += __uint_as_float(gt[h][i][1] << 16) * y[2];
            o[3] += __uint_as_float(gt[h][i][1] & 0xffff0000u) * y[3];
          } else {
            o[0] = y[0]; o[1] = y[1]; o[2] = y[2]; o[3] = y[3];
          }
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + crow[h] + n) = o;
        } else {
          u32x2 o;
          o[0] = pack_bf16x2(y[0], y[1]);
          o[1] = pack_bf16x2(y[2], y[3]);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + crow[h] + n) = o;
        }
      }
    }
  }
}

// Interior blocks (every row and feature in range, the common case) take a
// branch-free path; edge blocks check each row and feature group.
template <int EPI>
__device__ __forceinline__ void tile_epilogue(const GemmParams& p, const f32x4 (&acc)[4][8],
                                              int64_t m_base, int n_base, int lane) {
  if (m_base + 128 <= p.m && n_base + 64 <= p.n)
    tile_epilogue_impl<EPI, false>(p, acc, m_base, n_base, lane);
  else
    tile_epilogue_impl<EPI, true>(p, acc, m_base, n_base, lane);
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
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 64 + i * 32 + 8 * g + 4 * hi;
        if (n >= p.n) continue;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * g + e];
        store_epilogue<EPI>(p, m, n, y);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large-GEMM kernel.
namespace big {

constexpr int kTM = 256;                          // token rows per workgroup
constexpr int kTN = 256;                          // output features per workgroup
constexpr int kBK = 64;                           // k per slice
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowBytes = 2 * kBK;                // 128: one operand row of a slice
constexpr int kChunks = kRowBytes / 16;           // 8 chunks of 16 bytes per row
constexpr int kRowsPerLoad = 1024 / kRowBytes;    // 8 rows per wave-wide 16 B/lane load
constexpr int kHalfBytes = 128 * kRowBytes;       // 16 KB: 128 rows of one slice
constexpr int kLoadsHalf = 128 / kRowsPerLoad / 4;  // 4 loads per wave fill 128 rows
// LDS ring: W slices in 3 stages (32 KB each); the A rows of each group (the
// 128 token rows it multiplies) in 2 stages of their own (16 KB each).
constexpr int kWStages = 3;
constexpr int kAStages = 2;
constexpr int kTileW = kTN * kRowBytes;
constexpr int kOffA = kWStages * kTileW;                    // A half h, stage t at kOffA + (2h + t) * kHalfBytes
constexpr int kLdsBytes = kOffA + 2 * kAStages * kHalfBytes;  // 160 KB
constexpr int kGroupM = 8;

// The grid of a large GEMM: `whole` workgroups of one whole tile each, then
// `parts` workgroups per each of the remaining tiles, each with a contiguous
// share of K (partials: fp32 scratch of parts * (tiles - whole) tiles).
struct SplitPlan {
  int whole, parts;
  float* partials;
};

// 16-byte chunk c of a 128-byte row r sits at chunk position c ^ swz(r).  LDS
// serves 16 bank groups of 16 bytes per clock; rows r and r+2 start in the
// same bank group, and swz separates the 16 rows one operand read touches.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Waits until at most 4 * items of this wave's loads are in flight.
__device__ __forceinline__ void wait_items(int items) {
  if (items <= 0) wait_vmcnt<0>();
  else if (items == 1) wait_vmcnt<kLoadsHalf>();
  else if (items == 2) wait_vmcnt<2 * kLoadsHalf>();
  else wait_vmcnt<3 * kLoadsHalf>();
}
// Waits until every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }

// Workgroup barrier that the compiler may not move memory operations or any
// other instruction across (the phases below depend on that placement).
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Wave-wide 16-byte-per-lane load into LDS: lane i's 16 bytes at base + voff
// (voff a 32-bit per-lane byte offset, base wave-uniform) land at LDS byte
// lds_addr + 16*i (lds_addr wave-uniform).  Issued from inline assembly so
// the compiler does not guard LDS reads with waits on it; M0 is saved and
// restored.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lds_addr)
      : "memory");
}

typedef __attribute__((address_space(3))) char* lds_char_ptr;

// The 8 waves form two groups, one wave of each per SIMD: group 0 (waves
// 0-3) multiplies token rows 0-127 of the tile, group 1 rows 128-255, each
// wave 128 tokens x 64 features.  A wave alternates a memory phase (read the
// 16 A and 8 W operand fragments of one 64-k slice from LDS into registers,
// and issue its share of later slices' loads) and an MFMA phase (the 64
// MFMAs of that slice), the second group one phase behind the first, with a
// workgroup barrier at every phase boundary: on each SIMD one wave
// multiplies while the other moves data.  Group 0 reads slice s in phase 2s,
// group 1 in phase 2s+1.
//
// Loads.  Each group issues, after the barrier that opens its memory phase,
// 4 wave-wide loads per wave of two 128-row pieces of later slices:
//   phase 2s   (group 0): A rows 128-255 of slice s+1 ("A1"), then W rows
//                         0-127 of slice s+2 ("W1")
//   phase 2s+1 (group 1): A rows 0-127 of slice s+2 ("A0"), then W rows
//                         128-255 of slice s+2 ("W2")
// W has three stages and each A half two, so every piece has 3 phases (W1:
// 4) between its issue and the barrier before its first reader -- a slot is
// refilled as soon as both of its readers are done with it.  Before a
// barrier a wave waits only for its own pieces that the next phase reads
// (loads complete in order, so "at most n in flight" names them).  The LDS
// ring fills all 160 KB of the CU.
// Tile t of the grouped order: groups of kGroupM token tiles that sweep all
// feature tiles, so the workgroups running together share operand slices.
__device__ __forceinline__ void tile_of(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group;
  const int first_m = g * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_g = t - g * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p, int tiles_m, int tiles_n,
                                                           SplitPlan sp) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave / 4, wq = wave % 4;

  // Tile of this workgroup.  The first sp.whole workgroups each take a whole
  // tile, their ids renumbered XCD-contiguously (the dispatcher deals ids
  // round-robin over the 8 XCDs, each with its own L2) before the grouped
  // order.  The remaining workgroups split each of the last tiles into
  // sp.parts contiguous K ranges and store fp32 partial tiles.
  int tm, tn, part = -1, tail = 0;
  int k_begin = 0, k_tiles = p.k / kBK;
  {
    const int id = blockIdx.x;
    if (id < sp.whole) {
      const int xcd = id % 8, slot = id / 8;
      const int q = sp.whole / 8, r = sp.whole % 8;
      tile_of(xcd * q + min(xcd, r) + slot, tiles_m, tiles_n, tm, tn);
    } else {
      tail = (id - sp.whole) / sp.parts;
      part = (id - sp.whole) % sp.parts;
      tile_of(sp.whole + tail, tiles_m, tiles_n, tm, tn);
      k_begin = part * k_tiles / sp.parts;
      k_tiles = (part + 1) * k_tiles / sp.parts - k_begin;
    }
  }
  const int64_t m0 = static_cast<int64_t>(tm) * kTM;
  const int n0 = tn * kTN;

  // This wave's loads: rows [(wq*4 + n) * 8, +8) of a 128-row piece; lane i
  // lands at row i / 8, chunk position i % 8 and fetches the chunk that
  // swizzles there.  Group 0 loads A rows 128-255 and W rows 0-127, group 1
  // A rows 0-127 and W rows 128-255.  Rows past m or n are clamped (computed,
  // never stored).  Byte offsets from p.a and p.w fit 32 bits (checked by the
  // launcher).
  const int a_half = 1 - grp, w_half = grp;
  uint32_t a_vo[kLoadsHalf], w_vo[kLoadsHalf];
#pragma unroll
  for (int n = 0; n < kLoadsHalf; ++n) {
    const int r = (wq * kLoadsHalf + n) * kRowsPerLoad + lane / kChunks;  // row within the piece
    const int c = (lane % kChunks) ^ swz(r);
    int64_t m = m0 + a_half * 128 + r;
    if (m > p.m - 1) m = p.m - 1;
    a_vo[n] = static_cast<uint32_t>(a_row_offset(p, m) * 2 + c * 16);
    const int nr = min(n0 + w_half * 128 + r, p.n - 1);
    w_vo[n] = static_cast<uint32_t>(static_cast<int64_t>(nr) * p.k * 2 + c * 16);
  }
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_ptr)smem));
  // A piece of slice kt (of this workgroup's K range) into its stage (dst is
  // that piece's first byte).
  auto issue_a = [&](int kt) {
    const uint32_t dst = lds_base + kOffA + (2 * a_half + kt % kAStages) * kHalfBytes;
    const char* src = reinterpret_cast<const char*>(p.a) + static_cast<int64_t>(k_begin + kt) * kRowBytes;
#pragma unroll
    for (int n = 0; n < kLoadsHalf; ++n) lds_dma16(src, a_vo[n], dst + (wq * kLoadsHalf + n) * 1024);
  };
  auto issue_w = [&](int kt) {
    const uint32_t dst = lds_base + (kt % kWStages) * kTileW + w_half * kHalfBytes;
    const char* src = reinterpret_cast<const char*>(p.w) + static_cast<int64_t>(k_begin + kt) * kRowBytes;
#pragma unroll
    for (int n = 0; n < kLoadsHalf; ++n) lds_dma16(src, w_vo[n], dst + (wq * kLoadsHalf + n) * 1024);
  };

  // wave tile: 128 token rows (grp) x 64 features (wq), 8 x 4 MFMA 16x16
  // tiles.  Operand read offsets within the A piece / W stage: row = base row
  // + lane%16 (+16 per MFMA tile, an immediate), 16-byte chunk 4*ks + lane/16
  // of the row's 8 (k step ks of 32); the swizzle depends on the row's bits
  // 1..3, which the tile offsets do not change.
  int a_off[2], w_off[2];
  {
    const int r = lane % 16, q = lane / 16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      a_off[ks] = r * kRowBytes + (((4 * ks + q) ^ swz(r)) * 16);
      w_off[ks] = (wq * 64 + r) * kRowBytes + (((4 * ks + q) ^ swz(r)) * 16);
    }
  }

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;

  auto memory_phase = [&](int s, bf16x8 (&wf)[2][4], bf16x8 (&af)[2][8]) {
    const char* ws = smem + (s % kWStages) * kTileW;
    const char* as = smem + kOffA + (2 * grp + s % kAStages) * kHalfBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wf[ks][i] = *reinterpret_cast<const bf16x8*>(ws + w_off[ks] + i * 16 * kRowBytes);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        af[ks][j] = *reinterpret_cast<const bf16x8*>(as + a_off[ks] + j * 16 * kRowBytes);
    }
    wait_lgkm0();  // this wave's reads of slice s are done before its stage is refilled
  };
  auto mfma_phase = [&](const bf16x8 (&wf)[2][4], const bf16x8 (&af)[2][8]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16x16x32(wf[ks][i], af[ks][j], acc[i][j]);
  };

  if (grp == 0) {
    // issue order: W1(0), A1(0), W1(1), then per slice s: A1(s+1), W1(s+2)
    issue_w(0);
    issue_a(0);
    if (k_tiles > 1) issue_w(1);
    for (int s = 0; s < k_tiles; ++s) {
      // W1(s) (this wave's pieces of slice s that phase 2s reads) has landed;
      // A1(s) and W1(s+1) may still be in flight
      wait_items(1 + (s + 1 < k_tiles));
      phase_barrier();  // phase 2s
      if (s + 1 < k_tiles) issue_a(s + 1);
      if (s + 2 < k_tiles) issue_w(s + 2);
      bf16x8 wf[2][4], af[2][8];
      memory_phase(s, wf, af);
      // A1(s), read by group 1 in phase 2s+1, has landed; W1(s+1), A1(s+1)
      // and W1(s+2) may still be in flight
      wait_items(2 * (s + 1 < k_tiles) + (s + 2 < k_tiles));
      phase_barrier();  // phase 2s+1
      mfma_phase(wf, af);
    }
    phase_barrier();  // the second group's last phase
  } else {
    // issue order: A0(0), W2(0), A0(1), W2(1), then per slice s: A0(s+2), W2(s+2)
    issue_a(0);
    issue_w(0);
    if (k_tiles > 1) {
      issue_a(1);
      issue_w(1);
    }
    // A0(0) and W2(0) have landed before group 0 reads slice 0
    wait_items(k_tiles > 1 ? 2 : 0);
    phase_barrier();  // phase 0
    for (int s = 0; s < k_tiles; ++s) {
      phase_barrier();  // phase 2s+1
      if (s + 2 < k_tiles) {
        issue_a(s + 2);
        issue_w(s + 2);
      }
      bf16x8 wf[2][4], af[2][8];
      memory_phase(s, wf, af);
      // A0(s+1) and W2(s+1), read by group 0 in phase 2s+2, have landed
      wait_items(s + 2 < k_tiles ? 2 : 0);
      phase_barrier();  // phase 2s+2
      mfma_phase(wf, af);
    }
  }

  if (part < 0) {
    tile_epilogue<EPI>(p, acc, m0 + grp * 128, n0 + wq * 64, lane);
  } else {
    // partial tile, row-major 256 x 256 fp32: row grp*128 + 16j + lane%16,
    // columns wq*64 + 16i + 4*(lane/16) .. +3
    float* dst = sp.partials + static_cast<int64_t>(tail * sp.parts + part) * (kTM * kTN) +
                 (grp * 128 + lane % 16) * kTN + wq * 64 + 4 * (lane / 16);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(dst + j * 16 * kTN + i * 16) = acc[i][j];
  }
}

// Sum of the K-split partial tiles of the last tiles, in K order (fixed:
// deterministic), then the tile epilogue.  One thread per 4 adjacent output
// features of one token row; 64 workgroups of 256 threads per tile.
template <int EPI>
__global__ __launch_bounds__(256) void split_fixup_kernel(GemmParams p, int tiles_m, int tiles_n, SplitPlan sp) {
  const int tail = blockIdx.x / 64;
  const int idx = (blockIdx.x % 64) * 256 + threadIdx.x;  // 0 .. 16383
  const int r = idx / (kTN / 4), c = (idx % (kTN / 4)) * 4;
  int tm, tn;
  tile_of(sp.whole + tail, tiles_m, tiles_n, tm, tn);
  const int64_t m = static_cast<int64_t>(tm) * kTM + r;
  const int n = tn * kTN + c;
  if (m >= p.m || n >= p.n) return;
  const float* src = sp.partials + static_cast<int64_t>(tail * sp.parts) * (kTM * kTN) + r * kTN + c;
  f32x4 sum = *reinterpret_cast<const f32x4*>(src);
  for (int q = 1; q < sp.parts; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + static_cast<int64_t>(q) * (kTM * kTN));
    sum[0] += v[0]; sum[1] += v[1]; sum[2] += v[2]; sum[3] += v[3];
  }
  float y[4] = {sum[0], sum[1], sum[2], sum[3]};
  store_epilogue<EPI>(p, m, n, y);
}

}  // namespace big

// ---------------------------------------------------------------------------
// Matrix-vector products (M <= 8 token rows: the conditioning MLP and the
// modulation projections of the loop glue).  They read W once and little
// else, so they are HBM-bound: each wave owns 4 output features (one
// epilogue group), its lanes stream 16-byte chunks of those 4 W rows along K
// (a wave-wide step covers 512 k, coalesced), multiply them with the same
// chunks of the M A rows (L2-resident) into fp32 sums, and reduce the sums
// across the wave at the end (fixed order: deterministic).
namespace gemv {

constexpr int kRows = 4;           // output features per wave
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxM = 8;
constexpr int kStep = 64 * 8;      // k per wave-wide step (8 bf16 per lane)

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <int EPI, int M>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemmParams p) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int n0 = (blockIdx.x * kWaves + wave) * kRows;
  if (n0 >= p.n) return;  // n is a multiple of 8, so a wave's 4 rows are all valid or all not
  const uint16_t* wrow[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) wrow[r] = p.w + static_cast<int64_t>(n0 + r) * p.k;
  const uint16_t* arow[M];
#pragma unroll
  for (int m = 0; m < M; ++m) arow[m] = p.a + a_row_offset(p, m);
  float acc[M][kRows];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[m][r] = 0.f;
#pragma unroll 2
  for (int k = lane * 8; k < p.k; k += kStep) {  // k is a multiple of 8: chunks are whole
    u32x4 wv[kRows], av[M];
#pragma unroll
    for (int r = 0; r < kRows; ++r) wv[r] = *reinterpret_cast<const u32x4*>(wrow[r] + k);
#pragma unroll
    for (int m = 0; m < M; ++m) av[m] = *reinterpret_cast<const u32x4*>(arow[m] + k);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float a0 = bf_lo(av[m][j]), a1 = bf_hi(av[m][j]);
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
          acc[m][r] = fmaf(a0, bf_lo(wv[r][j]), acc[m][r]);
          acc[m][r] = fmaf(a1, bf_hi(wv[r][j]), acc[m][r]);
        }
      }
  }
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[m][r] = wave_sum(acc[m][r]);
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (lane == m) store_epilogue<EPI>(p, m, n0, acc[m]);
}

template <int EPI>
hipError_t launch(const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.n / kRows + kWaves - 1) / kWaves), block(kThreads);
  switch (p.m) {
    case 1: hipLaunchKernelGGL((gemv_kernel<EPI, 1>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<EPI, 2>), grid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL((gemv_kernel<EPI, 3>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemv_kernel<EPI, 4>), grid, block, 0, s, p); break;
    case 5: hipLaunchKernelGGL((gemv_kernel<EPI, 5>), grid, block, 0, s, p); break;
    case 6: hipLaunchKernelGGL((gemv_kernel<EPI, 6>), grid, block, 0, s, p); break;
    case 7: hipLaunchKernelGGL((gemv_kernel<EPI, 7>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((gemv_kernel<EPI, 8>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gemv

// ---------------------------------------------------------------------------
// Few output features (N <= 64) over a long K: the projection of the final
// hidden states to the latent channels.  The product is a stream over A (the
// W rows are L2-resident), so the kernel is built to read A once at HBM rate:
// a workgroup takes TG x 16 token rows and all (up to 64) features, its 4
// waves split K in four contiguous ranges, and each wave streams its range of
// A and W straight into registers (no LDS staging), the next 64-k chunk in
// flight while the current one is multiplied.  The four fp32 partial tiles
// are then summed through LDS in wave order (fixed: deterministic).
namespace thin_n {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdP = 64 + 4;  // padded partial row (floats): row r starts 4 bank groups after row r-1

template <int EPI, int TG>
__global__ __launch_bounds__(kThreads, TG > 4 ? 1 : 2) void gemm_kernel(GemmParams p) {
  constexpr int kRows = 16 * TG;
  __shared__ __attribute__((aligned(16))) float part[kWaves * kRows * kLdP];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int r = lane % 16, q = lane / 16;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kRows;

  // Operand rows of this lane: token m0 + 16j + r (clamped: rows past m are
  // computed, never stored), feature 16i + r (clamped likewise); 16-byte
  // chunk q of each 32-k step.
  const int kw = p.k / kWaves;  // a multiple of 64
  const int64_t kb = static_cast<int64_t>(wave) * kw;
  const uint16_t* arow[TG];
#pragma unroll
  for (int j = 0; j < TG; ++j) {
    int64_t m = m0 + 16 * j + r;
    if (m > p.m - 1) m = p.m - 1;
    arow[j] = p.a + a_row_offset(p, m) + kb + 8 * q;
  }
  const uint16_t* wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wrow[i] = p.w + static_cast<int64_t>(min(16 * i + r, p.n - 1)) * p.k + kb + 8 * q;

  f32x4 acc[4][TG];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 a0[2][TG], w0[2][4], a1[2][TG], w1[2][4];
  auto load = [&](bf16x8 (&af)[2][TG], bf16x8 (&wf)[2][4], int c) {
    const int ko = 64 * c;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int j = 0; j < TG; ++j) af[ks][j] = *reinterpret_cast<const bf16x8*>(arow[j] + ko + 32 * ks);
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[ks][i] = *reinterpret_cast<const bf16x8*>(wrow[i] + ko + 32 * ks);
    }
  };
  auto mma = [&](const bf16x8 (&af)[2][TG], const bf16x8 (&wf)[2][4]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TG; ++j) acc[i][j] = mfma16x16x32(wf[ks][i], af[ks][j], acc[i][j]);
  };
  const int chunks = kw / 64;
  load(a0, w0, 0);
  int c = 0;
  for (; c + 2 <= chunks; c += 2) {
    load(a1, w1, c + 1);
    mma(a0, w0);
    if (c + 2 < chunks) load(a0, w0, c + 2);
    mma(a1, w1);
  }
  if (c < chunks) mma(a0, w0);

  // Partial tile of this wave: acc[i][j][e] = sum over its K range for token
  // row 16j + r and feature 16i + 4q + e.
  float* mine = part + wave * kRows * kLdP;
#pragma unroll
  for (int j = 0; j < TG; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(mine + (16 * j + r) * kLdP + 16 * i + 4 * q) = acc[i][j];
  __syncthreads();

  // Sum in wave (K) order and store: thread t takes row t / (256 / kRows)
  // and kFeat consecutive features of it.
  static_assert(kThreads % kRows == 0, "whole rows per thread group");
  constexpr int kPerRow = kThreads / kRows;  // threads per row: 2, 4 or 8
  constexpr int kFeat = 64 / kPerRow;        // features per thread: 32, 16 or 8
  const int row = threadIdx.x / kPerRow;
  const int f0 = (threadIdx.x % kPerRow) * kFeat;
  const int64_t m = m0 + row;
  if (m >= p.m) return;
  const int64_t crow = c_row_offset(p, m);
#pragma unroll
  for (int g = 0; g < kFeat / 4; ++g) {
    const int n = f0 + 4 * g;
    if (n >= p.n) break;
    const float* src = part + row * kLdP + n;
    f32x4 s = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + w * kRows * kLdP);
      s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
    }
    float y[4] = {s[0], s[1], s[2], s[3]};
    if (p.bias) {
      const u32x2 bb = *reinterpret_cast<const u32x2*>(p.bias + n);
      y[0] += __uint_as_float(bb[0] << 16);
      y[1] += __uint_as_float(bb[0] & 0xffff0000u);
      y[2] += __uint_as_float(bb[1] << 16);
      y[3] += __uint_as_float(bb[1] & 0xffff0000u);
    }
    store_row<EPI>(p, m, crow, n, y);
  }
}

template <int EPI>
hipError_t launch(const GemmParams& p, hipStream_t s) {
  // The largest workgroup (128, 64 or 32 rows) of which there are at least
  // as many as compute units: every wave's W fragments serve more rows.
  const int64_t cu = compute_units() > 0 ? compute_units() : 256;
  if ((p.m + 127) / 128 >= cu) {
    hipLaunchKernelGGL((gemm_kernel<EPI, 8>), dim3(static_cast<unsigned>((p.m + 127) / 128)), dim3(kThreads), 0, s, p);
  } else if ((p.m + 63) / 64 >= cu) {
    hipLaunchKernelGGL((gemm_kernel<EPI, 4>), dim3(static_cast<unsigned>((p.m + 63) / 64)), dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL((gemm_kernel<EPI, 2>), dim3(static_cast<unsigned>((p.m + 31) / 32)), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace thin_n

// ---------------------------------------------------------------------------
// A short K (64 or 128) onto many output features: the input projection of
// the latent channels to the hidden width.  The product is a stream of
// stores (the fp32 output is ~64x larger than the operands), so the kernel
// is built to keep the stores flowing.  A workgroup takes a contiguous range
// of 32-row token blocks and 256 output features: it first copies the A rows
// of its whole range into LDS (at most 40 KB), then each wave, holding the W
// rows of its 64 features in registers for the whole kernel, walks the
// blocks: fragments from LDS, MFMAs, stores.  The loop issues no global
// loads, so no wait in it ever covers the stores (the vector-memory counter
// completes in issue order, loads and stores alike).
namespace thin_k {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsBytes = 40 * 1024;

// A and C offsets of token row m (m < 2^31, checked by the launcher: 32-bit
// row arithmetic).
__device__ __forceinline__ void row_offsets(const GemmParams& p, uint32_t m, int64_t& a_off, int64_t& c_off) {
  if (p.group_rows > 0) {
    const uint32_t g = m / static_cast<uint32_t>(p.group_rows);
    const uint32_t i = m - g * static_cast<uint32_t>(p.group_rows);
    a_off = g * p.a_group_stride + static_cast<int64_t>(i) * p.lda;
    c_off = g * p.c_group_stride + static_cast<int64_t>(i) * p.ldc;
  } else {
    a_off = static_cast<int64_t>(m) * p.lda;
    c_off = static_cast<int64_t>(m) * p.ldc;
  }
}

// LDS position of 16-byte chunk c of staged row R (rows of KS * 64 bytes):
// chunks are XOR-swizzled by row so that the 16 rows one fragment read
// touches fall in distinct bank groups (16 bytes each, 16 per clock).
template <int KS>
__device__ __forceinline__ int lds_chunk(int R, int c) {
  return KS == 2 ? (c ^ ((R >> 1) & 7)) : (c ^ (R & 15));
}

template <int EPI, int KS>  // KS = K / 32
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams p, int m_blocks, int per_wg) {
  constexpr int kRowBytes = KS * 64;
  constexpr int kChunks = kRowBytes / 16;  // 8 or 16 per row
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int r = lane % 16, q = lane / 16;
  const int b0 = blockIdx.y * per_wg;
  const int nb = min(per_wg, m_blocks - b0);

  // Stage the A rows of blocks b0 .. b0 + nb - 1 (rows past m clamped: computed, never stored).
  {
    const int chunks = nb * 32 * kChunks;
    for (int c0 = 0; c0 < chunks; c0 += kThreads * 4) {
      u32x4 v[4];
      int pos[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * kThreads + threadIdx.x;
        pos[u] = -1;
        if (c < chunks) {
          const int R = c / kChunks, ch = c % kChunks;
          const uint32_t m = static_cast<uint32_t>(min(static_cast<int64_t>(b0) * 32 + R, p.m - 1));
          int64_t a_off, c_off;
          row_offsets(p, m, a_off, c_off);
          v[u] = *reinterpret_cast<const u32x4*>(p.a + a_off + ch * 8);
          pos[u] = R * kRowBytes + lds_chunk<KS>(R, ch) * 16;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (pos[u] >= 0) *reinterpret_cast<u32x4*>(smem + pos[u]) = v[u];
    }
  }
  __syncthreads();

  const int n_base = (blockIdx.x * kWaves + wave) * 64;
  if (n_base >= p.n) return;  // no barriers below: a wave past n just ends
  const bool n_full = n_base + 64 <= p.n;

  bf16x8 wf[4][KS];
  u32x2 bias[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t nr = min(n_base + 16 * i + r, p.n - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) wf[i][ks] = *reinterpret_cast<const bf16x8*>(p.w + nr * p.k + 32 * ks + 8 * q);
    const int n = n_base + 16 * i + 4 * q;
    bias[i] = (p.bias && n < p.n) ? *reinterpret_cast<const u32x2*>(p.bias + n) : u32x2{0u, 0u};
  }

  // Block t of the range: acc[i][jj][e] is token row 32(b0 + t) + 16jj + r,
  // feature n_base + 16i + 4q + e.  kChecked: rows past m and features past
  // n are skipped (the last block, a wave at the end of n).
  auto block = [&](int t, auto checked) {
    constexpr bool kChecked = decltype(checked)::value;
    bf16x8 af[2][KS];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int R = t * 32 + 16 * jj + r;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        af[jj][ks] = *reinterpret_cast<const bf16x8*>(smem + R * kRowBytes + lds_chunk<KS>(R, 4 * ks + q) * 16);
    }
    f32x4 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc[i][jj] = mfma16x16x32(wf[i][ks], af[jj][ks], acc[i][jj]);
      }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int64_t m = static_cast<int64_t>(b0 + t) * 32 + 16 * jj + r;
      if (kChecked && m >= p.m) continue;
      int64_t a_off, c_off;
      row_offsets(p, static_cast<uint32_t>(m), a_off, c_off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n_base + 16 * i + 4 * q;
        if (kChecked && n >= p.n) continue;
        float y[4] = {acc[i][jj][0] + __uint_as_float(bias[i][0] << 16),
                      acc[i][jj][1] + __uint_as_float(bias[i][0] & 0xffff0000u),
                      acc[i][jj][2] + __uint_as_float(bias[i][1] << 16),
                      acc[i][jj][3] + __uint_as_float(bias[i][1] & 0xffff0000u)};
        store_row<EPI>(p, m, c_off, n, y);
      }
    }
  };
  using Unchecked = std::integral_constant<bool, false>;
  using Checked = std::integral_constant<bool, true>;
  // whole blocks (every row below m) unchecked when the wave's features are all in range
  const int whole = min(nb, static_cast<int>(p.m / 32) - b0);
  int t = 0;
  if (n_full)
    for (; t < whole; ++t) block(t, Unchecked{});
  for (; t < nb; ++t) block(t, Checked{});
}

template <int EPI>
hipError_t launch(const GemmParams& p, hipStream_t s) {
  const int m_blocks = static_cast<int>((p.m + 31) / 32);
  const int nx = (p.n + 64 * kWaves - 1) / (64 * kWaves);
  const int cu = compute_units();
  // blocks per workgroup: about 4 workgroups per compute unit, within the LDS
  const int max_per = kLdsBytes / (32 * 2 * p.k);
  const int64_t want = (static_cast<int64_t>(m_blocks) * nx + 4 * (cu > 0 ? cu : 256) - 1) /
                       (4 * (cu > 0 ? cu : 256));
  const int per_wg = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(max_per, want)));
  // (the dispatcher keeps this within 65535 workgroups along y)
  const dim3 grid(nx, (m_blocks + per_wg - 1) / per_wg);
  if (p.k == 64)
    hipLaunchKernelGGL((gemm_kernel<EPI, 2>), grid, dim3(kThreads), 0, s, p, m_blocks, per_wg);
  else if (p.k == 128)
    hipLaunchKernelGGL((gemm_kernel<EPI, 4>), grid, dim3(kThreads), 0, s, p, m_blocks, per_wg);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace thin_k

}  // namespace

// Compute units of the current device (cached per device; 0 if unknown).
int compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int cu = cached[dev].load(std::memory_order_relaxed);
  if (cu == 0) {
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
      return 0;
    cached[dev].store(cu, std::memory_order_relaxed);
  }
  return cu;
}

hipError_t launch_gemm(const GemmParams& p, int epilogue, hipStream_t s) {
  if (p.m == 0) return hipSuccess;
  if (p.k <= 0 || p.k % 64 != 0) return hipErrorInvalidValue;  // the tiled kernels step K by 64
  if (p.m <= gemv::kMaxM) {
    if (p.n % 8 != 0) return hipErrorInvalidValue;
    switch (epilogue) {
      case EPI_BF16: return gemv::launch<EPI_BF16>(p, s);
      case EPI_GELU: return gemv::launch<EPI_GELU>(p, s);
      case EPI_SILU: return gemv::launch<EPI_SILU>(p, s);
      case EPI_F32: return gemv::launch<EPI_F32>(p, s);
      case EPI_GATED: return gemv::launch<EPI_GATED>(p, s);
      case EPI_RES: return gemv::launch<EPI_RES>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  // Few features over a long K (the projection to the latent channels) and
  // a short K onto many features (the projection from them): stream kernels.
  const int thin = p.n <= 64 && p.k >= 1024 && p.k % 256 == 0 && p.m >= 256 ? 1
                   : (p.k == 64 || p.k == 128) && p.n >= 256 && p.m >= 1024 &&
                             (p.m + 31) / 32 <= int64_t{65535} * (thin_k::kLdsBytes / (64 * p.k)) ? 2 : 0;
  if (thin) {
    switch (epilogue) {
      case EPI_BF16: return thin == 1 ? thin_n::launch<EPI_BF16>(p, s) : thin_k::launch<EPI_BF16>(p, s);
      case EPI_GELU: return thin == 1 ? thin_n::launch<EPI_GELU>(p, s) : thin_k::launch<EPI_GELU>(p, s);
      case EPI_SILU: return thin == 1 ? thin_n::launch<EPI_SILU>(p, s) : thin_k::launch<EPI_SILU>(p, s);
      case EPI_F32: return thin == 1 ? thin_n::launch<EPI_F32>(p, s) : thin_k::launch<EPI_F32>(p, s);
      case EPI_GATED: return thin == 1 ? thin_n::launch<EPI_GATED>(p, s) : thin_k::launch<EPI_GATED>(p, s);
      case EPI_RES: return thin == 1 ? thin_n::launch<EPI_RES>(p, s) : thin_k::launch<EPI_RES>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  // The large kernel addresses operand bytes by 32-bit offsets from p.a and p.w.
  const int64_t a_extent = 2 * (p.group_rows > 0 ? ((p.m - 1) / p.group_rows) * p.a_group_stride +
                                                        ((p.m - 1) % p.group_rows) * p.lda
                                                  : (p.m - 1) * p.lda) + 2 * static_cast<int64_t>(p.k);
  const int64_t w_extent = 2 * static_cast<int64_t>(p.n) * p.k;
  const bool offsets_fit = a_extent <= (int64_t{1} << 32) && w_extent <= (int64_t{1} << 32);
  // Below K = 256 (four slices) the large kernel's one 128 KB-LDS workgroup per
  // CU cannot overlap a tile's load latency and store with other work; the
  // small kernel (two workgroups per CU) is faster there (input projection
  // 32760 x 5120 x 64: 0.178 vs 0.207 ms).
  if (p.m >= 4 * big::kTM && p.n >= big::kTN && p.k >= 256 && offsets_fit) {
    const int tiles_m = static_cast<int>((p.m + big::kTM - 1) / big::kTM);
    const int tiles_n = (p.n + big::kTN - 1) / big::kTN;
    const int total = tiles_m * tiles_n;
    // One workgroup per CU (160 KB of LDS each): a last round of f < CUs/2
    // tiles would leave most CUs idle, so with scratch those f tiles are
    // split along K over up to CUs/f workgroups (each >= 2 slices, at most 8
    // parts) and a second kernel sums the partials in K order.
    big::SplitPlan sp{total, 1, nullptr};
    const int slots = compute_units();
    const int f = slots > 0 ? total % slots : 0;
    if (p.split_ws && f > 0 && 2 * f <= slots) {
      int parts = std::min({slots / f, p.k / big::kBK / 2, 8, kMaxSplitParts / f});
      if (parts >= 2) sp = big::SplitPlan{total - f, parts, p.split_ws};
    }
    const int n_wg = sp.whole + (total - sp.whole) * sp.parts;
    dim3 grid(n_wg);
    dim3 block(big::kThreads);
    switch (epilogue) {
      case EPI_BF16: hipLaunchKernelGGL(big::gemm_kernel<EPI_BF16>, grid, block, 0, s, p, tiles_m, tiles_n, sp); break;
      case EPI_GELU: hipLaunchKernelGGL(big::gemm_kernel<EPI_GELU>, grid, block, 0, s, p, tiles_m, tiles_n, sp); break;
      case EPI_SILU: hipLaunchKernelGGL(big::gemm_kernel<EPI_SILU>, grid, block, 0, s, p, tiles_m, tiles_n, sp); break;
      case EPI_F32: hipLaunchKernelGGL(big::gemm_kernel<EPI_F32>, grid, block, 0, s, p, tiles_m, tiles_n, sp); break;
      case EPI_GATED: hipLaunchKernelGGL(big::gemm_kernel<EPI_GATED>, grid, block, 0, s, p, tiles_m, tiles_n, sp); break;
      case EPI_RES: hipLaunchKernelGGL(big::gemm_kernel<EPI_RES>, grid, block, 0, s, p, tiles_m, tiles_n, sp); break;
      default: return hipErrorInvalidValue;
    }
    if (sp.whole == total) return hipGetLastError();
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 fgrid((total - sp.whole) * 64);
    switch (epilogue) {
      case EPI_BF16: hipLaunchKernelGGL(big::split_fixup_kernel<EPI_BF16>, fgrid, dim3(256), 0, s, p, tiles_m, tiles_n, sp); break;
      case EPI_GELU: hipLaunchKernelGGL(big::split_fixup_kernel<EPI_GELU>, fgrid, dim3(256), 0, s, p, tiles_m, tiles_n, sp); break;
      case EPI_SILU: hipLaunchKernelGGL(big::split_fixup_kernel<EPI_SILU>, fgrid, dim3(256), 0, s, p, tiles_m, tiles_n, sp); break;
      case EPI_F32: hipLaunchKernelGGL(big::split_fixup_kernel<EPI_F32>, fgrid, dim3(256), 0, s, p, tiles_m, tiles_n, sp); break;
      case EPI_GATED: hipLaunchKernelGGL(big::split_fixup_kernel<EPI_GATED>, fgrid, dim3(256), 0, s, p, tiles_m, tiles_n, sp); break;
      case EPI_RES: hipLaunchKernelGGL(big::split_fixup_kernel<EPI_RES>, fgrid, dim3(256), 0, s, p, tiles_m, tiles_n, sp); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  dim3 grid((p.n + kTN - 1) / kTN, static_cast<unsigned>((p.m + kTM - 1) / kTM));
  dim3 block(kThreads);
  switch (epilogue) {
    case EPI_BF16: hipLaunchKernelGGL(gemm_kernel<EPI_BF16>, grid, block, 0, s, p); break;
    case EPI_GELU: hipLaunchKernelGGL(gemm_kernel<EPI_GELU>, grid, block, 0, s, p); break;
    case EPI_SILU: hipLaunchKernelGGL(gemm_kernel<EPI_SILU>, grid, block, 0, s, p); break;
    case EPI_F32: hipLaunchKernelGGL(gemm_kernel<EPI_F32>, grid, block, 0, s, p); break;
    case EPI_GATED: hipLaunchKernelGGL(gemm_kernel<EPI_GATED>, grid, block, 0, s, p); break;
    case EPI_RES: hipLaunchKernelGGL(gemm_kernel<EPI_RES>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dit
