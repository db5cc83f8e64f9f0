// Joint attention over [visual; text] tokens on bf16 MFMA (gfx950).
//
// Each query attends to the visual and the valid text keys of its batch row
// under one softmax ("Difflet", section 4).  Padded text keys sit after the
// valid ones, so the valid keys are the interval [0, n_vis + L_b) and one
// integer per row decides the mask ("Difflet", section 4.2, Representing
// Attention Mask): key tiles past the bound are never visited and only the one
// tile that straddles it is masked.  Key and value rows past the bound are
// never read at all (their loads are clamped to the last valid row), so
// whatever the padded slots hold cannot reach the output.
//
// The Trainium kernel on the pages (128-query tiles, scores kept on chip, a
// transpose of the probabilities before the value product) is prior art; the
// mechanics here are CDNA4's, chosen from measurements on gfx950:
//  * a workgroup is 8 waves of 32 queries (256 queries), two waves per SIMD.
//    The waves form two groups that alternate between an MFMA phase and a
//    softmax phase, one phase apart, with a workgroup barrier at every phase
//    boundary: while one wave of a SIMD multiplies, the other exponentiates.
//    The softmax work of a tile is split: the tile max, the update of the
//    reference max and half of the exponentials in the softmax phase, the
//    other half of the exponentials between the MFMAs of the wave's own MFMA
//    phase (a few independent VALU instructions per MFMA cost no MFMA time
//    there; long dependent chains would).
//  * K and V tiles (64 keys) stream from HBM/L2 straight into LDS with
//    global_load_lds_dwordx4 (no VGPR staging) through a 4-stage ring, two
//    tiles ahead of the math, issued by the group entering its softmax
//    phase (whose VALU-bound stream has issue slots to spare).  Rows are stored unpadded with their 16-byte
//    chunks XOR-swizzled by row so the K fragment reads and the transposing V
//    reads hit distinct bank groups.  The loads are issued from inline
//    assembly so the compiler does not guard each LDS read with a wait for
//    every load in flight (an explicit vmcnt wait + barrier per tile is the
//    synchronisation);
//  * scores are produced transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16, K
//    as the A operand): each lane then holds the scores of ONE query against 32
//    keys, so the row max needs one exchange between lane halves, and the
//    exponentiated scores are already laid out as the B operand of
//    O^T = V^T P^T (the key order inside each 16-key step is permuted the same
//    way in both operands, which leaves the sum unchanged);
//  * V^T fragments come from row-major V with ds_read_b64_tr_b16 (gfx950's
//    transposing LDS read): in each 16-lane group, output lane 4r+e takes
//    element e of the 8-byte reads of source lanes r, r+4, r+8, r+12, so
//    source lane s points at key k0 + s/4, columns d0 + 4(s%4) .. +3 and
//    output lane i receives keys k0..k0+3 of column d0 + i;
//  * softmax runs in the log2 domain: p = exp2(s*c - m) with c = scale*log2(e)
//    folded into one FMA before v_exp_f32; the running max and sum are fp32
//    and O is divided by the sum once at the end.  The MFMA accumulators are
//    VGPRs (the file is built with the VGPR form of MFMA) so the softmax
//    phase reads the scores without AGPR copies.
#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int kWaves = 8;      // two groups of 4 waves, one wave of each per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;        // keys per tile
constexpr int kStages = 4;     // LDS ring depth
constexpr int kBM = kWaves * 32;  // queries per workgroup (32 per wave)
// Value MFMAs of an MFMA phase issued after the barrier that ends it.  A wave
// reaches a workgroup barrier only once its issued MFMAs have drained, so
// with the phase's last MFMAs on the far side the matrix pipe stays busy
// across the hand-over to the other wave of the SIMD (measured: a two-wave
// ping-pong of 32 MFMAs per phase loses 97 cycles per barrier with 0
// trailing MFMAs, 53 with 2, 91 with 4).
#ifndef DIT_ATTN_TRAIL
#define DIT_ATTN_TRAIL 2
#endif
constexpr int kTrail = DIT_ATTN_TRAIL;
// How far (log2 units) the softmax reference of a query may lag its running
// maximum, once the query's partial sum of weights has reached kLagMinSum,
// before l and O are rescaled.
constexpr float kMaxLag = 2.f;
constexpr float kLagMinSum = 32.f;

template <int D>
struct Tile {
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kBytes = kBN * kRowBytes;         // one K or V tile
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows per wave-wide 16 B/lane load
  static constexpr int kLoads = kBN / kRowsPerLoad / kWaves;  // prologue: all 8 waves load
  static constexpr int kLoads4 = kBN / kRowsPerLoad / 4;      // later tiles: the 4 waves of group 1
  static constexpr int kStageBytes = 2 * kBytes;         // K tile then V tile
};

// 16-byte chunk c of tile row r is stored at chunk position c ^ swz(r).
// Measured on gfx950, LDS serves a 16-byte K fragment read in ~5.8 clocks
// and an 8-byte transposing read in ~3.0 when every group of lanes served
// together touches distinct 16-byte bank groups (16 of them, 256 bytes):
//  * K reads: lanes 0..15 read the same chunk of rows 0..15, so swz must be
//    a permutation over 16 consecutive rows (bank group = (row*kChunks + pos)
//    mod 16);
//  * V reads: lanes 0..31 read 4 consecutive chunks (one aligned group of 4)
//    of 4 consecutive rows, so those rows must move the group to 4 distinct
//    places.
// With 16 chunks per row (D = 128) swz = 4*(r&3) + ((r>>2)&3) meets both;
// with 8 chunks (D = 64, two rows per bank cycle) swz = 4*((r>>1)&1) +
// ((r>>2)&3) does.  swz depends on row % 16 only.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128)
    return 4 * (r & 3) + ((r >> 2) & 3);
  else
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// s_waitcnt with only vmcnt constrained (expcnt, lgkmcnt left at their max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_ptr;
typedef __attribute__((address_space(3))) const bf16x8* lds_bf16x8_ptr;
typedef __attribute__((address_space(3))) char* lds_char_ptr;

// One wave-wide 16-byte-per-lane load from global memory into LDS: lane i's
// 16 bytes at gbase + voff land at LDS byte lds_addr + 16*i.  gbase and
// lds_addr are wave-uniform.  M0 (the LDS base register) is saved and
// restored around the load.
__device__ __forceinline__ void lds_dma16(const char* gbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(gbase), "s"(lds_addr)
      : "memory");
}

// Per-lane byte offsets (from the tile's first key row) of the chunks this
// wave loads: wave w loads rows [(w*kLoads + n) * kRowsPerLoad, +kRowsPerLoad);
// lane i of a load lands at row i / kChunks, chunk position i % kChunks, so it
// fetches the chunk that swizzles there.  Rows past `last_row` (the last
// valid key, relative to the tile) are clamped to it.
template <int D, int NL>
__device__ __forceinline__ void dma_offsets(uint32_t (&voff)[NL], int wave, int lane,
                                            int64_t stride_bytes, int last_row) {
  using T = Tile<D>;
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int r = (wave * NL + n) * T::kRowsPerLoad + lane / T::kChunks;
    const int c = (lane % T::kChunks) ^ swz<D>(r);
    voff[n] = static_cast<uint32_t>(min(r, last_row) * stride_bytes + c * 16);
  }
}

template <int D, int NL>
__device__ __forceinline__ void dma_tile(const char* kg, const char* vg, const uint32_t (&voff)[NL],
                                         uint32_t lds_stage, int wave) {
  using T = Tile<D>;
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const uint32_t dst = lds_stage + (wave * NL + n) * 1024;
    lds_dma16(kg, voff[n], dst);
    lds_dma16(vg, voff[n], dst + T::kBytes);
  }
}

template <int D>
struct WaveState {
  static constexpr int kKS = D / 16;  // 16-wide k steps of K Q^T
  static constexpr int kDB = D / 32;  // 32-row blocks of O^T
  bf16x8 qf[kKS];     // Q fragments: Q[q][16*ks + 8*hi .. +7], q = lane%32
  f32x16 o[kDB];      // O^T accumulators: o[db][4g + e] = O[q][32db + 8g + 4*hi + e]
  f32x16 s[2];        // S^T of one tile: s[t][4g + e] = score of key 32t + 8g + 4*hi + e
  f32x16 sh;          // s[1] of the last softmax'ed tile as s*c - m: exponentiated in the next MFMA phase
  bf16x8 pf[4];       // p of one tile as the B operand of four 16-key value steps
  float m_run;        // reference max of the scaled scores (log2 domain): the running
                      // max, or up to kMaxLag below it
  float m_tile;       // max of the scaled scores of the tile in s (this lane's query)
  float mx[4];        // the four partial max chains of the tile in s
  bf16x8 vt[kTrail > 0 ? kTrail : 1];  // V^T fragments of the value MFMAs issued after the phase barrier
  float l_run;        // this lane's partial sum of p
  int k_off[kKS];     // K fragment byte offsets within a stage (row lane%32)
  int v_off[2][kDB];  // V^T transposing-read byte offsets (rows 8g + 4*hi + s16/4)
  uint32_t ka[kKS];     // LDS addresses of the next MFMA phase's K fragment reads
  uint32_t va[2][kDB];  // and of its V^T reads
};

// max of three floats.  This file is compiled with -fno-honor-nans (its
// scores and running maxima are never NaN: masked keys are -inf and padded
// key rows are never loaded), so the compiler fuses the two fmaxf into one
// v_max3_f32 without quieting ops and schedules it freely (an inline-asm
// v_max3 costs hazard no-ops between dependent maxima).
__device__ __forceinline__ float vmax3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// max / sum of a value with the one in the other half of the wave (lane^32),
// without an LDS round trip: v_permlane32_swap of (x, x) leaves
// (x[l], x[l+32]) in lanes l < 32 and (x[l-32], x[l]) in lanes l >= 32.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax3(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Step i (0..15) of the tile max: 32 scores -> 1 in 16 v_max3 on four
// independent chains (chain i % 4 covers 8 scores of one 16-row group).
template <int D>
__device__ __forceinline__ void tile_max_step(WaveState<D>& st, int i) {
  const int c4 = i % 4, k = i / 4;
  const int t = c4 / 2, r0 = 8 * (c4 % 2);
  if (k == 0) st.mx[c4] = vmax3(st.s[t][r0], st.s[t][r0 + 1], st.s[t][r0 + 2]);
  else if (k == 1) st.mx[c4] = vmax3(st.mx[c4], st.s[t][r0 + 3], st.s[t][r0 + 4]);
  else if (k == 2) st.mx[c4] = vmax3(st.mx[c4], st.s[t][r0 + 5], st.s[t][r0 + 6]);
  else st.mx[c4] = vmax3(st.mx[c4], st.s[t][r0 + 7], st.s[t][r0 + 7]);
  asm volatile("" : "+v"(st.mx[c4]));  // keep the four chains interleaved in this order
}

template <int D>
__device__ __forceinline__ void tile_max_finish(WaveState<D>& st, float c) {
  // c > 0 keeps the order
  st.m_tile = max_halves(vmax3(st.mx[0], st.mx[1], vmax3(st.mx[2], st.mx[3], st.mx[3]))) * c;
}

// MFMA phase: S^T of key tile j+1 (absent after the last tile), then
// O^T += V^T P^T for tile j (absent before the first tile), reading their K
// and V stages at the LDS addresses prep_addresses left in st.ka, st.va.  LDS
// reads and MFMAs, with independent VALU work of this wave placed between
// them, where it issues while the matrix pipe runs (measured on gfx950: up to
// ~4 FP32 VALU instructions per 32x32x16 MFMA cost no MFMA time): after each
// score MFMA one exponential (with its row sum and bf16 packing) of the
// second half of tile j.  Fragment reads run a fixed number of steps ahead of
// their MFMA (scheduling fences keep the compiler from hoisting all 32 of
// them, which would cost 128 VGPRs).
template <int D, bool kPVPart, bool kQKPart, int kTr = 0>
__device__ __forceinline__ void mfma_phase(WaveState<D>& st) {
  using T = Tile<D>;
  using W = WaveState<D>;
  constexpr int kPV = 4 * W::kDB;  // value steps: (u, db)
  constexpr int kQK = 2 * W::kKS;  // score steps: (ks, t), t fastest: two accumulator chains
  constexpr int kAhead = 2;  // fragment reads in flight ahead of their MFMA
  // The second half of the last softmax'ed tile (keys 32..63, held in sh as
  // s*c - m) is exponentiated here, between the MFMAs -- its exponentials,
  // row sums and bf16 packing are independent VALU work that issues while
  // the matrix pipe runs -- and becomes pf[2], pf[3] before the value MFMAs
  // that read them.  (With a value part there is always such a half.)
  float ep[16];
  float lp0, lp1;
  auto finish_part = [&](int i) {
    ep[i] = __builtin_amdgcn_exp2f(st.sh[i]);
    if (i % 2 == 1) {
      lp0 = i == 1 ? ep[0] : lp0 + ep[i - 1];
      lp1 = i == 1 ? ep[1] : lp1 + ep[i];
      u32x4 w = __builtin_bit_cast(u32x4, st.pf[2 + i / 8]);
      w[(i % 8) / 2] = pack_bf16x2(ep[i - 1], ep[i]);
      st.pf[2 + i / 8] = __builtin_bit_cast(bf16x8, w);
    }
  };
  static_assert(kQK == 16 || !kQKPart || D != 128, "one pending score per score MFMA at head_dim 128");
  if constexpr (kQKPart) {
    auto kread = [&](int i) {
      const int t = i % 2, ks = i / 2;
      return *(lds_bf16x8_ptr)(uintptr_t)(st.ka[ks] + 32 * t * T::kRowBytes);
    };
    bf16x8 kf[kQK];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) kf[i] = kread(i);
    const f32x16 zero = {};  // first step of each chain: an inline-constant 0 accumulator
#pragma unroll
    for (int i = 0; i < kQK; ++i) {
      if (i + kAhead < kQK) kf[i + kAhead] = kread(i + kAhead);
      __builtin_amdgcn_sched_barrier(0);
      st.s[i % 2] = mfma32x32x16(kf[i], st.qf[i / 2], i < 2 ? zero : st.s[i % 2]);
      if constexpr (kPVPart) {
        // 16 pending scores over kQK score MFMAs
        constexpr int kPer = 16 / kQK;
#pragma unroll
        for (int n = 0; n < kPer; ++n) finish_part(i * kPer + n);
      }
    }
  } else if constexpr (kPVPart) {
#pragma unroll
    for (int i = 0; i < 16; ++i) finish_part(i);
  }
  if constexpr (kPVPart) {
    st.l_run += lp0 + lp1;
    // keep the sums here, between the MFMAs, rather than let the compiler
    // sink them into the next softmax phase where l is read
    asm volatile("" : "+v"(st.l_run));
    auto vread = [&](int i) {
      const int u = i / W::kDB, db = i % W::kDB;
      const uint32_t row = 16 * u * T::kRowBytes;
      const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(uintptr_t)(st.va[0][db] + row));
      const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(uintptr_t)(st.va[1][db] + row));
      return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 vf[kPV];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) vf[i] = vread(i);
    static_assert(kTr <= kAhead, "trailing fragments must already be read");
#pragma unroll
    for (int i = 0; i < kPV - kTr; ++i) {
      if (i + kAhead < kPV) vf[i + kAhead] = vread(i + kAhead);
      __builtin_amdgcn_sched_barrier(0);
      st.o[i % W::kDB] = mfma32x32x16(vf[i], st.pf[i / W::kDB], st.o[i % W::kDB]);
    }
#pragma unroll
    for (int j = 0; j < kTr; ++j) st.vt[j] = vf[kPV - kTr + j];
  }
}

// The last kTr value MFMAs of an MFMA phase (their V^T fragments already in
// st.vt), issued right after the barrier that ends the phase.
template <int D, int kTr>
__device__ __forceinline__ void mfma_tail(WaveState<D>& st) {
  using W = WaveState<D>;
  constexpr int kPV = 4 * W::kDB;
#pragma unroll
  for (int j = 0; j < kTr; ++j) {
    const int i = kPV - kTr + j;
    st.o[i % W::kDB] = mfma32x32x16(st.vt[j], st.pf[i / W::kDB], st.o[i % W::kDB]);
  }
}

// Softmax phase for key tile j (keys j0 .. j0+63): the tile max, mask past
// the bound (only the tile that holds it), update of the reference max with the rescale of l and O when the tile's max passed
// it (by more than kMaxLag for a query whose weights sum to kLagMinSum or
// more), p = exp2(s*c - m)
// of the first 32 keys into the running sum and, rounded to bf16, into
// pf[0], pf[1]; the other 32 keys only as s*c - m (the next MFMA phase
// exponentiates them).  VALU only.
template <int D>
__device__ __forceinline__ void softmax_phase(WaveState<D>& st, int j0, int n_valid, int hi, float c) {
  using W = WaveState<D>;
  // The tile's max, 32 scores -> 1 in 16 v_max3 on four independent chains.
  // The tile that holds the bound needs no mask for this: its key rows past
  // the bound were loaded as copies of the last valid key's row, so those
  // scores repeat a valid one and leave the max unchanged.  (Taken here
  // rather than between the value MFMAs of the MFMA phase: that phase is the
  // longer of the two once most rescales are skipped.)
#pragma unroll
  for (int i = 0; i < 16; ++i) tile_max_step(st, i);
  tile_max_finish(st, c);
  if (j0 + kBN > n_valid) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (j0 + 32 * t + 8 * (r / 4) + 4 * hi + (r % 4) >= n_valid) st.s[t][r] = -INFINITY;
  }
  // Reference max.  The weights p = exp2(s*c - m) are right for any
  // reference m, since the final division by l cancels it; with m the exact
  // running maximum, the key that sets a new maximum gets weight exactly 1
  // and only the others are rounded to bf16.  l and O are rescaled
  // (wave-uniformly) when some query of the wave sees a score above its
  // reference, except that a query whose sum of weights l has reached
  // kLagMinSum lets the reference lag its maximum by up to kMaxLag: weights
  // then stay below 2^kMaxLag, and a key that sets a new maximum within that
  // lag is rounded like the others, which moves the output by at most
  // 2^(kMaxLag-9) / kLagMinSum = 2^-12 of the largest |v| per such key (the
  // ratio of a weight to l survives later rescales, and l only grows between
  // them).  Flat rows reach that sum within a few tiles, after which their
  // maxima rise rarely and by little, so most rescales are skipped; peaked
  // rows keep an exact reference.
  const float m_tile = st.m_tile;
  const float m_limit = st.l_run >= kLagMinSum ? st.m_run + kMaxLag : st.m_run;
  if (__builtin_amdgcn_ballot_w64(m_tile > m_limit) != 0) {
    const float m_new = vmax3(st.m_run, m_tile, m_tile);
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.m_run = m_new;
    st.l_run *= alpha;
    // O holds the value sums up to the previous tile; the next MFMA phase
    // adds this tile's, relative to the new maximum
#pragma unroll
    for (int db = 0; db < W::kDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) st.o[db][e] *= alpha;
  }
  const float nm = -st.m_run;
  // keys 0..31 of the tile: exponentiate, sum, pack into pf[0], pf[1]
  float l0, l1;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(st.s[0][8 * u + i], c, nm));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(st.s[0][8 * u + i + 1], c, nm));
      l0 = (u == 0 && i == 0) ? e0 : l0 + e0;
      l1 = (u == 0 && i == 0) ? e1 : l1 + e1;
      w[i / 2] = pack_bf16x2(e0, e1);
    }
    st.pf[u] = __builtin_bit_cast(bf16x8, w);
  }
  st.l_run += l0 + l1;
  // keys 32..63: only s*c - m here; the next MFMA phase exponentiates them
#pragma unroll
  for (int r = 0; r < 16; ++r) st.sh[r] = fmaf(st.s[1][r], c, nm);
}

// LDS addresses of the next MFMA phase's K and V^T reads (K tile in the
// stage at LDS byte kst, V tile in the stage at vst), added up in the
// softmax phase: taken out of the MFMA phase's in-order stream, which is the
// longer of the two once most rescales are skipped (measured 0.8-1.3 %
// faster).  The empty asm statements keep the additions here.
template <int D>
__device__ __forceinline__ void prep_addresses(WaveState<D>& st, uint32_t kst, uint32_t vst) {
  using T = Tile<D>;
  using W = WaveState<D>;
#pragma unroll
  for (int ks = 0; ks < W::kKS; ++ks) {
    st.ka[ks] = kst + st.k_off[ks];
    asm volatile("" : "+v"(st.ka[ks]));
  }
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int db = 0; db < W::kDB; ++db) {
      st.va[g][db] = vst + T::kBytes + st.v_off[g][db];
      asm volatile("" : "+v"(st.va[g][db]));
    }
}

// Issue the loads of tile j into its ring slot (clamping rows past the last
// valid key in the tile that holds the bound).
template <int D, int NL>
__device__ __forceinline__ void issue_tile(const char* kg0, const char* vg0, int64_t stride_bytes,
                                           int j, int n_valid, uint32_t lds_base, int wave,
                                           int lane, const uint32_t (&voff)[NL]) {
  using T = Tile<D>;
  const int64_t adv = static_cast<int64_t>(j) * kBN * stride_bytes;
  const uint32_t stage = lds_base + (j % kStages) * T::kStageBytes;
  if ((j + 1) * kBN <= n_valid) {
    dma_tile<D, NL>(kg0 + adv, vg0 + adv, voff, stage, wave);
  } else {
    uint32_t vc[NL];
    dma_offsets<D, NL>(vc, wave, lane, stride_bytes, n_valid - 1 - j * kBN);
    dma_tile<D, NL>(kg0 + adv, vg0 + adv, vc, stage, wave);
  }
}

// The workgroup's 8 waves form two groups (waves 0-3 and 4-7; each SIMD runs
// one wave of each) that alternate between an MFMA phase and a softmax phase,
// the second group one phase behind the first, with a workgroup barrier at
// every phase boundary.  While one wave of a SIMD multiplies, the other
// exponentiates, so the matrix core and the vector ALU work at the same time
// (measured on gfx950: VALU work in another wave hides behind MFMAs almost
// completely, VALU work in the same wave does not).
//
// Each wave runs the same sequence -- S of tile 0; softmax of tile 0; then
// for each tile k: {O += P V of tile k and S of tile k+1; softmax of tile
// k+1}; finally O += P V of the last tile -- with a barrier before every
// step.  The second group takes one extra barrier first (and the first group
// one at the end), which puts it exactly one phase behind.
template <int D, bool kOutF32>
__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnParams p) {
  using T = Tile<D>;
  using W = WaveState<D>;
  __shared__ __attribute__((aligned(1024))) char smem[kStages * T::kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave / 4;
  const int hi = lane / 32;
  // Workgroup -> (batch row, head, query tile).  The dispatcher deals
  // workgroup ids round-robin over the 8 XCDs, each with its own L2; the ids
  // are renumbered so that every XCD owns a contiguous run of (row, head)
  // pairs, query tile fastest.  The workgroups resident on one XCD then share
  // one head's K/V stream through that L2 (at c3 this halves the L2-miss
  // bytes of a launch) instead of every XCD streaming every head.
  // Workgroups past p.wg_main take one key range (part) of a query tile of
  // the split last round instead: tile p.wg_main + (id - p.wg_main) / parts.
  int b, h, qt, part = -1, tail = 0;
  {
    const int n_qt = (p.n_q + kBM - 1) / kBM;
    const int total = p.wg_main;
    const int id = blockIdx.x;
    int nid;
    if (id < total) {
      const int xcd = id % 8, slot = id / 8;
      const int per = total / 8, extra = total % 8;
      nid = xcd * per + min(xcd, extra) + slot;
    } else {
      tail = (id - total) / p.tail_parts;
      part = (id - total) % p.tail_parts;
      nid = total + tail;
    }
    qt = nid % n_qt;
    h = (nid / n_qt) % p.heads;
    b = nid / (n_qt * p.heads);
  }
  const int n_q = p.n_q;
  // Key tiles [tile0, tile0 + n_tiles) of the row's valid range, indexed
  // from tile0 below (n_valid relative to it as well).
  int n_tiles = (p.n_valid[b] + kBN - 1) / kBN;  // fully padded tiles are skipped
  int tile0 = 0, n_valid = p.n_valid[b];
  if (part >= 0) {
    tile0 = part * n_tiles / p.tail_parts;
    const int tile1 = (part + 1) * n_tiles / p.tail_parts;
    n_valid = min(n_valid, tile1 * kBN) - tile0 * kBN;
    n_tiles = tile1 - tile0;
  }
  const int64_t q_base = static_cast<int64_t>(b) * p.q_batch + h * D;
  const int64_t kv_base = static_cast<int64_t>(b) * p.kv_batch + static_cast<int64_t>(tile0) * kBN * p.kv_stride + h * D;
  const char* kg0 = reinterpret_cast<const char*>(p.k + kv_base);
  const char* vg0 = reinterpret_cast<const char*>(p.v + kv_base);
  const int64_t stride_bytes = p.kv_stride * 2;
  const int q_first = qt * kBM + wave * 32;

  if (n_tiles == 0) {
    // an empty key range (a partial of split attention whose partition holds
    // no valid key): the weighted sum is 0 and the log-denominator -inf, the
    // neutral element of the merge
    const int q = q_first + lane % 32;
    if (q < n_q) {
      const int64_t row = (static_cast<int64_t>(b) * n_q + q) * p.out_stride + h * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = 32 * db + 8 * g + 4 * hi;
          if constexpr (kOutF32) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + row + col) = z;
          } else {
            const u32x2 z = {0u, 0u};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + row + col) = z;
          }
        }
      if (p.lse && hi == 0) p.lse[(static_cast<int64_t>(b) * p.heads + h) * n_q + q] = -INFINITY;
    }
    return;
  }
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char_ptr)smem));
  const float c = p.scale_log2;

  uint32_t voff[T::kLoads];
  dma_offsets<D, T::kLoads>(voff, wave, lane, stride_bytes, kBN - 1);
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j)
    if (j < n_tiles) issue_tile<D, T::kLoads>(kg0, vg0, stride_bytes, j, n_valid, lds_base, wave, lane, voff);
  uint32_t voff4[T::kLoads4];
  dma_offsets<D, T::kLoads4>(voff4, wave % 4, lane, stride_bytes, kBN - 1);

  W st;
  // Q fragments.  The wait for them also covers the first tiles' loads;
  // waiting once here keeps the compiler from guarding later instructions
  // with waits on loads it cannot see complete.
  {
    const int q = min(q_first + lane % 32, n_q - 1);
    const uint16_t* src = p.q + q_base + static_cast<int64_t>(q) * p.q_stride + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < W::kKS; ++ks) st.qf[ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
  }
  wait_vmcnt<0>();
#pragma unroll
  for (int i = 0; i < W::kDB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[i][e] = 0.f;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  // LDS read offsets.  A K fragment row is lane%32 (+32t) and a V^T read row
  // is 16u + 8g + 4*hi + s16/4; the swizzle depends only on row % 16, so t
  // and u only add immediate row offsets.
  {
    const int r = lane % 32;
#pragma unroll
    for (int ks = 0; ks < W::kKS; ++ks) st.k_off[ks] = r * T::kRowBytes + (((2 * ks + hi) ^ swz<D>(r)) * 16);
    const int g16 = lane / 16, s16 = lane % 16;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int rv = 8 * g + 4 * hi + s16 / 4;
#pragma unroll
      for (int db = 0; db < W::kDB; ++db) {
        const int col = 32 * db + 16 * (g16 % 2) + 4 * (s16 % 4);
        st.v_off[g][db] = rv * T::kRowBytes + (((col / 8) ^ swz<D>(rv)) * 16) + (col % 8) * 2;
      }
    }
  }

  const bool a_grp_c = grp == 0;
  // Global phase 2m opens with "tile m has landed, ring slot of tile m-2 is
  // free" (the value reads of tile m-2 ended with phase 2m-1).  The first
  // group meets phase 2m before the MFMA phase that starts on tile m, the
  // second (one phase behind) before the softmax phase of tile m-1.  Tiles
  // 0..2 come from the prologue (every wave, waited for with the Q loads);
  // tile m+2 (m >= 1) is issued right after barrier 2m by the 4 waves of the
  // second group alone -- they are entering a softmax phase, whose in-order
  // stream has issue slots to spare between VALU instructions, while the
  // MFMA group's stream has none -- and those waves wait for their loads of
  // tile m (issued at phase 2m-4; only tile m+1's are newer) before barrier
  // 2m.
  constexpr int L4 = 2 * T::kLoads4;  // loads per loading wave per tile
  auto barrier_wait = [&](bool duty, int m) {
    duty = duty && !a_grp_c;
    if (duty && m >= 3 && m < n_tiles) {
      if (m + 1 < n_tiles) wait_vmcnt<L4>(); else wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
  };
  auto barrier_issue = [&](bool duty, int m) {
    duty = duty && !a_grp_c;
    if (duty && m >= 1 && m + 2 < n_tiles)
      issue_tile<D, T::kLoads4>(kg0, vg0, stride_bytes, m + 2, n_valid, lds_base, wave % 4, lane, voff4);
  };
  auto phase_barrier = [&](bool duty, int m) {
    barrier_wait(duty, m);
    barrier_issue(duty, m);
  };
  auto stage = [&](int j) { return lds_base + static_cast<uint32_t>((j % kStages) * T::kStageBytes); };
  // A wave in its MFMA phase runs at raised issue priority: when both waves
  // of a SIMD can issue, the MFMA (and the LDS reads feeding it) goes first
  // and the softmax's VALU work fills the cycles in between (measured 4-6 %
  // faster than equal priority, outputs unchanged).
  auto mfma_prio = [](bool on) {
    if (on)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
  };
  const bool a_grp = grp == 0;
  if (!a_grp) phase_barrier(true, 0);
  phase_barrier(a_grp, 0);
  mfma_prio(true);
  prep_addresses(st, stage(0), stage(0));
  mfma_phase<D, false, true>(st);
  mfma_prio(false);
  phase_barrier(!a_grp, 1);
  softmax_phase<D>(st, 0, n_valid, hi, c);
  prep_addresses(st, stage(1), stage(0));
  for (int k = 0; k + 1 < n_tiles; ++k) {
    phase_barrier(a_grp, k + 1);
    mfma_prio(true);
    mfma_phase<D, true, true, kTrail>(st);
    barrier_wait(!a_grp, k + 2);
    mfma_tail<D, kTrail>(st);  // keeps the matrix pipe busy across the hand-over
    mfma_prio(false);
    barrier_issue(!a_grp, k + 2);
    softmax_phase<D>(st, (k + 1) * kBN, n_valid, hi, c);
    prep_addresses(st, stage(k + 2), stage(k + 1));
  }
  phase_barrier(a_grp, n_tiles);
  mfma_prio(true);
  mfma_phase<D, true, false>(st);
  mfma_prio(false);
  if (a_grp) phase_barrier(false, 0);

  // Combine the two lane halves' partial sums, normalise, store.
  const int q = q_first + lane % 32;
  const float l_tot = sum_halves(st.l_run);
  if (part >= 0) {
    // a key range of a split tile: fp32 normalised partial and its
    // natural-log denominator, row (tail * parts + part) * 256 + query
    if (q < n_q) {
      const int64_t prow = (static_cast<int64_t>(tail) * p.tail_parts + part) * kBM + (q - qt * kBM);
      const float inv = 1.f / l_tot;
      float* dst = p.tail_o + prow * D;
#pragma unroll
      for (int db = 0; db < W::kDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = 32 * db + 8 * g + 4 * hi;
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = st.o[db][4 * g + e] * inv;
          *reinterpret_cast<f32x4*>(dst + col) = w;
        }
      if (hi == 0) p.tail_lse[prow] = st.m_run * 0.69314718055994531f + logf(l_tot);
    }
    return;
  }
  if (q < n_q) {
    const float inv = 1.f / l_tot;
    const int64_t row = (static_cast<int64_t>(b) * n_q + q) * p.out_stride + h * D;
#pragma unroll
    for (int db = 0; db < W::kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * db + 8 * g + 4 * hi;
        if constexpr (kOutF32) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = st.o[db][4 * g + e] * inv;
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + row + col) = w;
        } else {
          u32x2 w;
          w[0] = pack_bf16x2(st.o[db][4 * g] * inv, st.o[db][4 * g + 1] * inv);
          w[1] = pack_bf16x2(st.o[db][4 * g + 2] * inv, st.o[db][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + row + col) = w;
        }
      }
    if (p.lse && hi == 0)
      p.lse[(static_cast<int64_t>(b) * p.heads + h) * n_q + q] =
          st.m_run * 0.69314718055994531f + logf(l_tot);
  }
}

// Merge of the split tiles' key-range partials: one thread per 4 output
// elements of one query row; weights exp(lse_i - max lse) in fixed part
// order (deterministic), bf16 output at the row's place, and the merged
// log-denominator when the caller asked for it.
template <int D>
__global__ __launch_bounds__(256) void tail_merge_kernel(AttnParams p) {
  constexpr int kC = D / 4;
  const int n_qt = (p.n_q + kBM - 1) / kBM;
  const int n_tail = n_qt * p.heads * p.batch - p.wg_main;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(n_tail) * kBM * kC) return;
  const int c = static_cast<int>(idx % kC);
  const int r = static_cast<int>((idx / kC) % kBM);
  const int t = static_cast<int>(idx / (kC * kBM));
  const int nid = p.wg_main + t;
  const int qt = nid % n_qt, h = (nid / n_qt) % p.heads, b = nid / (n_qt * p.heads);
  const int q = qt * kBM + r;
  if (q >= p.n_q) return;
  const int parts = p.tail_parts;
  const int64_t row0 = static_cast<int64_t>(t) * parts * kBM + r;
  float ls[kAttnMaxTailParts];
  float lmax = -INFINITY;
  for (int i = 0; i < parts; ++i) {
    ls[i] = p.tail_lse[row0 + i * kBM];
    lmax = fmaxf(lmax, ls[i]);
  }
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < parts; ++i) {
    const float w = expf(ls[i] - lmax);
    const f32x4 o = *reinterpret_cast<const f32x4*>(p.tail_o + (row0 + i * kBM) * D + 4 * c);
    wsum += w;
    acc[0] = fmaf(w, o[0], acc[0]);
    acc[1] = fmaf(w, o[1], acc[1]);
    acc[2] = fmaf(w, o[2], acc[2]);
    acc[3] = fmaf(w, o[3], acc[3]);
  }
  const float inv = 1.f / wsum;
  u32x2 out;
  out[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  out[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  const int64_t orow = (static_cast<int64_t>(b) * p.n_q + q) * p.out_stride + h * D + 4 * c;
  *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + orow) = out;
  if (p.lse && c == 0) p.lse[(static_cast<int64_t>(b) * p.heads + h) * p.n_q + q] = lmax + logf(wsum);
}

}  // namespace

hipError_t launch_attention(const AttnParams& p_in, hipStream_t s) {
  AttnParams p = p_in;
  const int64_t n_wg = static_cast<int64_t>((p.n_q + kBM - 1) / kBM) * p.heads * p.batch;
  // One 512-thread workgroup per CU (128 KB of LDS each): a last round of
  // f query tiles after at least one full round leaves CUs - f idle.  With
  // scratch each of those f tiles is split into the number of key ranges p
  // (2..4, at most the fewest key tiles of a row, f * p partial tiles within
  // the scratch) whose f * p workgroups finish soonest, ceil(f p / CUs) / p
  // of a round, if that is under one round; the partials are merged after.
  p.wg_main = static_cast<int>(n_wg);
  p.tail_parts = 0;
  p.tail_o = p.tail_lse = nullptr;
  const int cu = compute_units();
  const int f = cu > 0 ? static_cast<int>(n_wg % cu) : 0;
  if (p.tail_ws && !p.out_f32 && cu > 0 && n_wg >= cu && f > 0) {
    int min_tiles = 1 << 30;
    for (int b = 0; b < p.batch; ++b) min_tiles = std::min(min_tiles, (p.n_valid[b] + kBN - 1) / kBN);
    int parts = 1;
    double best = 1.0;  // rounds the last f tiles take unsplit
    for (int q = 2; q <= kAttnMaxTailParts; ++q) {
      if (q > min_tiles || f * q > kAttnMaxTailTiles) break;
      const double t = static_cast<double>((f * q + cu - 1) / cu) / q;
      if (t < best - 1e-9) {
        best = t;
        parts = q;
      }
    }
    if (parts >= 2) {
      p.wg_main = static_cast<int>(n_wg) - f;
      p.tail_parts = parts;
      p.tail_o = p.tail_ws;
      p.tail_lse = p.tail_ws + static_cast<size_t>(f) * parts * kBM * p.head_dim;
    }
  }
  const int64_t n_launch = p.wg_main + static_cast<int64_t>(n_wg - p.wg_main) * p.tail_parts;
  if (n_launch * kThreads > 0xffffffffLL) return hipErrorInvalidValue;  // grid size in threads is 32-bit
  dim3 grid(static_cast<unsigned>(n_launch));
  dim3 block(kThreads);
  if (p.head_dim == 128 && !p.out_f32)
    hipLaunchKernelGGL((attn_kernel<128, false>), grid, block, 0, s, p);
  else if (p.head_dim == 128)
    hipLaunchKernelGGL((attn_kernel<128, true>), grid, block, 0, s, p);
  else if (p.head_dim == 64 && !p.out_f32)
    hipLaunchKernelGGL((attn_kernel<64, false>), grid, block, 0, s, p);
  else if (p.head_dim == 64)
    hipLaunchKernelGGL((attn_kernel<64, true>), grid, block, 0, s, p);
  else
    return hipErrorInvalidValue;
  if (p.tail_parts == 0) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = (n_wg - p.wg_main) * kBM * (p.head_dim / 4);
  dim3 mgrid(static_cast<unsigned>((threads + 255) / 256));
  if (p.head_dim == 128)
    hipLaunchKernelGGL((tail_merge_kernel<128>), mgrid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((tail_merge_kernel<64>), mgrid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dit
