// Device helpers shared by the MLA kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

typedef uint16_t bf16;  // bfloat16 bit pattern (storage type)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA A/B operand
typedef __attribute__((ext_vector_type(4))) short short4_t;     // transpose-read result
typedef __attribute__((ext_vector_type(16))) float f32x16;      // 32x32 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) float f32x4;        // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ float bf2f(bf16 x) { return __uint_as_float((uint32_t)x << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (bf16)0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

// Two floats -> packed pair of bf16 (low half = a), nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16>(const bf16* p) { return bf2f(*p); }

template <typename T> __device__ __forceinline__ void st(T* p, float v);
template <> __device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<bf16>(bf16* p, float v) { *p = f2bf(v); }

// RoPE angle of pair i at position pos: pos * base^(-2i/d_rope), formed in
// double so that positions in the tens of thousands keep their low bits; the
// caller takes sin/cos in double as well (few values per call).
__device__ __forceinline__ double rope_angle(int pos, int i, int d_rope, float base) {
  return (double)pos * pow((double)base, -2.0 * (double)i / (double)d_rope);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Context lengths of up to 256 rows, clamped at zero: row lane + 64 i in
// len[i] of each lane (0 past the last row). Loaded once per wave for the
// run-order helpers below.
__device__ inline void load_row_lens(int rows, const int32_t* __restrict__ ctx_lens, int (&len)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = lane + 64 * i;
    len[i] = row < rows ? max(ctx_lens[row], 0) : 0;
  }
}

// Longest runs first. A decode step cuts each query row's context (one new
// token per row) into runs of `run` tokens, one workgroup each; the last run
// of a row is usually shorter. Dispatch slot k (blocks start in slot order)
// takes the k-th run in the order: every full run, row by row, then the rows'
// last runs from the longest down (ties: lower row first). In plain row order
// the short last runs sit among the full ones, so with a little more than one
// round of full runs some full runs start only when another has finished; in
// this order the short runs fill in behind the full ones. Every wave works it
// out by itself from the context lengths (len from load_row_lens; O(rows^2 /
// 64) for the last runs, so the host uses it for at most 256 rows). Returns
// false when slot k has no run; else the run's row, its index in the row and
// the row's context length.
__device__ inline bool longest_run_first(int rows, int run, const int (&len)[4], int k, int& row_out,
                                         int& split_out, int& len_out) {
  const int lane = threadIdx.x & 63;
  if (rows <= 64) {
    // every row as long as the first and a whole number of runs: the order
    // is plain row order (no scan)
    const int len0 = __builtin_amdgcn_readfirstlane(len[0]);
    if (__ballot(lane < rows && len[0] != len0) == 0 && len0 > 0 && len0 % run == 0) {
      const int nf = len0 / run;
      if (k >= rows * nf) return false;
      row_out = k / nf;
      split_out = k - row_out * nf;
      len_out = len0;
      return true;
    }
  }
  int n_full = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (64 * i >= rows) break;
    const int nf = len[i] / run;
    int incl = nf;  // inclusive prefix sum over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int rel = k - n_full;
    const uint64_t hit = __ballot(rel >= incl - nf && rel < incl);
    if (hit != 0) {
      const int l = __builtin_ctzll(hit);
      row_out = 64 * i + l;
      split_out = rel - (__builtin_amdgcn_readlane(incl, l) - __builtin_amdgcn_readlane(nf, l));
      len_out = __builtin_amdgcn_readlane(len[i], l);
      return true;
    }
    n_full += __builtin_amdgcn_readlane(incl, 63);
  }
  // last runs: rank = number of rows whose last run is longer, or as long
  // and earlier (rows without one have rem = 0 and are never counted)
  const int kp = k - n_full;
  int rem[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rem[i] = len[i] % run;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (64 * i >= rows) break;
    const int row = 64 * i + lane;
    int rank = 0;
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      if (64 * i2 >= rows) break;
      for (int j = 0; j < 64; ++j) {
        const int r = __builtin_amdgcn_readlane(rem[i2], j);
        rank += (r > rem[i]) || (r == rem[i] && 64 * i2 + j < row);
      }
    }
    const uint64_t hit = __ballot(rem[i] > 0 && rank == kp);
    if (hit != 0) {
      const int l = __builtin_ctzll(hit);
      row_out = 64 * i + l;
      len_out = __builtin_amdgcn_readlane(len[i], l);
      split_out = len_out / run;  // after the row's full runs
      return true;
    }
  }
  return false;
}

// Run length, in pages, for the longest-first order. The host picks pps from
// the longest context alone. When the actual contexts then give a few more
// runs than the chip holds at once (`budget` workgroups), the runs past the
// first round, the shortest last runs, start only when others have finished,
// and the step can take up to about two runs' time. This returns the
// smallest run length in (pps, min(max_pps, 5 pps / 4)] whose runs all fit
// in one round; pps itself when its runs fit already, when they need more
// than two rounds, or when no such length exists. (In a list-scheduling
// model of ragged batches, runs up to a quarter longer won whenever they
// saved the second round; longer runs, or saving a third round, lost about
// as often as they won.) Every wave works it out by itself from the context
// lengths (len from load_row_lens); the result is wave-uniform.
__device__ inline int one_round_run_pages(int pps, int max_pps, int budget, int page, const int (&len)[4]) {
  int pages[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pages[i] = (len[i] + page - 1) / page;
  auto runs = [&](int q) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) n += (pages[i] + q - 1) / q;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
    return __builtin_amdgcn_readfirstlane(n);  // the same in every lane: keep it scalar
  };
  const int r0 = runs(pps);
  if (r0 <= budget || r0 > 2 * budget) return pps;
  const int lim = min(max_pps, pps + pps / 4);
  if (lim <= pps || runs(lim) > budget) return pps;
  int lo = pps, hi = lim;  // runs(lo) > budget >= runs(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (runs(mid) <= budget) hi = mid;
    else lo = mid;
  }
  return hi;
}

}  // namespace mla
