// Leaf-level pieces shared by the prefill and decode kernels.
//
// Leaf score ("Block Sparse Attention with Log-Linear Complexity", agihunt.info summary,
// pyramid paragraph: level 0 is the raw keys; LSE paragraph): for leaf block j and query i,
// the sum over the group's G heads of LSE over keys t in block j with t <= i of
// s * <q_h, k_t>.  Selection: the forced blocks {0, b-1, b} (LSE paragraph) plus the
// Top-(K-|F|) of the other leaf candidates, ascending, padded with (-1, -inf).
#pragma once

#include "dev_common.h"

namespace pisa {

// VALU score of one leaf tile for one query group: lane = key of the tile.
template <typename T, int D, int G>
__device__ float score_tile_valu(const T* __restrict__ keys /* this (b,h) */, int j, int i, int N, int C,
                                 const float* qs, int lane, float s) {
  constexpr int VEC = Vec<T>::N;
  constexpr int QS = D + 4;
  const int t = j * C + lane;
  const bool valid = lane < C && t < N && t <= i;
  float dot[G];
#pragma unroll
  for (int r = 0; r < G; ++r) dot[r] = 0.f;
  if (valid) {
    const T* kr = keys + (int64_t)t * D;
#pragma unroll 4
    for (int e = 0; e < D; e += VEC) {
      float x[VEC];
      Vec<T>::load(kr + e, x);
#pragma unroll
      for (int r = 0; r < G; ++r) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) dot[r] += x[v] * qs[r * QS + e + v];
      }
    }
  }
  float total = 0.f;
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const float y = valid ? s * dot[r] : -INFINITY;
    const float m = wave_max(y);
    const float sum = wave_sum(valid ? expf(y - m) : 0.f);
    total += m + logf(sum);
  }
  return total;
}

// One wavefront writes the final selection of one query group.  Lane x < twoK holds
// routed leaf candidate `leaf` (-1 if none; never a forced block) with score `sc`;
// F[0..nf) are the forced blocks with scores fsc[0..nf).
__device__ __forceinline__ void finalize_row(int leaf, float sc, const int* F, int nf, const float* fsc, int K,
                                             int twoK, int lane, int32_t* __restrict__ oi,
                                             float* __restrict__ os) {
  // Rank on a total order of (score desc, index asc): ranks are distinct even for scores
  // that compare unordered, so at most K - |F| candidates are kept.
  const uint32_t u = __float_as_uint(sc);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  const uint64_t my = leaf >= 0 ? (((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)leaf)) : 0ull;
  int rank = 0;
  for (int y = 0; y < twoK; ++y) {
    const uint64_t oy = __shfl(my, y);
    rank += oy > my;
  }
  const int kept = leaf >= 0 && rank < K - nf;
  // ascending output position: selected entries (kept or forced) with a smaller index
  const int fj = lane < nf ? (lane == 0 ? F[0] : (lane == 1 ? F[1] : F[2])) : 0x7fffffff;
  int pos = 0, pf = 0;
  for (int y = 0; y < twoK; ++y) {
    const int oy = __shfl(leaf, y);
    const int ky = __shfl(kept, y);
    pos += ky && oy < leaf;
    pf += ky && oy < fj;
  }
  for (int f = 0; f < nf; ++f) {
    pos += F[f] < leaf;
    pf += F[f] < fj;
  }
  if (kept && pos < K) {
    oi[pos] = leaf;
    os[pos] = sc;
  }
  if (lane < nf && pf < K) {
    oi[pf] = fj;
    os[pf] = fsc[lane];
  }
  const int nkept = (int)__popcll(__ballot(kept));
  const int nsel = nkept + nf;
  if (lane >= nsel && lane < K) {
    oi[lane] = -1;
    os[lane] = -INFINITY;
  }
}

}  // namespace pisa
