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

// Key row of result register v in lane half hh of a v_mfma_f32_32x32x16_bf16 tile (A rows
// = keys): 8 (v / 4) + 4 hh + (v mod 4).
__device__ __forceinline__ int key_row(int v, int hh) { return 8 * (v >> 2) + 4 * hh + (v & 3); }

// ---- key tiles on the matrix cores (v_mfma_f32_32x32x16_bf16, wave64): lane l supplies
// row (l & 31) of A and column (l & 31) of B, each with the 8 consecutive k of group
// (l >> 5); its 16 results are column (l & 31), rows key_row(v, l >> 5).  The head
// dimension is walked as k-step s, group hh -> dims 16s + 8hh .. +8 for A and B alike.

// Rows [row0, row0 + 64) of one (b,h)'s keys (zero past N) staged into LDS by a workgroup
// of 256 threads in two phases, so that several tiles' loads (and other loads of the
// caller) are in flight together before the first store.
template <int D>
struct KeyTile {
  static constexpr int LDSR = D + 8;
  static constexpr int TPR = D / 8;                 // 16-byte pieces per key row
  static constexpr int NP = kLeaf * TPR / 256;      // pieces per thread
  static_assert(kLeaf * TPR % 256 == 0, "a tile splits evenly over 256 threads");
  uint4 v[NP];
  __device__ __forceinline__ void load(const bf16* __restrict__ kb, int row0, int N) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int t = threadIdx.x + 256 * u, r = t / TPR, c = (t % TPR) * 8;
      v[u] = row0 + r < N ? *reinterpret_cast<const uint4*>(kb + (int64_t)(row0 + r) * D + c) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16* kt) const {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int t = threadIdx.x + 256 * u, r = t / TPR, c = (t % TPR) * 8;
      *reinterpret_cast<uint4*>(kt + r * LDSR + c) = v[u];
    }
  }
};
template <int D>
__device__ __forceinline__ void stage_tile(const bf16* __restrict__ kb, int row0, int N, bf16* kt) {
  KeyTile<D> t;
  t.load(kb, row0, N);
  t.store(kt);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// B fragments of one query row for v_mfma_f32_32x32x16_bf16: k-step s, lane half
// hh = lane >> 5 <-> dims 16s + 8hh .. +8 (the two lanes of a column read 32 contiguous
// bytes of its query row per load).
template <int D>
__device__ __forceinline__ void load_bfrag(const bf16* __restrict__ qrow, bool valid, int hh, bf16x8* bq) {
  constexpr int KS = D / 16;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (valid) {
      bq[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hh);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) bq[s][e] = (__bf16)0.f;
    }
  }
}

// B fragments of one column: k-step s at p + s * step (p already at the lane's 8 dims).
// Always loads: a caller with no row for the column points p at any valid row and
// discards that column's results, which costs less than zeroing the fragments under a
// branch.
template <int D>
__device__ __forceinline__ void load_bfrag_step(const bf16* __restrict__ p, int step, bf16x8* bq) {
  constexpr int KS = D / 16;
#pragma unroll
  for (int s = 0; s < KS; ++s) bq[s] = *reinterpret_cast<const bf16x8*>(p + step * s);
}

// 64 keys (LDS tile, two M-tiles of 32) x 32 columns: acc0/acc1[v] of lane l hold keys
// key_row(v, l >> 5) and 32 + key_row(v, l >> 5) against column l & 31.
template <int D>
__device__ __forceinline__ void tile_mfma32(const bf16* kt, const bf16x8* bq, int lane, f32x16& acc0,
                                            f32x16& acc1) {
  constexpr int LDSR = D + 8;
  constexpr int KS = D / 16;
  const int col = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    acc0[v] = 0.f;
    acc1[v] = 0.f;
  }
  // key fragments one k-step ahead (step s + 1's reads in flight while step s's products
  // issue), held in that order through scheduling: otherwise each product waits out its
  // own LDS round trip
  bf16x8 a[2][2];
  auto rd = [&](int s, bf16x8 (&f)[2]) {
    f[0] = *reinterpret_cast<const bf16x8*>(kt + col * LDSR + 16 * s + 8 * hh);
    f[1] = *reinterpret_cast<const bf16x8*>(kt + (32 + col) * LDSR + 16 * s + 8 * hh);
  };
  rd(0, a[0]);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (s + 1 < KS) rd(s + 1, a[(s + 1) & 1]);
    acc0 = mfma32(a[s & 1][0], bq[s], acc0);
    acc1 = mfma32(a[s & 1][1], bq[s], acc1);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (s + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
}

// LSE over the 64 keys of this lane's column (32 here, 32 in lane l ^ 32), in units of
// the scaled dot product.  Masked keys hold -inf; at least one key is live.
__device__ __forceinline__ float column_lse32(const f32x16& a0, const f32x16& a1, float s, float s_log2e) {
  // The max: fmed3 against +inf in a register the compiler cannot see through is the max of
  // two raw MFMA results without canonicalising each first (which fmaxf would do), then a
  // chain of v_max3_f32 over those 16 pair maxima (24 instructions for 32 values).
  float pinf = INFINITY;
  asm volatile("" : "+s"(pinf));
  float c[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) c[v] = __builtin_amdgcn_fmed3f(a0[v], a1[v], pinf);
  float m = vmax3(c[0], c[1], c[2]);
#pragma unroll
  for (int v = 3; v < 15; v += 2) m = vmax3(m, c[v], c[v + 1]);
  m = vmax3(m, c[15], c[15]);
  m = xor32_max(m);
  // exp(s (a - m)) as 2^(a s log2(e) - m s log2(e)): one fused multiply-add per key
  const float ms = m * s_log2e;
  float sum = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v)
    sum += __builtin_amdgcn_exp2f(fmaf(a0[v], s_log2e, -ms)) + __builtin_amdgcn_exp2f(fmaf(a1[v], s_log2e, -ms));
  sum = xor32_sum(sum);
  // sum >= 1 (the max key contributes 2^0), so log2 times ln 2 needs no range handling
  return s * m + 0.6931471805599453f * __builtin_amdgcn_logf(sum);
}

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
#pragma unroll 8
  for (int y = 0; y < twoK; ++y) {  // unrolled: the lane reads go out together
    const uint64_t oy = __shfl(my, y);
    rank += oy > my;
  }
  const int kept = leaf >= 0 && rank < K - nf;
  // ascending output position: selected entries (kept or forced) with a smaller index
  const int fj = lane < nf ? (lane == 0 ? F[0] : (lane == 1 ? F[1] : F[2])) : 0x7fffffff;
  int pos = 0, pf = 0;
#pragma unroll 8
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

// The same selection for 64 / SL query groups at once (SL >= 2K slots per group, a power of
// two): lane = (group lane / SL, slot lane % SL) holds candidate `leaf` (-1 if none) with
// score `sc`; fsc is this lane's group's forced-block scores.  kx and lx are 64-entry
// per-wavefront LDS scratch; `live` is false for lanes of a group past the last query
// (they take part in the exchange but write nothing).
template <int SL>
__device__ __forceinline__ void finalize_rows(int leaf, float sc, const int* F, int nf, const float* fsc, int K,
                                              int lane, bool live, uint64_t* kx, int32_t* lx,
                                              int32_t* __restrict__ oi, float* __restrict__ os) {
  const int base = lane & ~(SL - 1), slot = lane & (SL - 1);
  const uint32_t u = __float_as_uint(sc);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  const uint64_t my = leaf >= 0 ? (((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)leaf)) : 0ull;
  kx[lane] = my;
  wave_sync();
  int rank = 0;
#pragma unroll
  for (int y = 0; y < SL; y += 2) {
    const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(kx + base + y);
    rank += (kk.x > my) + (kk.y > my);
  }
  const bool kept = leaf >= 0 && rank < K - nf;
  lx[lane] = kept ? leaf : 0x7fffffff;
  wave_sync();
  // ascending output position: selected entries (kept or forced) with a smaller index
  const int fj = slot < nf ? (slot == 0 ? F[0] : (slot == 1 ? F[1] : F[2])) : 0x7fffffff;
  int pos = 0, pf = 0;
#pragma unroll
  for (int y = 0; y < SL; y += 4) {
    const int4 o = *reinterpret_cast<const int4*>(lx + base + y);
    pos += (o.x < leaf) + (o.y < leaf) + (o.z < leaf) + (o.w < leaf);
    pf += (o.x < fj) + (o.y < fj) + (o.z < fj) + (o.w < fj);
  }
  for (int f = 0; f < nf; ++f) {
    pos += F[f] < leaf;
    pf += F[f] < fj;
  }
  const uint64_t gmask = (SL == 64) ? ~0ull : (((1ull << SL) - 1ull) << base);
  const int nsel = (int)__popcll(__ballot(kept) & gmask) + nf;
  if (live) {
    if (kept && pos < K) {
      oi[pos] = leaf;
      os[pos] = sc;
    }
    if (slot < nf && pf < K) {
      oi[pf] = fj;
      os[pf] = fsc[slot];
    }
    if (slot >= nsel && slot < K) {
      oi[slot] = -1;
      os[slot] = -INFINITY;
    }
  }
  wave_sync();  // kx, lx are rewritten by the next call
}

}  // namespace pisa
