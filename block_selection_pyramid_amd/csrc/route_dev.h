// The top-down pyramid walk for one query group, run by one wavefront.
//
// "Block Sparse Attention with Log-Linear Complexity": rcap.io explainer, top-down walk
// paragraph (score the candidates of a level, keep the Top-K, expand only their children,
// at most g*K candidates per level) and scoring paragraph (a candidate's score is the
// LogSumExp over its child summaries of q.child); agihunt.info summary, kernels paragraph
// (the G query heads of a GQA group share the selection: their per-head LSEs are summed).
//
// Layout per level: candidate x owns child slots 2x and 2x+1 (g = 2).  A pass covers 32
// child slots; lane l scores slot (l & 31) over half (l >> 5) of the head dimension for
// all G heads, the halves are combined with one cross-lane exchange, the pair of lanes of
// a candidate combines its two children into per-head LSEs, and the group score is the
// sum over heads.  Top-K is a rank count over at most 64 candidates (score descending,
// block index ascending); the kept node of rank r expands into slots 2r, 2r+1.  Candidate
// ids live in LDS; a -1 marks an empty slot (a child that does not exist or is not yet
// visible to the query).
#pragma once

#include "dev_common.h"

namespace pisa {

constexpr int kQPad = 4;  // floats of padding per query row in LDS

// Per-wave LDS scratch of the walk.
struct WalkLds {
  int32_t X[kMaxCand];
  float cs[kMaxCand];
};

// Scores the nx candidates X[0..nx) of level l (>= 2) for one query group whose rows
// (fp32) sit in qs[r * (D + kQPad) + e]; writes cs[x] (-inf for empty slots).
template <int D, int G>
__device__ __forceinline__ void score_level(const Geo& geo, const float* __restrict__ P, const float* qs, int bq,
                                            int l, int nx, WalkLds* w, int lane) {
  const float* Pc = P + (int64_t)geo.off[l - 1] * D;
  const int nchild = geo.n[l - 1];
  const int cshift = l - 2;  // child c (level l-1) covers leaf blocks from c << cshift
  const int half = lane >> 5;
  for (int base = 0; base < 2 * nx; base += 32) {
    const int slot = base + (lane & 31);
    const int x = slot >> 1;
    const int node = x < nx ? w->X[x] : -1;
    const int c = node >= 0 ? 2 * node + (slot & 1) : -1;
    const bool valid = c >= 0 && c < nchild && ((int64_t)c << cshift) <= bq;
    float dot[G];
#pragma unroll
    for (int r = 0; r < G; ++r) dot[r] = 0.f;
    if (valid) {
      const float* pv = Pc + (int64_t)c * D + half * (D / 2);
#pragma unroll 4
      for (int e = 0; e < D / 2; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(pv + e);
#pragma unroll
        for (int r = 0; r < G; ++r) {
          const float4 qv = *reinterpret_cast<const float4*>(qs + r * (D + kQPad) + half * (D / 2) + e);
          dot[r] += v.x * qv.x + v.y * qv.y + v.z * qv.z + v.w * qv.w;
        }
      }
    }
    float sc = 0.f;
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const float full = dot[r] + __shfl_xor(dot[r], 32);
      const float y = valid ? geo.s * full : -INFINITY;
      const float y2 = __shfl_xor(y, 1);
      const float m = fmaxf(y, y2);
      // m is finite whenever the candidate exists: its first child is always visible.
      sc += m + logf(expf(y - m) + expf(y2 - m));
    }
    if (lane < 32 && (slot & 1) == 0 && x < nx) w->cs[x] = node >= 0 ? sc : -INFINITY;
  }
  wave_sync();
}

// Runs the walk; on return w->X[0..nx) holds the leaf candidates (ids or -1) and the
// function returns nx (<= 2K).  qs must be filled and visible to the wave.
template <int D, int G>
__device__ int route_walk(const Geo& geo, const float* __restrict__ P, const float* qs, int bq, WalkLds* w,
                          int lane) {
  const int L = geo.L, K = geo.K;
  if (L == 1) {
    const int nx = bq + 1;  // every visible leaf block (n_1 <= g*K)
    if (lane < nx) w->X[lane] = lane;
    wave_sync();
    return nx;
  }
  int nx = min(geo.n[L], (bq >> (L - 1)) + 1);  // visible top-level nodes form a prefix
  if (lane < nx) w->X[lane] = lane;
  wave_sync();
  for (int l = L; l >= 2; --l) {
    score_level<D, G>(geo, P, qs, bq, l, nx, w, lane);
    // rank of each existing candidate
    int rank = K;
    int myid = -1;
    if (lane < nx) {
      myid = w->X[lane];
      if (myid >= 0) {
        const float my = w->cs[lane];
        rank = 0;
        for (int y = 0; y < nx; ++y) {
          const int oid = w->X[y];
          const float o = w->cs[y];
          rank += oid >= 0 && (o > my || (o == my && oid < myid));
        }
      }
    }
    const unsigned long long exist = __ballot(lane < nx && myid >= 0);
    const int nkept = min(K, (int)__popcll(exist));
    wave_sync();
    // expand kept nodes into the next level's slots
    const int nchild = geo.n[l - 1];
    const int cshift = l - 2;
    if (myid >= 0 && rank < K) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ch = 2 * myid + c;
        const bool ok = ch < nchild && ((int64_t)ch << cshift) <= bq;
        w->X[2 * rank + c] = ok ? ch : -1;
      }
    }
    nx = 2 * nkept;
    wave_sync();
  }
  return nx;
}

// Loads the G query rows of one group into LDS as fp32.  qrow(r) points at head r's row.
template <typename T, int D, int G>
__device__ __forceinline__ void load_qrows(const T* const* rows, float* qs, int lane) {
  constexpr int VEC = Vec<T>::N;
  constexpr int PER_ROW = D / VEC;
  for (int t = lane; t < G * PER_ROW; t += kWave) {
    const int r = t / PER_ROW, e = (t % PER_ROW) * VEC;
    float x[VEC];
    Vec<T>::load(rows[r] + e, x);
#pragma unroll
    for (int v = 0; v < VEC; ++v) qs[r * (D + kQPad) + e + v] = x[v];
  }
}

}  // namespace pisa
