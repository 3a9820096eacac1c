// Pyramid construction ("Block Sparse Attention with Log-Linear Complexity", agihunt.info
// summary, pyramid paragraph; rcap.io explainer, tree paragraph):
// level 1 node j = mean of the keys of leaf block j, level l node j = mean of level l-1
// nodes 2j, 2j+1 (g = 2), unweighted over the children that exist.  Every mean also goes
// to the routing copy, scaled by s log2(e) and split into bf16 hi + lo.
//
// One workgroup reduces a subtree: 8 consecutive nodes of level l0 (each the mean of
// FAN rows of the level below: C raw keys for l0 = 1, g nodes above that) and then the
// up-to-3 levels above them from LDS.  For l0 = 1 the workgroup streams 8*C contiguous
// key rows with 16-byte loads, four nodes' rows in flight at once, so k is read from HBM
// exactly once.  Further launches with l0 = 5, 9, ... cover taller pyramids.
#include "dev_common.h"

namespace pisa {

namespace {

constexpr int kSub = 8;        // level-l0 nodes per workgroup (16 at 256K: build 90 -> 85 us, more workgroups)
constexpr int kSubLevels = 3;  // levels built from LDS above l0 (log2 kSub)

template <typename Tin, int D>
struct RowsShape {
  static constexpr int VEC = Vec<Tin>::N;
  static constexpr int TPR = D / VEC;    // threads per row
  static constexpr int RPP = 256 / TPR;  // rows per pass
};

// Mean of rows [r0, r1) of s (D wide) by a 256-thread workgroup: thread (column segment,
// rp) sums rows r0 + rp, r0 + rp + RPP, ... of its VEC columns in order, then thread e < D
// adds the RPP partial sums in order and divides.  Returns the mean in threads e < D.  One
// fixed order, so the pyramid build and the incremental append produce the same bits.
// Every thread of the workgroup must call it (it synchronises twice).
template <typename Tin, int D>
__device__ __forceinline__ float rows_mean(const Tin* s, int r0, int r1,
                                           float (&red)[RowsShape<Tin, D>::RPP][D], int tid) {
  constexpr int VEC = RowsShape<Tin, D>::VEC, TPR = RowsShape<Tin, D>::TPR, RPP = RowsShape<Tin, D>::RPP;
  const int cseg = tid % TPR, rp = tid / TPR;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  for (int r = r0 + rp; r < r1; r += RPP) {
    float x[VEC];
    Vec<Tin>::load(s + (int64_t)r * D + cseg * VEC, x);
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += x[v];
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) red[rp][cseg * VEC + v] = acc[v];
  __syncthreads();
  float m = 0.f;
  if (tid < D) {
    float t = 0.f;
#pragma unroll 8
    for (int p = 0; p < RPP; ++p) t += red[p][tid];
    m = t / (float)(r1 - r0);
  }
  __syncthreads();
  return m;
}

// Means of the nb <= NB consecutive nodes j0 .. j0+nb-1, node j over rows [j*FAN,
// min(j*FAN + FAN, src_rows)) of s, with rows_mean's arithmetic for each node (a thread adds
// its rows of the node in row order, then thread e < D adds the RPP partial sums in order
// and divides), so a subtree build and an incremental append give the same bits.  Every
// load of the NB nodes is issued before the first addition.  Returns the means in threads
// e < D.  Every thread of the workgroup must call it (it synchronises twice).
template <typename Tin, int D, int FAN, int NB>
__device__ __forceinline__ void rows_mean_multi(const Tin* s, int j0, int nb, int src_rows,
                                                float (&red)[NB][RowsShape<Tin, D>::RPP][D], int tid,
                                                float (&m)[NB]) {
  constexpr int VEC = RowsShape<Tin, D>::VEC, TPR = RowsShape<Tin, D>::TPR, RPP = RowsShape<Tin, D>::RPP;
  constexpr int RPT = (FAN + RPP - 1) / RPP;  // rows of a node per thread (at most)
  const int cseg = tid % TPR, rp = tid / TPR;
  float x[NB][RPT][VEC];
  bool ok[NB][RPT];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int r0 = (j0 + u) * FAN, r1 = min(r0 + FAN, src_rows);
#pragma unroll
    for (int t = 0; t < RPT; ++t) {
      const int r = r0 + rp + t * RPP;
      ok[u][t] = u < nb && rp + t * RPP < FAN && r < r1;
      Vec<Tin>::load(s + (int64_t)(ok[u][t] ? r : 0) * D + cseg * VEC, x[u][t]);  // row 0 always exists
    }
  }
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    float acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
#pragma unroll
    for (int t = 0; t < RPT; ++t)
      if (ok[u][t]) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] += x[u][t][v];
      }
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[u][rp][cseg * VEC + v] = acc[v];
  }
  __syncthreads();
  if (tid < D) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      float t = 0.f;
#pragma unroll 8
      for (int p = 0; p < RPP; ++p) t += red[u][p][tid];
      const int r0 = (j0 + u) * FAN;
      m[u] = t / (float)(min(r0 + FAN, src_rows) - r0);
    }
  }
  __syncthreads();
}

constexpr int kBuildNodes = 4;  // level-l0 nodes whose rows one workgroup loads at once

// FAN: rows per level-l0 node (C raw keys for l0 = 1, g nodes above).
template <typename Tin, int D, int FAN>
__global__ __launch_bounds__(256) void pyr_sub_kernel(const Tin* __restrict__ src, int64_t src_bh_stride,
                                                      int32_t src_rows, float* __restrict__ pyr, Geo geo,
                                                      int32_t l0) {
  __shared__ float red[kBuildNodes][RowsShape<Tin, D>::RPP][D];
  __shared__ float lvl[2][kSub][D];

  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int j0 = blockIdx.x * kSub;
  const int nodes = min(kSub, geo.n[l0] - j0);
  const Tin* s = src + (int64_t)bh * src_bh_stride;
  float* P = pyr + (int64_t)bh * geo.Tp * D;
  bf16* R = reinterpret_cast<bf16*>(pyr + geo.means_floats()) + (int64_t)bh * geo.Tp * 2 * D;
  for (int jb0 = 0; jb0 < nodes; jb0 += kBuildNodes) {
    const int nb = min(kBuildNodes, nodes - jb0);
    float m[kBuildNodes];
    rows_mean_multi<Tin, D, FAN, kBuildNodes>(s, j0 + jb0, nb, src_rows, red, tid, m);
    if (tid < D) {
#pragma unroll
      for (int u = 0; u < kBuildNodes; ++u) {
        if (u >= nb) break;
        const int j = j0 + jb0 + u;
        P[(int64_t)(geo.off[l0] + j) * D + tid] = m[u];
        store_rcopy<D>(R, geo.off[l0] + j, tid, m[u] * geo.s_log2e);
        lvl[0][jb0 + u][tid] = m[u];  // read back only by this thread
      }
    }
  }
  __syncthreads();

  // Levels above l0 inside this subtree (g = 2): parents of [jbase, jbase + cnt).
  int cur = 0, cnt = nodes, jbase = j0;
  for (int l = l0 + 1; l <= geo.L && l <= l0 + kSubLevels; ++l) {
    const int pbase = jbase >> 1;
    const int pend = min(((jbase + cnt - 1) >> 1) + 1, geo.n[l]);
    const int pc = pend - pbase;
    if (tid < D) {
      for (int t = 0; t < pc; ++t) {
        const int p = pbase + t;
        const int c0 = 2 * p, c1 = min(2 * p + 2, geo.n[l - 1]);
        float a = 0.f;
        for (int c = c0; c < c1; ++c) a += lvl[cur][c - jbase][tid];
        const float m = a / (float)(c1 - c0);
        P[(int64_t)(geo.off[l] + p) * D + tid] = m;
        store_rcopy<D>(R, geo.off[l] + p, tid, m * geo.s_log2e);
        lvl[cur ^ 1][t][tid] = m;
      }
    }
    __syncthreads();
    cur ^= 1;
    cnt = pc;
    jbase = pbase;
  }
}

template <typename Tin, int D>
int build_t(const Geo& g, const Tin* k, float* pyr, hipStream_t st) {
  const int bhs = g.B * g.Hkv;
  for (int l0 = 1; l0 <= g.L; l0 += kSubLevels + 1) {
    dim3 grid((g.n[l0] + kSub - 1) / kSub, bhs);
    if (l0 == 1) {
      pyr_sub_kernel<Tin, D, kLeaf><<<grid, 256, 0, st>>>(k, (int64_t)g.N * D, g.N, pyr, g, 1);
    } else {
      const float* src = pyr + (int64_t)g.off[l0 - 1] * D;
      pyr_sub_kernel<float, D, 2><<<grid, 256, 0, st>>>(src, (int64_t)g.Tp * D, g.n[l0 - 1], pyr, g, l0);
    }
    if (hipGetLastError() != hipSuccess) return PISA_ERR_HIP;
  }
  return PISA_OK;
}

// ---- incremental append (a growing key cache; pyramid laid out for the capacity) ----
//
// "Block Sparse Attention with Log-Linear Complexity", agihunt.info summary, pyramid
// paragraph: a new key changes only its leaf block's mean and that block's ancestors, one
// node per level.  Sequence b grows from old_len[b] to new_len[b] keys; the leaf blocks
// holding positions old_len .. new_len - 1 are recomputed from their raw keys (rows_mean:
// the same bits as a fresh build), then every level above recomputes the ancestors of that
// block range from their children present at new_len, up to the capacity's top level (so
// levels that only a longer cache will walk are kept current too).

// Clamped dirty leaf-block range [*lo, *hi] of sequence b; false when nothing changed.
__device__ __forceinline__ bool dirty_blocks(const Geo& cap, const int32_t* old_len, const int32_t* new_len, int b,
                                             int max_blocks, int* len, int* lo, int* hi) {
  const int nl = min(max(new_len[b], 0), cap.N);
  const int ol = min(max(old_len[b], 0), nl);
  *len = nl;
  if (nl <= ol) return false;
  *lo = ol / cap.C;
  *hi = min((nl - 1) / cap.C, *lo + max_blocks - 1);
  return true;
}

template <typename Tin, int D>
__global__ __launch_bounds__(256) void append_leaf_kernel(const Tin* __restrict__ k, Geo cap,
                                                          const int32_t* __restrict__ old_len,
                                                          const int32_t* __restrict__ new_len, int32_t max_blocks,
                                                          float* __restrict__ pyr) {
  __shared__ float red[RowsShape<Tin, D>::RPP][D];
  const int tid = threadIdx.x, bh = blockIdx.y;
  int len, lo, hi;
  if (!dirty_blocks(cap, old_len, new_len, bh / cap.Hkv, max_blocks, &len, &lo, &hi)) return;  // whole workgroup
  const int j0 = lo + blockIdx.x * kSub;
  const Tin* s = k + (int64_t)bh * cap.N * D;
  float* P = pyr + (int64_t)bh * cap.Tp * D;
  bf16* R = reinterpret_cast<bf16*>(pyr + cap.means_floats()) + (int64_t)bh * cap.Tp * 2 * D;
  for (int j = j0; j < j0 + kSub && j <= hi; ++j) {
    const float m = rows_mean<Tin, D>(s, j * cap.C, min(j * cap.C + cap.C, len), red, tid);
    if (tid < D) {
      P[(int64_t)(cap.off[1] + j) * D + tid] = m;
      store_rcopy<D>(R, cap.off[1] + j, tid, m * cap.s_log2e);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void append_up_kernel(Geo cap, const int32_t* __restrict__ old_len,
                                                        const int32_t* __restrict__ new_len, int32_t max_blocks,
                                                        float* __restrict__ pyr) {
  const int tid = threadIdx.x, bh = blockIdx.x;
  int len, lo, hi;
  if (!dirty_blocks(cap, old_len, new_len, bh / cap.Hkv, max_blocks, &len, &lo, &hi)) return;  // whole workgroup
  float* P = pyr + (int64_t)bh * cap.Tp * D;
  bf16* R = reinterpret_cast<bf16*>(pyr + cap.means_floats()) + (int64_t)bh * cap.Tp * 2 * D;
  int nprev = (len + cap.C - 1) / cap.C;  // nodes of level l - 1 at this length
  for (int l = 2; l <= cap.L; ++l) {
    const int ncur = (nprev + 1) >> 1;
    const int plo = lo >> (l - 1), phi = hi >> (l - 1);
    for (int t = tid; t < (phi - plo + 1) * D; t += 256) {
      const int node = plo + t / D, e = t % D;
      if (node >= ncur) continue;
      const int c0 = 2 * node, c1 = min(2 * node + 2, nprev);
      float a = 0.f;
      for (int c = c0; c < c1; ++c) a += P[(int64_t)(cap.off[l - 1] + c) * D + e];
      const float m = a / (float)(c1 - c0);
      P[(int64_t)(cap.off[l] + node) * D + e] = m;
      store_rcopy<D>(R, cap.off[l] + node, e, m * cap.s_log2e);
    }
    __syncthreads();  // level l is complete before level l + 1 reads it (one CU, one L1)
    nprev = ncur;
  }
}

// One new key per sequence (max_new_keys == 1): the key's leaf block and its ancestors, one
// node per level, in one workgroup per (b, h).  A single leaf block changed, so the path's
// siblings are clean: each thread e < D loads element e of all of them before the first
// addition and carries the path's means in a register, with a fresh build's arithmetic
// (rows_mean for the leaf; a parent adds its children left to right and divides by their
// count), up to the capacity's top level as append_up_kernel does.
template <typename Tin, int D>
__global__ __launch_bounds__(256) void append_path_kernel(const Tin* __restrict__ k, Geo cap,
                                                          const int32_t* __restrict__ old_len,
                                                          const int32_t* __restrict__ new_len,
                                                          float* __restrict__ pyr) {
  __shared__ float red[RowsShape<Tin, D>::RPP][D];
  const int tid = threadIdx.x, bh = blockIdx.x;
  int len, lo, hi;
  if (!dirty_blocks(cap, old_len, new_len, bh / cap.Hkv, 1, &len, &lo, &hi)) return;  // whole workgroup
  float* P = pyr + (int64_t)bh * cap.Tp * D;
  bf16* R = reinterpret_cast<bf16*>(pyr + cap.means_floats()) + (int64_t)bh * cap.Tp * 2 * D;
  const int n1 = (len + cap.C - 1) / cap.C;  // leaf blocks at this length
  // sib[l]: element tid of the sibling of the path's level-l node (when it exists)
  float sib[kMaxLevels + 1];
  if (tid < D) {
    int np = n1, pth = lo;
#pragma unroll
    for (int l = 1; l <= kMaxLevels; ++l) {
      if (l < cap.L) {
        const int sb = pth ^ 1;
        sib[l] = sb < np ? P[(int64_t)(cap.off[l] + sb) * D + tid] : 0.f;
        np = (np + 1) >> 1;
        pth >>= 1;
      }
    }
  }
  float m = rows_mean<Tin, D>(k + (int64_t)bh * cap.N * D, lo * cap.C, min(lo * cap.C + cap.C, len), red, tid);
  if (tid < D) {
    P[(int64_t)(cap.off[1] + lo) * D + tid] = m;
    store_rcopy<D>(R, cap.off[1] + lo, tid, m * cap.s_log2e);
    int np = n1, pth = lo;
#pragma unroll
    for (int l = 2; l <= kMaxLevels; ++l) {
      if (l <= cap.L) {
        const int p = pth >> 1;
        const int cnt = min(2 * p + 2, np) - 2 * p;  // children of p at this length
        float a = 0.f;
        if (cnt == 2) {
          a += pth == 2 * p ? m : sib[l - 1];
          a += pth == 2 * p ? sib[l - 1] : m;
        } else {
          a += m;
        }
        m = a / (float)cnt;
        P[(int64_t)(cap.off[l] + p) * D + tid] = m;
        store_rcopy<D>(R, cap.off[l] + p, tid, m * cap.s_log2e);
        np = (np + 1) >> 1;
        pth = p;
      }
    }
  }
}

template <typename Tin, int D>
int append_t(const Geo& cap, const Tin* k, const int32_t* old_len, const int32_t* new_len, int max_new,
             float* pyr, hipStream_t st) {
  if (max_new == 1) {
    append_path_kernel<Tin, D><<<cap.B * cap.Hkv, 256, 0, st>>>(k, cap, old_len, new_len, pyr);
    return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
  }
  const int max_blocks = (max_new + cap.C - 1) / cap.C + 1;  // a range of max_new positions spans this many
  dim3 grid((max_blocks + kSub - 1) / kSub, cap.B * cap.Hkv);
  append_leaf_kernel<Tin, D><<<grid, 256, 0, st>>>(k, cap, old_len, new_len, max_blocks, pyr);
  if (hipGetLastError() != hipSuccess) return PISA_ERR_HIP;
  if (cap.L >= 2) {
    append_up_kernel<D><<<cap.B * cap.Hkv, 256, 0, st>>>(cap, old_len, new_len, max_blocks, pyr);
    if (hipGetLastError() != hipSuccess) return PISA_ERR_HIP;
  }
  return PISA_OK;
}

}  // namespace

int launch_append(const Geo& cap, int dtype, const void* k, const int32_t* old_len, const int32_t* new_len,
                  int max_new, float* pyr, hipStream_t st) {
  if (dtype == PISA_BF16) {
    if (cap.d == 128) return append_t<bf16, 128>(cap, (const bf16*)k, old_len, new_len, max_new, pyr, st);
    if (cap.d == 64) return append_t<bf16, 64>(cap, (const bf16*)k, old_len, new_len, max_new, pyr, st);
  } else {
    if (cap.d == 128) return append_t<float, 128>(cap, (const float*)k, old_len, new_len, max_new, pyr, st);
    if (cap.d == 64) return append_t<float, 64>(cap, (const float*)k, old_len, new_len, max_new, pyr, st);
  }
  return PISA_ERR_UNSUPPORTED;
}

int launch_build_pyramid(const Geo& g, int dtype, const void* k, float* pyr, hipStream_t st) {
  if (dtype == PISA_BF16) {
    if (g.d == 128) return build_t<bf16, 128>(g, (const bf16*)k, pyr, st);
    if (g.d == 64) return build_t<bf16, 64>(g, (const bf16*)k, pyr, st);
  } else {
    if (g.d == 128) return build_t<float, 128>(g, (const float*)k, pyr, st);
    if (g.d == 64) return build_t<float, 64>(g, (const float*)k, pyr, st);
  }
  return PISA_ERR_UNSUPPORTED;
}

}  // namespace pisa
