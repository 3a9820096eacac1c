// Pyramid construction ("Block Sparse Attention with Log-Linear Complexity", agihunt.info
// summary, pyramid paragraph; rcap.io explainer, "think of the keys as leaves of a tree"):
// level 1 node j = mean of the keys of leaf block j, level l node j = mean of level l-1
// nodes 2j, 2j+1 (g = 2), unweighted over the children that exist.  Every mean also goes
// to the routing copy, scaled by s log2(e) and split into bf16 hi + lo.
//
// One workgroup reduces a subtree: 16 consecutive nodes of level l0 (each the mean of
// `fan` rows of the level below: C raw keys for l0 = 1, g nodes above that) and then the
// up-to-4 levels above them from LDS.  For l0 = 1 the workgroup streams 16*C contiguous
// key rows with 16-byte loads (16 rows per pass for d = 128 bf16), so k is read from HBM
// exactly once.  A further launch with l0 = 6, 11, ... covers taller pyramids.
#include "dev_common.h"

namespace pisa {

namespace {

constexpr int kSub = 16;       // level-l0 nodes per workgroup
constexpr int kSubLevels = 4;  // levels built from LDS above l0 (log2 kSub)

template <typename Tin, int D>
__global__ __launch_bounds__(256) void pyr_sub_kernel(const Tin* __restrict__ src, int64_t src_bh_stride,
                                                      int32_t src_rows, int32_t fan, float* __restrict__ pyr,
                                                      Geo geo, int32_t l0) {
  constexpr int VEC = Vec<Tin>::N;
  constexpr int TPR = D / VEC;    // threads per row
  constexpr int RPP = 256 / TPR;  // rows per pass
  __shared__ float red[RPP][D];
  __shared__ float lvl[2][kSub][D];

  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int j0 = blockIdx.x * kSub;
  const int nodes = min(kSub, geo.n[l0] - j0);
  const Tin* s = src + (int64_t)bh * src_bh_stride;
  float* P = pyr + (int64_t)bh * geo.T * D;
  bf16* R = reinterpret_cast<bf16*>(pyr + geo.means_floats()) + (int64_t)bh * geo.T * 2 * D;
  const int cseg = tid % TPR, rp = tid / TPR;

  for (int jb = 0; jb < nodes; ++jb) {
    const int j = j0 + jb;
    const int r0 = j * fan;
    const int r1 = min(r0 + fan, src_rows);
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
    if (tid < D) {
      float t = 0.f;
#pragma unroll 8
      for (int p = 0; p < RPP; ++p) t += red[p][tid];
      const float m = t / (float)(r1 - r0);
      P[(int64_t)(geo.off[l0] + j) * D + tid] = m;
      store_rcopy<D>(R, geo.off[l0] + j, tid, m * geo.s_log2e);
      lvl[0][jb][tid] = m;
    }
    __syncthreads();
  }

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
      pyr_sub_kernel<Tin, D><<<grid, 256, 0, st>>>(k, (int64_t)g.N * D, g.N, g.C, pyr, g, 1);
    } else {
      const float* src = pyr + (int64_t)g.off[l0 - 1] * D;
      pyr_sub_kernel<float, D><<<grid, 256, 0, st>>>(src, (int64_t)g.T * D, g.n[l0 - 1], g.g, pyr, g, l0);
    }
    if (hipGetLastError() != hipSuccess) return PISA_ERR_HIP;
  }
  return PISA_OK;
}

}  // namespace

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
