// Prefill routing (stage one of the two-stage prefill: walk levels L..2 per query group)
// plus the histogram of routed (query group, level-2 node) pairs per (batch, KV head,
// level-2 node) that the leaf grouping needs.  bf16 inputs: the upper levels are scored
// densely per leaf block (separate launch, down to level 2 itself when there are at most
// kDenseMaxChildren leaf blocks), the levels below by per-query gathers on the matrix
// cores from the pyramid's hi/lo routing copy, up to four consecutive queries per
// wavefront; fp32 inputs: one wavefront per query group on the VALU for the whole walk.
//
// Output per query group: 2K slots of leaf candidates that are not forced blocks (the
// forced blocks are scored separately), -1 elsewhere; slots 2r and 2r+1 are the children
// of the kept level-2 node of rank r.
#include <type_traits>

#include "route_dev.h"

namespace pisa {

namespace {

constexpr int kLowerQueries = 512;  // queries per level-2 routing workgroup

// fp32 inputs: one wavefront per query group, VALU scorer.
template <int D, int G>
__global__ __launch_bounds__(256) void route_valu_kernel(const float* __restrict__ q, const float* __restrict__ pyr,
                                                         Geo geo, int32_t* __restrict__ cand) {
  __shared__ float qs_all[4][G * (D + kQPad)];
  __shared__ WalkLds wl_all[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;
  const int bh = blockIdx.y;
  if (i >= geo.N) return;  // whole wavefront; no workgroup barrier follows
  WalkLds* w = &wl_all[wave];
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  const float* rows[G];
#pragma unroll
  for (int r = 0; r < G; ++r) rows[r] = q + (((int64_t)b * geo.Hq + h * G + r) * geo.N + i) * D;
  const int bq = i / geo.C;
  float* qs = qs_all[wave];
  load_qrows<float, D, G>(rows, qs, lane);
  wave_sync();
  ValuScorer<D, G> sc{pyr + (int64_t)bh * geo.Tp * D, qs};
  const int nx = route_walk(geo, sc, bq, w, lane);
  const int twoK = 2 * geo.K;
  if (lane < twoK) {
    int leaf = lane < nx ? w->X[lane] : -1;
    if (leaf >= 0 && is_forced(leaf, bq)) leaf = -1;
    cand[((int64_t)bh * geo.N + i) * twoK + lane] = leaf;
  }
}

// bf16 inputs, the levels below the dense launch: each wavefront takes GPW query groups
// (consecutive queries of one leaf block) with their 2K candidates of level l_x -- written
// by the dense upper-level launch, or the visible prefix of level 2 when L == 2 -- and
// walks levels l_x .. 2 by per-query gathers of the child summaries from the routing copy
// (these levels are too wide to score densely: level 2's children are the leaf-block
// means), keeping the Top-K per level, then writes the leaf candidates that are not forced
// blocks.  The gathers read the hi halves only and re-score exactly just the candidates
// whose error bounds leave their membership open (MfmaWalk::walk_levels<true>).  Workgroup w
// serves (b, h) = w mod (B*Hkv), so the workgroups of one XCD (w mod 8) share few heads
// and gather from an L2-sized part of the routing copy.
template <int D, int G, int GPW>
__global__ __launch_bounds__(256) void route_mfma_kernel(const bf16* __restrict__ q, const float* __restrict__ pyr,
                                                         Geo geo, int32_t l_x, const int32_t* __restrict__ x2,
                                                         int32_t* __restrict__ cand, int32_t* __restrict__ cnt) {
  using Walk = MfmaWalk<D, G, GPW>;
  // per-level-2-node histogram (when the nodes fit), flushed with one global add per bin
  extern __shared__ __attribute__((aligned(16))) int hist[];
  __shared__ WalkLdsM<GPW> wl_all[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int BH = geo.B * geo.Hkv;
  const int bh = blockIdx.x % BH;
  const int qr0 = (blockIdx.x / BH) * kLowerQueries;
  const bool lhist = geo.n1p <= kHistMaxBins;
  if (lhist) {
    for (int t = threadIdx.x; t < geo.n1p; t += 256) hist[t] = 0;
    __syncthreads();
  }
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  Walk mw;
  mw.R = reinterpret_cast<const bf16*>(pyr + geo.means_floats()) + (int64_t)bh * geo.Tp * 2 * D;

  WalkLdsM<GPW>* w = &wl_all[wave];
  const int64_t qbase = ((int64_t)b * geo.Hq + h * G) * geo.N;
  const int twoK = 2 * geo.K;
  const int gl = lane / Walk::CW, xl = lane % Walk::CW;
  for (int quad = wave; quad < kLowerQueries / GPW; quad += 4) {
    const int i0 = qr0 + quad * GPW;
    if (i0 >= geo.N) break;  // uniform across the wavefront
    const int i = i0 + gl;   // this lane's query (for its group's slots)
    const int64_t row = (int64_t)bh * geo.N + i;
    const int bq = i0 / geo.C;  // GPW divides C: the wave's queries share one leaf block
    int nx;
    if (geo.L >= 2) {
      mw.load_q([&](int g, int r) -> const bf16* {
        const int ii = i0 + g;
        return ii < geo.N ? q + ((qbase + (int64_t)r * geo.N) + ii) * D : nullptr;
      }, lane);
      if (geo.L >= 3) {
        if (xl < twoK) w->X[gl * Walk::CW + xl] = i < geo.N ? __builtin_nontemporal_load(&x2[row * twoK + xl]) : -1;
        wave_sync();
        nx = twoK;
      } else {
        nx = mw.init_level(geo, bq, 2, w, lane);
      }
      nx = mw.template walk_levels<true>(geo, bq, geo.L >= 3 ? l_x : 2, 2, nx, w, lane);
    } else {
      nx = mw.init_level(geo, bq, 1, w, lane);
    }
    int leaf = -1;
    if (xl < twoK && i < geo.N) {
      leaf = xl < nx ? w->X[gl * Walk::CW + xl] : -1;
      if (leaf >= 0 && is_forced(leaf, bq)) leaf = -1;
      __builtin_nontemporal_store(leaf, &cand[row * twoK + xl]);
    }
    // slots 2r and 2r+1 hold the two children of one kept level-2 node (or -1): count the
    // pair once, in its even lane, under node = leaf >> 1
    const int sib = __shfl_xor(leaf, 1);
    if ((xl & 1) == 0 && (leaf >= 0 || sib >= 0)) {
      const int node = (leaf >= 0 ? leaf : sib) >> 1;
      if (lhist) atomicAdd(&hist[node], 1);
      else atomicAdd(&cnt[bh * geo.n1p + node], 1);
    }
    wave_sync();
  }
  if (lhist) {
    __syncthreads();
    for (int t = threadIdx.x; t < geo.n1p; t += 256)
      if (hist[t]) atomicAdd(&cnt[bh * geo.n1p + t], hist[t]);
  }
}

template <int D, int G, int GPW>
int route_mfma_launch(const Geo& g, const void* q, const void* k, const float* pyr, int32_t* x2, float* fsc,
                      int32_t* cand, int32_t* cnt, void* qg, uint8_t* lo8, hipEvent_t mid, hipStream_t st) {
  if (g.L >= 3) {
    // every routing level dense: the dense launch writes the leaf candidates
    const bool all_dense = dense_bottom(g) == 2;
    const int rc = launch_route_upper_dense(g, q, pyr, k, all_dense ? cand : x2, fsc, qg, st);
    if (rc != PISA_OK) return rc;
    if (all_dense) {
      if (mid && hipEventRecord(mid, st) != hipSuccess) return PISA_ERR_HIP;
      return launch_count_pairs(g, cand, cnt, st);
    }
  }
  if (mid && hipEventRecord(mid, st) != hipSuccess) return PISA_ERR_HIP;
  const unsigned grid = (unsigned)(g.B * g.Hkv * ((g.N + kLowerQueries - 1) / kLowerQueries));
  const size_t hbytes = g.n1p <= kHistMaxBins ? sizeof(int) * (size_t)g.n1p : 0;
  const int l_x = g.L >= 3 ? dense_bottom(g) - 1 : 2;  // level of the candidates in x2
  if (route_sub_supported(g, l_x)) return launch_route_sub(g, l_x, q, pyr, x2, cand, cnt, qg, lo8, st);
  route_mfma_kernel<D, G, GPW><<<grid, 256, hbytes, st>>>((const bf16*)q, pyr, g, l_x, x2, cand, cnt);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

template <int D, int G>
int route_mfma_g(const Geo& g, const void* q, const void* k, const float* pyr, int32_t* x2, float* fsc,
                 int32_t* cand, int32_t* cnt, void* qg, uint8_t* lo8, hipEvent_t mid, hipStream_t st) {
  const int gpw = route_groups_per_wave(g.G, g.K);
  if constexpr (G <= 4) {
    if (gpw == 4) return route_mfma_launch<D, G, 4>(g, q, k, pyr, x2, fsc, cand, cnt, qg, lo8, mid, st);
  }
  if constexpr (G <= 8) {
    if (gpw == 2) return route_mfma_launch<D, G, 2>(g, q, k, pyr, x2, fsc, cand, cnt, qg, lo8, mid, st);
  }
  return route_mfma_launch<D, G, 1>(g, q, k, pyr, x2, fsc, cand, cnt, qg, lo8, mid, st);
}

template <int D>
int route_d(const Geo& g, int dtype, const void* q, const void* k, const float* pyr, int32_t* x2, float* fsc,
            int32_t* cand, int32_t* cnt, void* qg, uint8_t* lo8, hipEvent_t mid, hipStream_t st) {
  if (dtype == PISA_BF16) {
    switch (g.G) {
      case 1: return route_mfma_g<D, 1>(g, q, k, pyr, x2, fsc, cand, cnt, qg, lo8, mid, st);
      case 2: return route_mfma_g<D, 2>(g, q, k, pyr, x2, fsc, cand, cnt, qg, lo8, mid, st);
      case 4: return route_mfma_g<D, 4>(g, q, k, pyr, x2, fsc, cand, cnt, qg, lo8, mid, st);
      case 8: return route_mfma_g<D, 8>(g, q, k, pyr, x2, fsc, cand, cnt, qg, lo8, mid, st);
      case 16: return route_mfma_g<D, 16>(g, q, k, pyr, x2, fsc, cand, cnt, qg, lo8, mid, st);
      default: return PISA_ERR_UNSUPPORTED;
    }
  }
  dim3 grid((g.N + 3) / 4, g.B * g.Hkv);
  const float* qq = (const float*)q;
  switch (g.G) {
    case 1: route_valu_kernel<D, 1><<<grid, 256, 0, st>>>(qq, pyr, g, cand); break;
    case 2: route_valu_kernel<D, 2><<<grid, 256, 0, st>>>(qq, pyr, g, cand); break;
    case 4: route_valu_kernel<D, 4><<<grid, 256, 0, st>>>(qq, pyr, g, cand); break;
    case 8: route_valu_kernel<D, 8><<<grid, 256, 0, st>>>(qq, pyr, g, cand); break;
    case 16: route_valu_kernel<D, 16><<<grid, 256, 0, st>>>(qq, pyr, g, cand); break;
    default: return PISA_ERR_UNSUPPORTED;
  }
  if (hipGetLastError() != hipSuccess) return PISA_ERR_HIP;
  return (mid && hipEventRecord(mid, st) != hipSuccess) ? PISA_ERR_HIP : PISA_OK;
}

__global__ void zero_kernel(int32_t* __restrict__ a, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) a[t] = 0;
}

}  // namespace

int launch_route(const Geo& g, int dtype, const void* q, const void* k, const float* pyr, int32_t* x2,
                 float* fsc, int32_t* cand, int32_t* cnt, void* qg, uint8_t* lo8, hipEvent_t mid, hipStream_t st) {
  if (g.d == 128) return route_d<128>(g, dtype, q, k, pyr, x2, fsc, cand, cnt, qg, lo8, mid, st);
  if (g.d == 64) return route_d<64>(g, dtype, q, k, pyr, x2, fsc, cand, cnt, qg, lo8, mid, st);
  return PISA_ERR_UNSUPPORTED;
}

int launch_zero(int32_t* a, int64_t n, hipStream_t st) {
  if (n <= 0) return PISA_OK;
  zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a, n);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

}  // namespace pisa
