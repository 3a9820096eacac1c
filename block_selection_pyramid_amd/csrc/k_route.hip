// Prefill routing (stage one of the two-stage prefill: walk levels L..2 per query group)
// plus the histogram of leaf candidates per (batch, KV head, leaf block) that the leaf
// grouping needs.  One wavefront per query group, four consecutive queries (same leaf
// block, hence the same visible pyramid) per workgroup.
//
// Output per query group: 2K slots of leaf candidates that are not forced blocks (the
// forced blocks are scored separately), -1 elsewhere.
#include "route_dev.h"

namespace pisa {

namespace {

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void route_kernel(const T* __restrict__ q, const float* __restrict__ pyr, Geo geo,
                                                    int32_t* __restrict__ cand, int32_t* __restrict__ cnt) {
  __shared__ float qs_all[4][G * (D + kQPad)];
  __shared__ WalkLds wl_all[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;
  const int bh = blockIdx.y;
  if (i >= geo.N) return;  // whole wavefront; no workgroup barrier follows
  float* qs = qs_all[wave];
  WalkLds* w = &wl_all[wave];
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;

  const T* rows[G];
#pragma unroll
  for (int r = 0; r < G; ++r) rows[r] = q + (((int64_t)b * geo.Hq + h * G + r) * geo.N + i) * D;
  load_qrows<T, D, G>(rows, qs, lane);
  wave_sync();

  const int bq = i / geo.C;
  const float* P = pyr + (int64_t)bh * geo.T * D;
  const int nx = route_walk<D, G>(geo, P, qs, bq, w, lane);

  const int twoK = 2 * geo.K;
  if (lane < twoK) {
    int leaf = lane < nx ? w->X[lane] : -1;
    if (leaf >= 0 && is_forced(leaf, bq)) leaf = -1;
    cand[((int64_t)bh * geo.N + i) * twoK + lane] = leaf;
    if (leaf >= 0) atomicAdd(&cnt[bh * geo.n1 + leaf], 1);
  }
}

template <typename T, int D>
int route_g(const Geo& g, const void* q, const float* pyr, int32_t* cand, int32_t* cnt, hipStream_t st) {
  dim3 grid((g.N + 3) / 4, g.B * g.Hkv);
  const T* qq = (const T*)q;
  switch (g.G) {
    case 1: route_kernel<T, D, 1><<<grid, 256, 0, st>>>(qq, pyr, g, cand, cnt); break;
    case 2: route_kernel<T, D, 2><<<grid, 256, 0, st>>>(qq, pyr, g, cand, cnt); break;
    case 4: route_kernel<T, D, 4><<<grid, 256, 0, st>>>(qq, pyr, g, cand, cnt); break;
    case 8: route_kernel<T, D, 8><<<grid, 256, 0, st>>>(qq, pyr, g, cand, cnt); break;
    case 16: route_kernel<T, D, 16><<<grid, 256, 0, st>>>(qq, pyr, g, cand, cnt); break;
    default: return PISA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

__global__ void zero_kernel(int32_t* __restrict__ a, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) a[t] = 0;
}

}  // namespace

int launch_route(const Geo& g, int dtype, const void* q, const float* pyr, int32_t* cand, int32_t* cnt,
                 hipStream_t st) {
  if (dtype == PISA_BF16) {
    if (g.d == 128) return route_g<bf16, 128>(g, q, pyr, cand, cnt, st);
    if (g.d == 64) return route_g<bf16, 64>(g, q, pyr, cand, cnt, st);
  } else {
    if (g.d == 128) return route_g<float, 128>(g, q, pyr, cand, cnt, st);
    if (g.d == 64) return route_g<float, 64>(g, q, pyr, cand, cnt, st);
  }
  return PISA_ERR_UNSUPPORTED;
}

int launch_zero(int32_t* a, int64_t n, hipStream_t st) {
  if (n <= 0) return PISA_OK;
  zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a, n);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

}  // namespace pisa
