// Leaf grouping: the second prefill stage collects the queries routed to one leaf block
// so that the block is scored for all of them at once ("Block Sparse Attention with
// Log-Linear Complexity", rcap.io explainer, kernel paragraph).  A counting sort: the routing kernel histograms the routed pairs per
// (batch, KV head, level-2 node), whose two children are adjacent leaf blocks that the
// prefill leaf kernel scores together; here an exclusive scan turns the counts into list
// offsets and into offsets of fixed-size work chunks, and a scatter writes each entry into
// its list.  Block-sparse attention sorts its (query, block) pairs by single leaf blocks
// with the same scan and scatter_hist_kernel / scatter_kernel.  Order inside a list does
// not affect any result: every entry's score is computed on its own and written back to
// its slot.
#include "dev_common.h"

namespace pisa {

namespace {

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ cnt, int32_t M, int32_t qc,
                                                            int32_t* __restrict__ off, int32_t* __restrict__ choff) {
  __shared__ int32_t s_e[kScanThreads], s_c[kScanThreads];
  const int t = threadIdx.x;
  const int per = (M + kScanThreads - 1) / kScanThreads;
  const int lo = min(M, t * per), hi = min(M, lo + per);
  int se = 0, sc = 0;
  for (int x = lo; x < hi; ++x) {
    const int c = cnt[x];
    se += c;
    sc += (c + qc - 1) / qc;
  }
  s_e[t] = se;
  s_c[t] = sc;
  __syncthreads();
  // inclusive Hillis-Steele scan of the per-thread sums
  for (int o = 1; o < kScanThreads; o <<= 1) {
    const int ae = t >= o ? s_e[t - o] : 0;
    const int ac = t >= o ? s_c[t - o] : 0;
    __syncthreads();
    s_e[t] += ae;
    s_c[t] += ac;
    __syncthreads();
  }
  int be = s_e[t] - se, bc = s_c[t] - sc;  // exclusive prefix of this thread's segment
  for (int x = lo; x < hi; ++x) {
    off[x] = be;
    choff[x] = bc;
    const int c = cnt[x];
    be += c;
    bc += (c + qc - 1) / qc;
  }
  if (t == kScanThreads - 1) {
    off[M] = s_e[t];
    choff[M] = s_c[t];
  }
}

// Lists are numbered (range, b h, block): query i belongs to range i / R (R a multiple of
// kLeafQueries; R >= N gives one range, list = bh * n1 + block).
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ cand, int64_t slots, int32_t N,
                                                      int32_t twoK, int32_t n1, int32_t BH, int32_t R,
                                                      const int32_t* __restrict__ off, int32_t* __restrict__ cursor,
                                                      int32_t* __restrict__ entries) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= slots) return;
  const int leaf = cand[t];
  if (leaf < 0) return;
  const int slot = (int)(t % twoK);
  const int64_t qg = t / twoK;  // bh * N + i
  const int bh = (int)(qg / N), i = (int)(qg % N);
  const int list = ((i / R) * BH + bh) * n1 + leaf;
  const int pos = off[list] + atomicAdd(&cursor[list], 1);
  entries[pos] = (i << 6) | slot;
}

// Workgroup = kLeafQueries consecutive queries of one (b, h): count its candidates per
// leaf block in LDS, reserve one range per non-empty block with a single returning global
// add, then place each entry with an LDS counter.
__global__ __launch_bounds__(256) void scatter_hist_kernel(const int32_t* __restrict__ cand, int32_t N, int32_t BH,
                                                           int32_t twoK, int32_t n1, int32_t R,
                                                           const int32_t* __restrict__ off,
                                                           int32_t* __restrict__ cursor,
                                                           int32_t* __restrict__ entries) {
  extern __shared__ int lds[];
  int* hist = lds;        // n1 counts, then reserved bases
  int* lcur = lds + n1;   // n1 local cursors
  const int bh0 = blockIdx.x % BH;
  const int q0 = (blockIdx.x / BH) * kLeafQueries;
  const int q1 = min(N, q0 + kLeafQueries);
  // the workgroup's queries share one range (R is a multiple of kLeafQueries): its lists
  // are those of "row" (range, b h)
  const int lrow = (q0 / R) * BH + bh0;
  for (int t = threadIdx.x; t < n1; t += 256) {
    hist[t] = 0;
    lcur[t] = 0;
  }
  __syncthreads();
  const int32_t* c = cand + ((int64_t)bh0 * N + q0) * twoK;
  const int n = (q1 - q0) * twoK;
  for (int t = threadIdx.x; t < n; t += 256) {
    const int leaf = c[t];
    if (leaf >= 0) atomicAdd(&hist[leaf], 1);
  }
  __syncthreads();
  for (int t = threadIdx.x; t < n1; t += 256) {
    const int h = hist[t];
    if (h) hist[t] = off[lrow * n1 + t] + atomicAdd(&cursor[lrow * n1 + t], h);
  }
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += 256) {
    const int leaf = c[t];
    if (leaf < 0) continue;
    const int pos = hist[leaf] + atomicAdd(&lcur[leaf], 1);
    entries[pos] = ((q0 + t / twoK) << 6) | (t % twoK);
  }
}

// Leaf-pair lists: the children 2m, 2m+1 of a kept level-2 node m sit in slots 2r, 2r+1
// of a query group's row (either may be -1: forced, not visible or missing).  Entry
// (i << 6 | r) goes to list m once when either slot holds a block.
__device__ __forceinline__ int pair_node(const int32_t* __restrict__ slots2) {
  const int a = slots2[0], c = slots2[1];
  return a >= 0 ? a >> 1 : (c >= 0 ? c >> 1 : -1);
}

__global__ __launch_bounds__(256) void scatter_pairs_kernel(const int32_t* __restrict__ cand, int64_t pairs,
                                                            int32_t N, int32_t K, int32_t n1p,
                                                            const int32_t* __restrict__ off,
                                                            int32_t* __restrict__ cursor,
                                                            int32_t* __restrict__ entries) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= pairs) return;
  const int node = pair_node(cand + 2 * t);
  if (node < 0) return;
  const int r = (int)(t % K);
  const int64_t qg = t / K;  // bh * N + i
  const int bh = (int)(qg / N), i = (int)(qg % N);
  const int list = bh * n1p + node;
  const int pos = off[list] + atomicAdd(&cursor[list], 1);
  entries[pos] = (i << 6) | r;
}

constexpr int kScatterBatch = 16;

// Workgroup = qpw consecutive queries of one (b, h), as scatter_hist_kernel, over level-2
// nodes.
__global__ __launch_bounds__(256) void scatter_pairs_hist_kernel(const int32_t* __restrict__ cand, int32_t N,
                                                                 int32_t BH, int32_t K, int32_t n1p, int32_t qpw,
                                                                 const int32_t* __restrict__ off,
                                                                 int32_t* __restrict__ cursor,
                                                                 int32_t* __restrict__ entries) {
  extern __shared__ int lds[];
  int* hist = lds;         // n1p counts, then reserved bases
  int* lcur = lds + n1p;   // n1p local cursors
  const int bh = blockIdx.x % BH;
  const int q0 = (blockIdx.x / BH) * qpw;
  const int q1 = min(N, q0 + qpw);
  for (int t = threadIdx.x; t < n1p; t += 256) {
    hist[t] = 0;
    lcur[t] = 0;
  }
  __syncthreads();
  const int32_t* c = cand + ((int64_t)bh * N + q0) * 2 * K;
  const int n = (q1 - q0) * K;
  // kScatterBatch pairs per thread at a time: their loads (and below, their returning
  // atomics) are all in flight before the first result is used (256K, batches of 1, 8,
  // 16 and 32: 140, 119, 112 and 113 us)
  for (int t0 = threadIdx.x; t0 < n; t0 += 256 * kScatterBatch) {
    int nd[kScatterBatch];
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u) nd[u] = t0 + 256 * u < n ? pair_node(c + 2 * (t0 + 256 * u)) : -1;
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u)
      if (nd[u] >= 0) atomicAdd(&hist[nd[u]], 1);
  }
  __syncthreads();
  for (int t0 = threadIdx.x; t0 < n1p; t0 += 256 * kScatterBatch) {
    int base[kScatterBatch];
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u) {
      const int t = t0 + 256 * u;
      const int h = t < n1p ? hist[t] : 0;
      base[u] = h ? off[bh * n1p + t] + atomicAdd(&cursor[bh * n1p + t], h) : 0;
    }
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u)
      if (t0 + 256 * u < n1p) hist[t0 + 256 * u] = base[u];
  }
  __syncthreads();
  for (int t0 = threadIdx.x; t0 < n; t0 += 256 * kScatterBatch) {
    int nd[kScatterBatch], pos[kScatterBatch];
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u) nd[u] = t0 + 256 * u < n ? pair_node(c + 2 * (t0 + 256 * u)) : -1;
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u) pos[u] = nd[u] >= 0 ? hist[nd[u]] + atomicAdd(&lcur[nd[u]], 1) : 0;
#pragma unroll
    for (int u = 0; u < kScatterBatch; ++u) {
      const int t = t0 + 256 * u;
      if (nd[u] >= 0) entries[pos[u]] = ((q0 + t / K) << 6) | (t % K);
    }
  }
}

// Workgroup = qpw consecutive queries of one (b, h): the leaf-pair histogram of
// their candidate slots, counted in LDS and flushed with one global add per non-empty
// node (direct global adds when the nodes do not fit).
__global__ __launch_bounds__(256) void count_pairs_kernel(const int32_t* __restrict__ cand, int32_t N, int32_t BH,
                                                          int32_t K, int32_t n1p, int32_t qpw,
                                                          int32_t* __restrict__ cnt) {
  extern __shared__ int hist[];
  const int bh = blockIdx.x % BH;
  const int q0 = (blockIdx.x / BH) * qpw;
  const int q1 = min(N, q0 + qpw);
  const bool lhist = n1p <= kHistMaxBins;
  if (lhist) {
    for (int t = threadIdx.x; t < n1p; t += 256) hist[t] = 0;
    __syncthreads();
  }
  const int32_t* c = cand + ((int64_t)bh * N + q0) * 2 * K;
  const int n = (q1 - q0) * K;
  for (int t = threadIdx.x; t < n; t += 256) {
    const int node = pair_node(c + 2 * t);
    if (node < 0) continue;
    if (lhist) atomicAdd(&hist[node], 1);
    else atomicAdd(&cnt[bh * n1p + node], 1);
  }
  if (lhist) {
    __syncthreads();
    for (int t = threadIdx.x; t < n1p; t += 256)
      if (hist[t]) atomicAdd(&cnt[bh * n1p + t], hist[t]);
  }
}

}  // namespace

int launch_count_pairs(const Geo& g, const int32_t* cand, int32_t* cnt, hipStream_t st) {
  const int qpw = group_queries(g);
  const unsigned grid = (unsigned)(g.B * g.Hkv * ((g.N + qpw - 1) / qpw));
  const size_t hbytes = g.n1p <= kHistMaxBins ? sizeof(int) * (size_t)g.n1p : 0;
  count_pairs_kernel<<<grid, 256, hbytes, st>>>(cand, g.N, g.B * g.Hkv, g.K, g.n1p, qpw, cnt);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

int launch_scatter_pairs(const Geo& g, const int32_t* cand, const int32_t* off, int32_t* cursor, int32_t* entries,
                         hipStream_t st) {
  if (g.n1p <= kHistMaxBins) {
    const int qpw = group_queries(g);
    const unsigned grid = (unsigned)(g.B * g.Hkv * ((g.N + qpw - 1) / qpw));
    scatter_pairs_hist_kernel<<<grid, 256, 2 * sizeof(int) * (size_t)g.n1p, st>>>(cand, g.N, g.B * g.Hkv, g.K,
                                                                                    g.n1p, qpw, off, cursor, entries);
    return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
  }
  const int64_t pairs = (int64_t)g.B * g.Hkv * g.N * g.K;
  scatter_pairs_kernel<<<(unsigned)((pairs + 255) / 256), 256, 0, st>>>(cand, pairs, g.N, g.K, g.n1p, off, cursor,
                                                                         entries);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

int launch_scan(const int32_t* cnt, int32_t M, int32_t qc, int32_t* off, int32_t* choff, hipStream_t st) {
  scan_kernel<<<1, kScanThreads, 0, st>>>(cnt, M, qc, off, choff);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

int launch_scatter(const Geo& g, int per_row, int32_t R, const int32_t* cand, const int32_t* off, int32_t* cursor,
                   int32_t* entries, hipStream_t st) {
  if (R <= 0 || R % kLeafQueries != 0) return PISA_ERR_INVALID_ARG;
  if (g.n1 <= kHistMaxBins) {
    const unsigned grid = (unsigned)(g.B * g.Hkv * ((g.N + kLeafQueries - 1) / kLeafQueries));
    scatter_hist_kernel<<<grid, 256, 2 * sizeof(int) * (size_t)g.n1, st>>>(cand, g.N, g.B * g.Hkv, per_row, g.n1,
                                                                            R, off, cursor, entries);
    return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
  }
  const int64_t slots = (int64_t)g.B * g.Hkv * g.N * per_row;
  scatter_kernel<<<(unsigned)((slots + 255) / 256), 256, 0, st>>>(cand, slots, g.N, per_row, g.n1, g.B * g.Hkv, R,
                                                                   off, cursor, entries);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

}  // namespace pisa
