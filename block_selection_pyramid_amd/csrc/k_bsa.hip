// Full-scan BSA block selection, the baseline the pyramid selector is timed against
// ("Block Sparse Attention with Log-Linear Complexity": agihunt.info summary, opening and
// baselines paragraphs; rcap.io explainer, picking-step and comparison-point paragraphs):
// every query is scored against the mean-pooled summary of every causal key block, which
// costs O(N^2 / C), and the best blocks are kept.  Shared with the pyramid selector: the
// G heads of a GQA group sum their scores, the first, previous and current blocks are
// forced in, ties go to the lower block index.  A block's score is the plain dot product
// s<q, mean>; the forced blocks are not ranked and report +inf.
//
// The scan is a dense contraction on the matrix cores.  A workgroup holds the rows of QW
// consecutive queries of one (b, h) as B operands (32 (query, head) columns per column
// group) and streams the leaf-block summaries of the pyramid's hi/lo routing copy through
// LDS in tiles of 32 blocks (v_mfma_f32_32x32x16_bf16; hi and lo accumulate into one fp32
// result, so the products are the scores in log2 units).  After the head sum, a score
// enters its query's candidate list in LDS only if it beats the query's current K'-th
// best key (K' = K - 3 ranked blocks); a list that the next tile could overflow is cut
// back to its K' best by a rank count, which raises the threshold.  The output step
// merges the K' best with the forced blocks in ascending block order.
#include "route_dev.h"
#include "tile_dev.h"

namespace pisa {

namespace {

// Candidate-list capacity per query: K' kept keys plus one tile's worth of insertions.
template <int KC>
constexpr int bsa_cap() {
  return KC + 32;
}

template <int D, int G, int KC>
constexpr size_t bsa_lds_bytes() {
  return 2 * (size_t)(2 * (D / 16) * 1024) + (size_t)kDenseWaves * DenseShape<G>::QPW * (8 * bsa_cap<KC>() + 16);
}

__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int key_block(uint64_t key) { return (int)~(uint32_t)key; }

// Cuts a candidate list (n <= 64 keys, one per lane) back to its kp best; returns the
// new count.  Lane `rank == kp - 1` stores the kp-th best key as the new threshold.
__device__ __forceinline__ int bsa_compact(uint64_t* list, int32_t* cnt, uint64_t* thr, int kp, int lane) {
  const int n = *cnt;
  const uint64_t my = lane < n ? list[lane] : 0ull;
  int rank = 0;
  for (int u = 0; u < n; ++u) rank += list[u] > my;
  wave_sync();
  if (lane < n && rank < kp) list[rank] = my;
  if (lane < n && rank == kp - 1) *thr = my;
  const int m = min(n, kp);
  if (lane == 0) *cnt = m;
  wave_sync();
  return m;
}

template <int D, int G, int KC>
__global__ __launch_bounds__(256, 2) void bsa_kernel(const bf16* __restrict__ q, const float* __restrict__ pyr,
                                                     Geo geo, int32_t* __restrict__ out_idx,
                                                     float* __restrict__ out_score) {
  constexpr int NCG = DenseShape<G>::NCG, QPW = DenseShape<G>::QPW;
  constexpr int KS = D / 16;         // k-steps of 16 dims
  constexpr int F = 2 * KS;          // 1 KB fragments of a staged tile (hi, lo per k-step)
  constexpr int TILE = F * 1024;     // bytes of one staged tile of 32 summaries
  constexpr int CAP = bsa_cap<KC>();
  constexpr int QW = kDenseWaves * QPW;
  constexpr int GE = G < 16 ? G : 16, VPL = 16 / GE;  // lane r of a query's G lanes takes VPL values
  static_assert(CAP <= 64, "a candidate list fits one key per lane");

  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  char* wl = lds + 2 * TILE + wave * (QPW * (8 * CAP + 16));
  uint64_t* list = reinterpret_cast<uint64_t*>(wl);                      // [QPW][CAP]
  uint64_t* thr = reinterpret_cast<uint64_t*>(wl + QPW * 8 * CAP);       // [QPW]
  int32_t* cnt = reinterpret_cast<int32_t*>(wl + QPW * (8 * CAP + 8));   // [QPW]

  const int N = geo.N, C = geo.C, K = geo.K;
  const int kp = K - 3;  // ranked blocks of every query that has candidates (b >= 3)
  const int BH = geo.B * geo.Hkv;
  const int bh = blockIdx.x % BH;  // workgroups of one XCD (w mod 8) share few heads
  const int nchunk = (N + QW - 1) / QW;
  const int iwg = (nchunk - 1 - (int)(blockIdx.x / BH)) * QW;  // longest prefixes first
  const int iw = iwg + wave * QPW;
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  const int bqmax = (min(N, iwg + QW) - 1) / C;
  const char* Rb = reinterpret_cast<const char*>(pyr + geo.means_floats()) + (int64_t)bh * geo.Tp * (4 * D);

  const int j = lane & 31, hh = lane >> 5, r = j % G;
  bf16x8 qf[NCG][KS];
  int bqc[NCG];
  load_query_cols<D, G, NCG>(q, geo, b, h, iw, lane, qf, bqc);
  int last[NCG];  // last candidate block of the lane's query (candidates: 1 .. b - 2)
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) last[cg] = iw + cg * (32 / G) + j / G < N ? bqc[cg] - 2 : -1;

  if (lane < QPW) {
    cnt[lane] = 0;
    thr[lane] = 0ull;
  }
  wave_sync();
  uint64_t th[NCG];
  float thf[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    th[cg] = 0ull;
    thf[cg] = -INFINITY;
  }

  // tiles of 32 summaries covering the candidate blocks 1 .. bqmax - 2
  const int nt = (kp > 0 && bqmax >= 3) ? (bqmax - 2) / 32 + 1 : 0;
  u32x4 stg[F / kDenseWaves];
  if (nt > 0) {
    dense_load_tile<D>(Rb, geo, 2, 0, wave, lane, stg);
    dense_store_tile<D>(lds, 0, wave, lane, stg);
  }
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    // unconditional prefetch (the last tile reloads itself): a branch here would make the
    // compiler wait for each load in turn
    dense_load_tile<D>(Rb, geo, 2, min(t + 1, nt - 1), wave, lane, stg);
    const char* Tt = lds + (t & 1) * TILE;
    f32x16 acc[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[cg][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(Tt + ((2 * ks) * 64 + lane) * 16);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(Tt + ((2 * ks + 1) * 64 + lane) * 16);
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        acc[cg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qf[cg][ks], acc[cg], 0, 0, 0);
        acc[cg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qf[cg][ks], acc[cg], 0, 0, 0);
      }
    }
    // Epilogue.  Result row (block 32t + row) 8a + 4hh + v sits in acc[4a + v]; after the
    // head sum the G lanes of a query hold the same 16 values and lane r takes values
    // r*VPL .. r*VPL + VPL - 1.  A value whose score reaches the threshold's is keyed and
    // compared in full (rare once the list has filled).
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float sv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) sv[e] = group_sum<G>(acc[cg][e]);
      const int qi = cg * (32 / G) + j / G;
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        float v = sv[u];
#pragma unroll
        for (int k = 1; k < GE; ++k) v = r == k ? sv[k * VPL + u] : v;
        const int e = r * VPL + u;
        const int blk = 32 * t + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (blk >= 1 && blk <= last[cg] && v >= thf[cg]) {
          const uint64_t key = cand_key(v, blk);
          if (key > th[cg]) {
            const int pos = atomicAdd(&cnt[qi], 1);
            list[qi * CAP + pos] = key;
          }
        }
      }
    }
    wave_sync();
    // lists that the next tile could overflow are cut back to their kp best
    const unsigned long long full = __ballot(lane < QPW && cnt[lane] > CAP - 32);
    if (full) {
      for (unsigned long long m = full; m; m &= m - 1) {
        const int qi = __builtin_ctzll(m);
        bsa_compact(list + qi * CAP, cnt + qi, thr + qi, kp, lane);
      }
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        th[cg] = thr[cg * (32 / G) + j / G];
        thf[cg] = th[cg] ? key_score(th[cg]) : -INFINITY;
      }
    }
    if (t + 1 < nt) dense_store_tile<D>(lds, (t + 1) & 1, wave, lane, stg);
    __syncthreads();
  }

  // ---- output: forced blocks and the kp best candidates, ascending by block index
  const float ln2 = 0.6931471805599453f;
  for (int qi = 0; qi < QPW; ++qi) {
    const int i = iw + qi;
    if (i >= N) break;  // uniform across the wavefront
    const int bq = i / C;
    const int n = bsa_compact(list + qi * CAP, cnt + qi, thr + qi, kp, lane);
    const uint64_t* lq = list + qi * CAP;
    int32_t* oi = out_idx + ((int64_t)bh * N + i) * K;
    float* os = out_score + ((int64_t)bh * N + i) * K;
    const int nf = bq == 0 ? 1 : (bq == 1 ? 2 : 3);
    if (lane < n) {
      const uint64_t my = lq[lane];
      const int blk = key_block(my);
      int pos = 1;  // block 0 comes first; every candidate lies in 1 .. b - 2
      for (int u = 0; u < n; ++u) pos += key_block(lq[u]) < blk;
      oi[pos] = blk;
      os[pos] = key_score(my) * ln2;
    }
    if (lane == 32) {
      oi[0] = 0;
      os[0] = INFINITY;
    }
    if (lane == 33 && nf >= 2) {
      oi[1 + n] = bq >= 2 ? bq - 1 : bq;
      os[1 + n] = INFINITY;
    }
    if (lane == 34 && nf == 3) {
      oi[2 + n] = bq;
      os[2 + n] = INFINITY;
    }
    if (lane < K && lane >= nf + n) {  // K <= 32: lanes 32..34 never pad
      oi[lane] = -1;
      os[lane] = -INFINITY;
    }
  }
}

template <int D, int G, int KC>
int bsa_launch(const Geo& g, const bf16* q, const float* pyr, int32_t* oi, float* os, hipStream_t st) {
  constexpr int QW = kDenseWaves * DenseShape<G>::QPW;
  const unsigned grid = (unsigned)(g.B * g.Hkv * ((g.N + QW - 1) / QW));
  bsa_kernel<D, G, KC><<<grid, 64 * kDenseWaves, bsa_lds_bytes<D, G, KC>(), st>>>(q, pyr, g, oi, os);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

template <int D, int G>
int bsa_k(const Geo& g, const bf16* q, const float* pyr, int32_t* oi, float* os, hipStream_t st) {
  if (g.K - 3 <= 8) return bsa_launch<D, G, 8>(g, q, pyr, oi, os, st);
  if (g.K - 3 <= 16) return bsa_launch<D, G, 16>(g, q, pyr, oi, os, st);
  return bsa_launch<D, G, 32>(g, q, pyr, oi, os, st);
}

template <int D>
int bsa_g(const Geo& g, const bf16* q, const float* pyr, int32_t* oi, float* os, hipStream_t st) {
  switch (g.G) {
    case 1: return bsa_k<D, 1>(g, q, pyr, oi, os, st);
    case 2: return bsa_k<D, 2>(g, q, pyr, oi, os, st);
    case 4: return bsa_k<D, 4>(g, q, pyr, oi, os, st);
    case 8: return bsa_k<D, 8>(g, q, pyr, oi, os, st);
    case 16: return bsa_k<D, 16>(g, q, pyr, oi, os, st);
    default: return PISA_ERR_UNSUPPORTED;
  }
}

}  // namespace

int launch_bsa(const Geo& g, const void* q, const float* pyr, int32_t* out_idx, float* out_score, hipStream_t st) {
  if (g.K > 32) return PISA_ERR_UNSUPPORTED;
  if (g.d == 128) return bsa_g<128>(g, (const bf16*)q, pyr, out_idx, out_score, st);
  if (g.d == 64) return bsa_g<64>(g, (const bf16*)q, pyr, out_idx, out_score, st);
  return PISA_ERR_UNSUPPORTED;
}

}  // namespace pisa
