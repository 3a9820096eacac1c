// Query-major leaf scoring and the fused decode kernel.
//
// Query-major: one wavefront per query group gathers each of its candidate leaf tiles and
// the forced tiles and scores them on the VALU (lane = key).  This is the fp32-input
// prefill path (MFMA has no fp32 x fp32 form at the needed rate; fp32 inputs are the
// small correctness workloads).
//
// Decode ("Block Sparse Attention with Log-Linear Complexity", agihunt.info summary,
// kernels paragraph: a single-stage kernel for decode avoids launch overhead; rcap.io
// explainer: one query at a time leaves no cross-query tile reuse): one workgroup of 8
// wavefronts per (sequence, KV head).  All of them first load the query rows and stage
// the top pyramid levels' routing copy in LDS (one parallel burst).  bf16: wavefronts 0..3
// then walk the pyramid for the new query at position N-1 together, its top levels from
// LDS and two levels per round of gathers below them, each scoring a quarter of every
// round's tiles (MfmaWalk::pair_step_mw; wavefront 0 runs the Top-Ks), while wavefronts
// 4..6 hold the forced tiles' loads (known up front) and score them after the walk; fp32:
// wavefront 0 walks alone and wavefronts 1..3 score the forced tiles.  Then every
// wavefront scores two of the <= 2K routed tiles with both tiles' loads in flight together
// (bf16 on the matrix cores, 16 keys x 32 dims per MFMA against the G head columns), and
// wavefront 0 writes the selection.  One launch per step.  With
// per-sequence lengths each workgroup first re-derives its sequence's level table in LDS
// (node offsets stay those of the capacity layout that pisa_append_keys maintains).
#include <type_traits>

#include "final_dev.h"
#include "route_dev.h"

namespace pisa {

namespace {

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void qmajor_kernel(const T* __restrict__ q, const T* __restrict__ k, Geo geo,
                                                     const int32_t* __restrict__ cand, int32_t* __restrict__ out_idx,
                                                     float* __restrict__ out_score) {
  __shared__ float qs_all[4][G * (D + kQPad)];
  __shared__ float sc_all[4][kMaxCand + 4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave;
  const int bh = blockIdx.y;
  if (i >= geo.N) return;  // whole wavefront; no workgroup barrier follows
  float* qs = qs_all[wave];
  float* scs = sc_all[wave];
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  const T* rows[G];
#pragma unroll
  for (int r = 0; r < G; ++r) rows[r] = q + (((int64_t)b * geo.Hq + h * G + r) * geo.N + i) * D;
  load_qrows<T, D, G>(rows, qs, lane);
  wave_sync();

  const int bq = i / geo.C;
  int F[3];
  const int nf = forced_blocks(bq, F);
  const int twoK = 2 * geo.K;
  const int64_t row = (int64_t)bh * geo.N + i;
  const int leaf = lane < twoK ? cand[row * twoK + lane] : -1;
  const T* keys = k + (int64_t)bh * geo.N * D;
  for (int t = 0; t < twoK + nf; ++t) {
    const int j = t < twoK ? __shfl(leaf, t) : F[t - twoK];
    if (j < 0) continue;  // uniform across the wavefront
    const float s = score_tile_valu<T, D, G>(keys, j, i, geo.N, geo.C, qs, lane, geo.s);
    if (lane == 0) scs[t] = s;
  }
  wave_sync();
  const float sc = leaf >= 0 ? scs[lane] : -INFINITY;
  finalize_row(leaf, sc, F, nf, scs + twoK, geo.K, twoK, lane, out_idx + row * geo.K, out_score + row * geo.K);
}

// Eight wavefronts: the two-level gathers of the walk (pair_step) and two routed tiles per
// wavefront need up to 256 VGPRs per lane.
constexpr int kDecodeWaves = 8;
constexpr int64_t kDecodeStageBytes = 64 * 1024;  // LDS for the staged top levels

template <int D, int G>
struct DecodeLds {
  float qs[G * (D + kQPad)];
  WalkLds wl;
  WalkLdsM<1> wlm;
  int32_t tj[kMaxCand + 4];
  float tsc[kMaxCand + 4];
};

// The decode step for one (sequence, KV head) = blockIdx.x.  geo: the sequence's geometry
// (its length N and level table; node offsets, T and the batch shape of the buffers);
// kstride: key rows per (b, h) in k (the cache capacity).
template <typename T, int D, int G>
__device__ __forceinline__ void decode_body(const T* __restrict__ q, const T* __restrict__ k,
                                            const float* __restrict__ pyr, const Geo& geo, int64_t kstride,
                                            int stage_lo, char* stage, DecodeLds<D, G>& sh, int32_t* __restrict__ out_idx,
                                            float* __restrict__ out_score) {
  float* qs = sh.qs;
  WalkLds& wl = sh.wl;
  WalkLdsM<1>& wlm = sh.wlm;
  int32_t* tj = sh.tj;
  float* tsc = sh.tsc;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x;
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  const int i = geo.N - 1;
  const int bq = i / geo.C;
  int F[3];
  const int nf = forced_blocks(bq, F);
  const int twoK = 2 * geo.K;
  int leaf = -1;
  const T* rows[G];
#pragma unroll
  for (int r = 0; r < G; ++r) rows[r] = q + ((int64_t)b * geo.Hq + h * G + r) * D;

  // query rows (fp32 in LDS for the VALU scoring of fp32 inputs; the bf16 path reads its
  // MFMA fragments from q itself) and the staged top levels, by all wavefronts
  if constexpr (!std::is_same<T, bf16>::value) {
    constexpr int VEC = Vec<T>::N;
    constexpr int PER_ROW = D / VEC;
    for (int t = threadIdx.x; t < G * PER_ROW; t += 64 * kDecodeWaves) {
      const int r = t / PER_ROW, e = (t % PER_ROW) * VEC;
      float x[VEC];
      Vec<T>::load(q + ((int64_t)b * geo.Hq + h * G + r) * D + e, x);
#pragma unroll
      for (int v = 0; v < VEC; ++v) qs[r * (D + kQPad) + e + v] = x[v];
    }
  }
  const bf16* R = reinterpret_cast<const bf16*>(pyr + geo.means_floats()) + (int64_t)bh * geo.Tp * 2 * D;
  int sbase = 0;
  if constexpr (std::is_same<T, bf16>::value) {
    using Walk = MfmaWalk<D, G, 1>;
    sbase = stage_lo < geo.L ? geo.off[stage_lo] : 0;
    const int snodes = stage_lo < geo.L ? geo.off[geo.L] - sbase : 0;
    constexpr int kChunks = Walk::kRec / 16;  // 16-byte pieces per node
    constexpr int NT = 64 * kDecodeWaves;
    // every thread's pieces loaded before the first is stored: one round trip, not one per
    // piece (the staged levels fit kDecodeStageBytes, so kIt pieces per thread suffice)
    constexpr int kIt = (int)(((kDecodeStageBytes / Walk::kRecLds) * kChunks + NT - 1) / NT);
    const int npieces = snodes * kChunks;
    u32x4 v[kIt];
#pragma unroll
    for (int u = 0; u < kIt; ++u) {
      const int t = threadIdx.x + u * NT;
      v[u] = t < npieces ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(R) +
                                                          rc_piece_bytes(sbase + t / kChunks, t % kChunks, D))
                         : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kIt; ++u) {
      const int t = threadIdx.x + u * NT;
      if (t < npieces) *reinterpret_cast<u32x4*>(stage + (t / kChunks) * Walk::kRecLds + 16 * (t % kChunks)) = v[u];
    }
  }
  __syncthreads();

  const T* keys = k + (int64_t)bh * kstride * D;
  // one tile score into tsc[t], by the whole wavefront
  auto score_tile = [&](int t, int j) {
    float s;
    if constexpr (std::is_same<T, bf16>::value) {
      MfmaWalk<D, G, 1> tw;  // this wavefront's query fragments
      tw.load_q([&](int, int r) -> const bf16* { return rows[r]; }, lane);
      s = score_tile_mfma<D, G>(keys, j, i, geo.N, geo.C, tw.qb[0], lane, geo.s, geo.s_log2e);
    } else {
      s = score_tile_valu<T, D, G>(keys, j, i, geo.N, geo.C, qs, lane, geo.s);
    }
    if (lane == 0) tsc[t] = s;
  };
  if constexpr (std::is_same<T, bf16>::value) {
    // The walk on wavefronts 0..3 (each scoring a quarter of every step's tiles); the
    // forced tiles, known up front, on wavefronts 4..6: their loads go out before the walk
    // and are scored after it, so the walk's workgroup barriers never wait on them.
    using Walk = MfmaWalk<D, G, 1>;
    Walk mw;
    mw.R = R;
    mw.lds = stage;
    mw.stage_lo = stage_lo < geo.L ? stage_lo : 1 << 30;
    mw.stage_base = sbase;
    mw.load_q([&](int, int r) -> const bf16* { return rows[r]; }, lane);
    const int fw = wave - Walk::kWalkWaves;
    const bool fmine = fw >= 0 && fw < nf;
    const int fj[1] = {fmine ? (fw == 0 ? F[0] : (fw == 1 ? F[1] : F[2])) : -1};
    bf16x8 fa[1][4][D / 32];
    if (fmine) load_key_tiles<D, 1>(keys, fj, geo.N, geo.C, lane, fa);
    const int nx = mw.walk_pairs_mw(geo, bq, &wlm, lane, wave);
    if (wave == 0 && lane < twoK) {
      leaf = lane < nx ? wlm.X[lane] : -1;
      if (leaf >= 0 && is_forced(leaf, bq)) leaf = -1;
      tj[lane] = leaf;
    }
    if (fmine) {
      float fs[1];
      score_loaded_tiles<D, G, 1>(fa, fj, i, geo.N, geo.C, mw.qb[0], lane, geo.s, geo.s_log2e, fs);
      if (lane == 0) tsc[twoK + fw] = fs[0];
    }
  } else {
    if (wave == 0) {
      ValuScorer<D, G> sc{pyr + (int64_t)bh * geo.Tp * D, qs};
      const int nx = route_walk(geo, sc, bq, &wl, lane);
      if (lane < twoK) {
        leaf = lane < nx ? wl.X[lane] : -1;
        if (leaf >= 0 && is_forced(leaf, bq)) leaf = -1;
        tj[lane] = leaf;
      }
    } else if (wave <= nf) {
      // the forced tiles are known up front: wavefronts 1..nf score them during the walk
      score_tile(twoK + wave - 1, wave == 1 ? F[0] : (wave == 2 ? F[1] : F[2]));
    }
  }
  __syncthreads();
  // the routed leaf candidates (forced blocks excluded): tiles t and t + kDecodeWaves of a
  // wavefront scored together (bf16), so their loads are in flight at once
  for (int t = wave; t < twoK; t += 2 * kDecodeWaves) {
    const int t2 = t + kDecodeWaves;
    const int j0 = tj[t], j1 = t2 < twoK ? tj[t2] : -1;
    if constexpr (std::is_same<T, bf16>::value) {
      if (j0 >= 0 || j1 >= 0) {
        MfmaWalk<D, G, 1> tw;
        tw.load_q([&](int, int r) -> const bf16* { return rows[r]; }, lane);
        const int jt[2] = {j0, j1};
        float sc2[2];
        score_tiles_mfma<D, G, 2>(keys, jt, i, geo.N, geo.C, tw.qb[0], lane, geo.s, geo.s_log2e, sc2);
        if (lane == 0) {
          if (j0 >= 0) tsc[t] = sc2[0];
          if (j1 >= 0) tsc[t2] = sc2[1];
        }
      }
    } else {
      if (j0 >= 0) score_tile(t, j0);
      if (j1 >= 0) score_tile(t2, j1);
    }
  }
  __syncthreads();
  if (wave == 0) {
    const float sc = leaf >= 0 ? tsc[lane] : -INFINITY;
    finalize_row(leaf, sc, F, nf, tsc + twoK, geo.K, twoK, lane, out_idx + (int64_t)bh * geo.K,
                 out_score + (int64_t)bh * geo.K);
  }
}

// Level table of a sequence of n keys inside geometry g (whose node offsets, T and batch
// shape stay those of the buffers): n_0 = n, n_l = ceil halving, L = first level <= gK.
__device__ __forceinline__ void relevel(Geo& g, int n) {
  g.N = n;
  g.n[0] = n;
  int m = (n + g.C - 1) / g.C, L = 1;
  g.n[1] = m;
  while (m > g.g * g.K && L + 1 < kMaxLevels) {
    m = (m + 1) >> 1;
    g.n[++L] = m;
  }
  g.L = L;
  g.n1 = g.n[1];
}

// lengths == nullptr: every sequence holds geo.N keys.  Otherwise sequence b holds
// lengths[b] keys (clamped to [1, geo.N]) of a cache of capacity geo.N, and the pyramid is
// laid out for the capacity (pisa_append_keys).
template <typename T, int D, int G, bool VARLEN>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                   const float* __restrict__ pyr, Geo geo,
                                                                   const int32_t* __restrict__ lengths,
                                                                   int32_t stage_lo, int32_t* __restrict__ out_idx,
                                                                   float* __restrict__ out_score) {
  extern __shared__ __attribute__((aligned(16))) char stage[];  // bf16: levels [stage_lo, L-1]
  __shared__ DecodeLds<D, G> sh;
  if constexpr (VARLEN) {
    __shared__ Geo gs;
    if (threadIdx.x == 0) {
      gs = geo;
      relevel(gs, min(max(lengths[blockIdx.x / geo.Hkv], 1), geo.N));
    }
    __syncthreads();
    decode_body<T, D, G>(q, k, pyr, gs, geo.N, stage_lo, stage, sh, out_idx, out_score);
  } else {
    decode_body<T, D, G>(q, k, pyr, geo, geo.N, stage_lo, stage, sh, out_idx, out_score);
  }
}

template <typename T, int D>
int qmajor_g(const Geo& g, const void* q, const void* k, const int32_t* cand, int32_t* oi, float* os,
             hipStream_t st) {
  dim3 grid((g.N + 3) / 4, g.B * g.Hkv);
  const T* qq = (const T*)q;
  const T* kk = (const T*)k;
  switch (g.G) {
    case 1: qmajor_kernel<T, D, 1><<<grid, 256, 0, st>>>(qq, kk, g, cand, oi, os); break;
    case 2: qmajor_kernel<T, D, 2><<<grid, 256, 0, st>>>(qq, kk, g, cand, oi, os); break;
    case 4: qmajor_kernel<T, D, 4><<<grid, 256, 0, st>>>(qq, kk, g, cand, oi, os); break;
    case 8: qmajor_kernel<T, D, 8><<<grid, 256, 0, st>>>(qq, kk, g, cand, oi, os); break;
    case 16: qmajor_kernel<T, D, 16><<<grid, 256, 0, st>>>(qq, kk, g, cand, oi, os); break;
    default: return PISA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

template <typename T, int D, bool VARLEN>
int decode_g(const Geo& g, const void* q, const void* k, const float* pyr, const int32_t* lengths, int32_t* oi,
             float* os, hipStream_t st) {
  const unsigned grid = g.B * g.Hkv;
  const T* qq = (const T*)q;
  const T* kk = (const T*)k;
  // bf16: stage the levels >= 2 nearest the top whose routing-copy records fit the budget
  int stage_lo = g.L;
  int64_t bytes = 0;
  if (std::is_same<T, bf16>::value) {
    constexpr int64_t kRecLds = 4 * D + 16;
    while (stage_lo - 1 >= 2) {
      const int64_t add = (int64_t)g.n[stage_lo - 1] * kRecLds;
      if (bytes + add > kDecodeStageBytes) break;
      bytes += add;
      --stage_lo;
    }
  }
  const unsigned block = 64 * kDecodeWaves;
  switch (g.G) {
    case 1: decode_kernel<T, D, 1, VARLEN><<<grid, block, (size_t)bytes, st>>>(qq, kk, pyr, g, lengths, stage_lo, oi, os); break;
    case 2: decode_kernel<T, D, 2, VARLEN><<<grid, block, (size_t)bytes, st>>>(qq, kk, pyr, g, lengths, stage_lo, oi, os); break;
    case 4: decode_kernel<T, D, 4, VARLEN><<<grid, block, (size_t)bytes, st>>>(qq, kk, pyr, g, lengths, stage_lo, oi, os); break;
    case 8: decode_kernel<T, D, 8, VARLEN><<<grid, block, (size_t)bytes, st>>>(qq, kk, pyr, g, lengths, stage_lo, oi, os); break;
    case 16: decode_kernel<T, D, 16, VARLEN><<<grid, block, (size_t)bytes, st>>>(qq, kk, pyr, g, lengths, stage_lo, oi, os); break;
    default: return PISA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

}  // namespace

int launch_qmajor(const Geo& g, int dtype, const void* q, const void* k, const int32_t* cand, int32_t* out_idx,
                  float* out_score, hipStream_t st) {
  if (dtype == PISA_BF16) {
    if (g.d == 128) return qmajor_g<bf16, 128>(g, q, k, cand, out_idx, out_score, st);
    if (g.d == 64) return qmajor_g<bf16, 64>(g, q, k, cand, out_idx, out_score, st);
  } else {
    if (g.d == 128) return qmajor_g<float, 128>(g, q, k, cand, out_idx, out_score, st);
    if (g.d == 64) return qmajor_g<float, 64>(g, q, k, cand, out_idx, out_score, st);
  }
  return PISA_ERR_UNSUPPORTED;
}

template <bool VARLEN>
int decode_d(const Geo& g, int dtype, const void* q, const void* k, const float* pyr, const int32_t* lengths,
             int32_t* out_idx, float* out_score, hipStream_t st) {
  if (dtype == PISA_BF16) {
    if (g.d == 128) return decode_g<bf16, 128, VARLEN>(g, q, k, pyr, lengths, out_idx, out_score, st);
    if (g.d == 64) return decode_g<bf16, 64, VARLEN>(g, q, k, pyr, lengths, out_idx, out_score, st);
  } else {
    if (g.d == 128) return decode_g<float, 128, VARLEN>(g, q, k, pyr, lengths, out_idx, out_score, st);
    if (g.d == 64) return decode_g<float, 64, VARLEN>(g, q, k, pyr, lengths, out_idx, out_score, st);
  }
  return PISA_ERR_UNSUPPORTED;
}

int launch_decode(const Geo& g, int dtype, const void* q, const void* k, const float* pyr, const int32_t* lengths,
                  int32_t* out_idx, float* out_score, hipStream_t st) {
  return lengths ? decode_d<true>(g, dtype, q, k, pyr, lengths, out_idx, out_score, st)
                 : decode_d<false>(g, dtype, q, k, pyr, nullptr, out_idx, out_score, st);
}

}  // namespace pisa
