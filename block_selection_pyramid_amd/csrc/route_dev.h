// The top-down pyramid walk for one query group, run by one wavefront.
//
// "Block Sparse Attention with Log-Linear Complexity": rcap.io explainer, top-down walk
// paragraph (score the candidates of a level, keep the Top-K, expand only their children,
// at most g*K candidates per level) and scoring paragraph (a candidate's score is the
// LogSumExp over its child summaries of q.child); agihunt.info summary, kernels paragraph
// (the G query heads of a GQA group share the selection: their per-head LSEs are summed).
// Under the PISA-1 / PISA-2 ablations the per-head LSE is replaced by its first- or
// second-order truncation about the children's mean (pair_trunc).
//
// Candidate x of a level owns child slots 2x and 2x+1 (g = 2).  Candidate ids live in LDS;
// -1 marks an empty slot (a child that does not exist or is not yet visible to the query).
// Top-K is a rank count over at most 64 candidates (score descending, block index
// ascending); the kept node of rank r expands into slots 2r, 2r+1 of the next level.
//
// bf16 inputs use MfmaWalk (matrix cores, several query groups per wavefront; the child
// summaries come from the pyramid's bf16 hi/lo routing copy of s log2(e) times the means,
// whose hi and lo accumulate into the same fp32 result, so a dot product is the scaled
// score in log2 units to 2^-18 relative).
// fp32 inputs use route_walk with ValuScorer: lane l scores child slot (l & 31) over half
// (l >> 5) of the head dimension for all G heads from the fp32 means and fp32 query rows
// in LDS.
#pragma once

#include "dev_common.h"

namespace pisa {

constexpr int kQPad = 4;  // floats of padding per query row in LDS (VALU scorer)

typedef __attribute__((ext_vector_type(4))) float f32x4;

// Per-wave LDS scratch of the walk.
struct WalkLds {
  int32_t X[kMaxCand];
  float cs[kMaxCand];
};

__device__ __forceinline__ bool child_visible(int c, int nchild, int cshift, int bq) {
  return c >= 0 && c < nchild && ((int64_t)c << cshift) <= bq;
}

// ---------------------------------------------------------------- MFMA walk
// Order-preserving 64-bit key of (score, node): larger key = better candidate (higher
// score, then lower index).  0 marks an empty slot (every real key is larger).
__device__ __forceinline__ uint64_t cand_key(float score, int node) {
  const uint32_t u = __float_as_uint(score);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(~(uint32_t)node);
}

template <int GPW>
struct alignas(16) WalkLdsM {  // 16-byte aligned: key arrays are read two keys at a time
  int32_t X[kMaxCand];   // GPW groups x (64 / GPW) candidate slots
  uint64_t key[kMaxCand];
  // bounded-approximation walk (walk_levels<true>): approximate scores and their error
  // bounds, candidate classes, and the uncertain candidates re-scored exactly
  float sc[kMaxCand], er[kMaxCand];
  int32_t cls[kMaxCand], U[kMaxCand];
  uint64_t key2[kMaxCand];
  int32_t nx_shared;  // the walk's candidate count, for the wavefronts that share a walk
};

// |lo| <= 2^-8 (1 + 2^-8) |hi| elementwise for hi = v rounded to nearest in bf16 and
// lo = v - hi rounded again, so |q.lo| <= this factor times |q|.|hi| (with slack for the
// fp32 accumulation of that product).
constexpr float kLoBound = 0.00393677f;  // 2^-8 (1 + 2^-7)

// One wavefront walks GPW query groups (consecutive queries of one (b, h), hence one
// leaf block and one visible pyramid) at once.  Scoring: v_mfma_f32_16x16x32_bf16 with
// A = 16 child summaries x 32 dims (bf16 hi, then lo, of the routing copy) and B = 32
// dims x 16 columns where column n carries head n % G of group n / G (k-step s, lane
// group kg = lane >> 4 <-> dims 32s + 8kg .. +8, for A and B alike).  Group g's MFMAs
// use a B that is zero outside its own columns, so all groups accumulate into one tile
// and every column of the result belongs to exactly one (group, head).  Lane l then holds
// (group, head) of column (l & 15) for child rows 4(l >> 4) + v; the pair LSE and the
// head sum run in the log2 domain with the native exp2/log2 (ranking is unchanged by the
// positive factor ln 2).  Ranking: lane l handles slot (l % (64/GPW)) of group
// l / (64/GPW) and counts the better keys of its group.
template <int D, int G, int GPW>
struct MfmaWalk {
  static constexpr int KS = D / 32;    // k-steps of 32 dims
  static constexpr int CW = 64 / GPW;  // candidate slots (lanes) per group
  static_assert(G * GPW <= 16, "one column per (group, head)");
  static constexpr int kRec = 4 * D;         // bytes of one node in the routing copy
  static constexpr int kRecLds = 4 * D + 16; // padded LDS record (spreads lanes over banks)
  const bf16* R;                       // routing copy of this (b, h)'s pyramid (global)
  const char* lds = nullptr;           // staged copy of levels [stage_lo, L-1], or null
  int stage_lo = 1 << 30;              // lowest level held in LDS
  int stage_base = 0;                  // node offset of stage_lo in the pyramid
  // Four groups per wavefront use the mixed-row tiles of score_m, whose B operand is each
  // lane's own query fragment: qb[0] only.  Fewer groups keep one zero-padded B per group.
  static constexpr bool kMixed = GPW == 4;
  bf16x8 qb[kMixed ? 1 : GPW][KS];

  // row(g, r): pointer to query head r of group g, or nullptr if the group is padding
  // (its columns stay zero; its results are never written).
  template <class RowFn>
  __device__ void load_q(RowFn row, int lane) {
    const int n = lane & 15, kg = lane >> 4;
    const int gown = n / G, r = n % G;
    if constexpr (kMixed) {
      const bf16* p = gown < GPW ? row(gown, r) : nullptr;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (p) {
          qb[0][s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p + 32 * s + 8 * kg));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qb[0][s][e] = (__bf16)0.f;
        }
      }
      return;
    }
#pragma unroll
    for (int g = 0; g < (kMixed ? 1 : GPW); ++g) {
      const bf16* p = (g == gown) ? row(g, r) : nullptr;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (p) {
          // streamed once: keep query rows from displacing the pyramid in L2
          qb[g][s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p + 32 * s + 8 * kg));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qb[g][s][e] = (__bf16)0.f;
        }
      }
    }
  }

  // Loads of one batch: TB tiles x GPW groups, all issued before the first MFMA.  An
  // invisible or missing child reads node 0 of the level instead (always present); its
  // rows are masked to -inf in the epilogue, so the loads need no branches.
  static constexpr int TB = GPW == 1 ? 2 : 1;  // tiles per batch

  template <bool kLds, bool kLo>
  __device__ __forceinline__ void load_batch(const Geo& geo, const char* Lc, int bq, int l,
                                             int nx, int t0, const int32_t* Xs, int lane,
                                             bf16x8 (&hi)[GPW][TB][KS], bf16x8 (&lo)[GPW][TB][KS]) const {
    const int nchild = geo.n[l - 1];
    const int cshift = l - 2;
    const int m = lane & 15, kg = lane >> 4;
    int ca[GPW][TB];
#pragma unroll
    for (int g = 0; g < GPW; ++g)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int cs = 16 * (t0 + tb) + m;
        const int xa = cs >> 1;
        const int na = xa < nx ? Xs[g * CW + xa] : -1;
        const int c = na >= 0 ? 2 * na + (cs & 1) : -1;
        ca[g][tb] = child_visible(c, nchild, cshift, bq) ? c : 0;
      }
#pragma unroll
    for (int g = 0; g < GPW; ++g)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        // k-step s, lane group kg <-> dims 32s + 8kg .. +8: the four lanes of a row read 64
        // contiguous bytes of one 128-byte chunk per instruction
        if constexpr (kLds) {
          const char* rp = Lc + (int64_t)ca[g][tb] * kRecLds + 16 * kg;
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            hi[g][tb][s] = *reinterpret_cast<const bf16x8*>(rp + 128 * s);
            if constexpr (kLo) lo[g][tb][s] = *reinterpret_cast<const bf16x8*>(rp + 128 * s + 64);
          }
        } else {
          const bf16* rp = R + rc_node(geo.off[l - 1] + ca[g][tb], D) + rc_piece(kg);  // piece 4 s + kg
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            hi[g][tb][s] = *reinterpret_cast<const bf16x8*>(rp + 256 * s);
            if constexpr (kLo) lo[g][tb][s] = *reinterpret_cast<const bf16x8*>(rp + 256 * s + 64);
          }
        }
      }
  }

  // Scores candidates Xs[g*CW + 0..nx) of level l (>= 2) into keys[].  kApprox: from the
  // hi halves only, also writing each candidate's approximate score to sc[] and a bound on
  // its distance from the hi + lo score to er[] (the MFMA of |hi| against |q| takes the
  // place of the lo one, and the lo halves are not read).
  template <bool kLds, bool kApprox>
  __device__ void score_t(const Geo& geo, int bq, int l, int nx, const int32_t* Xs, uint64_t* keys, float* sc,
                          float* er, int lane) const {
    const char* Lc = kLds ? lds + (int64_t)(geo.off[l - 1] - stage_base) * kRecLds : nullptr;
    const int nchild = geo.n[l - 1];
    const int cshift = l - 2;
    const int m = lane & 15, kg = lane >> 4;
    const int gown = m / G, r = m % G;  // epilogue: this lane's column = (group, head)
    const int ntiles = (2 * nx + 15) >> 4;
    for (int t0 = 0; t0 < ntiles; t0 += TB) {
      bf16x8 hi[GPW][TB][KS], lo[GPW][TB][KS];
      load_batch<kLds, !kApprox>(geo, Lc, bq, l, nx, t0, Xs, lane, hi, lo);
      // every load of the batch goes out before the first MFMA: left to itself the compiler
      // interleaves them with the products and waits on the first few, so one level costs
      // several round trips to L2 or HBM instead of one (G <= 4: with more heads per group
      // the decode kernel would spill)
      if constexpr (G <= 4) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int t = t0 + tb;
        if (t >= ntiles) break;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < GPW; ++g)
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[g][tb][s], qb[kMixed ? 0 : g][s], acc, 0, 0, 0);
            if constexpr (kApprox) {
              // |hi| and |q|: clear the bf16 sign bits (|q| formed at each use: keeping it
              // for the whole walk would cost a wavefront per SIMD)
              u32x4 qa = __builtin_bit_cast(u32x4, qb[kMixed ? 0 : g][s]);
              asm volatile("" : "+v"(qa));
              qa &= 0x7FFF7FFFu;
              const u32x4 ha = __builtin_bit_cast(u32x4, hi[g][tb][s]) & 0x7FFF7FFFu;
              acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ha),
                                                             __builtin_bit_cast(bf16x8, qa), acc2, 0, 0, 0);
            } else {
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[g][tb][s], qb[kMixed ? 0 : g][s], acc, 0, 0, 0);
            }
          }
        float lse[2], err[2];
        int node[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int x = 8 * t + 2 * kg + p;  // candidate owning child rows 4kg + 2p, +1
          node[p] = (gown < GPW && x < nx) ? Xs[gown * CW + x] : -1;
          float y[2], bnd[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int ch = node[p] >= 0 ? 2 * node[p] + c : -1;
            const bool vis = child_visible(ch, nchild, cshift, bq);
            y[c] = vis ? acc[2 * p + c] : -INFINITY;
            bnd[c] = vis ? acc2[2 * p + c] : 0.f;
          }
          const float a = fmaxf(y[0], y[1]), b = fminf(y[0], y[1]);
          const float v = geo.scorer == PISA_LSE ? a + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(b - a))
                                                 : pair_trunc(a, b, 1.f, trunc_c2(geo.scorer, true));
          lse[p] = node[p] >= 0 ? v : 0.f;
          // the pair LSE moves by at most the larger child error; 2^-20 |score| more covers
          // the differing fp32 rounding of the two evaluations
          err[p] = node[p] >= 0 ? kLoBound * fmaxf(bnd[0], bnd[1]) + 9.6e-7f * fabsf(v) : 0.f;
        }
        lse[0] = group_sum<G>(lse[0]);
        lse[1] = group_sum<G>(lse[1]);
        if constexpr (kApprox) {
          err[0] = group_sum<G>(err[0]);
          err[1] = group_sum<G>(err[1]);
        }
        if (r == 0 && gown < GPW) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int x = 8 * t + 2 * kg + p;
            if (x < nx) {
              keys[gown * CW + x] = node[p] >= 0 ? cand_key(lse[p], node[p]) : 0ull;
              if constexpr (kApprox) {
                sc[gown * CW + x] = lse[p];
                er[gown * CW + x] = err[p];
              }
            }
          }
        }
      }
    }
    wave_sync();
  }

  // score_t for four groups per wavefront with mixed-row tiles.  Tile j (16 child rows)
  // holds in row block rb (rows 4rb .. 4rb+3) the slots 4j .. 4j+3 (candidates 2j, 2j+1,
  // two children each) of group (rb + j) mod 4, so one MFMA chain per tile takes every
  // lane's own query fragment as B (no zero columns).  The MFMA result lane for column
  // (gown, r) and row block kg = lane >> 4 holds its own group's rows in the tiles with
  // j = gown - kg (mod 4): one tile of every four.  A level of nx candidates per group
  // takes ceil(nx / 2) tiles; the hi-only pass loads two tiles per batch, the exact pass
  // (hi + lo) one.
  template <bool kLds, bool kApprox>
  __device__ void score_m(const Geo& geo, int bq, int l, int nx, const int32_t* Xs, uint64_t* keys, float* sc,
                          float* er, int lane) const {
    static_assert(GPW == 4, "mixed-row tiles rotate four groups over four row blocks");
    // tiles per batch: small batches keep the launch at 126 VGPRs, four wavefronts per SIMD
    // (256K, gather launch: hi-only batches of 2 and exact ones of 1 tile took 3.05 ms, 2/2
    // 3.10, 1/1 3.13, 4/2 (three wavefronts per SIMD) 3.17, 8/2 3.37)
    constexpr int TBM = kApprox ? 2 : 1;
    const char* Lc = kLds ? lds + (int64_t)(geo.off[l - 1] - stage_base) * kRecLds : nullptr;
    const int nchild = geo.n[l - 1];
    const int cshift = l - 2;
    const int m = lane & 15, kg = lane >> 4;
    const int gown = m / G, r = m % G;     // epilogue: this lane's column = (group, head)
    const int rb = m >> 2, v = m & 3;      // loads: this lane's A row = row block, row in it
    const int jo = (gown - kg) & 3;        // epilogue: tiles j = jo (mod 4) hold this lane's rows
    const int ntiles = (nx + 1) >> 1;
    for (int j0 = 0; j0 < ntiles; j0 += TBM) {
      bf16x8 hi[TBM][KS], lo[TBM][KS];
      // An invisible or missing child reads node 0 of the level instead (always present);
      // its rows are masked to -inf in the epilogue, so the loads need no branches.
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) {
        const int j = j0 + tb;
        const int ga = (rb + j) & 3;
        const int x = 2 * j + (v >> 1);
        const int na = x < nx ? Xs[ga * CW + x] : -1;
        const int c = na >= 0 ? 2 * na + (v & 1) : -1;
        const int ca = child_visible(c, nchild, cshift, bq) ? c : 0;
        if constexpr (kLds) {
          const char* rp = Lc + (int64_t)ca * kRecLds + 16 * kg;
#pragma unroll
          for (int s2 = 0; s2 < KS; ++s2) {
            hi[tb][s2] = *reinterpret_cast<const bf16x8*>(rp + 128 * s2);
            if constexpr (!kApprox) lo[tb][s2] = *reinterpret_cast<const bf16x8*>(rp + 128 * s2 + 64);
          }
        } else {
          const bf16* rp = R + rc_node(geo.off[l - 1] + ca, D) + rc_piece(kg);  // piece 4 s2 + kg
#pragma unroll
          for (int s2 = 0; s2 < KS; ++s2) {
            hi[tb][s2] = *reinterpret_cast<const bf16x8*>(rp + 256 * s2);
            if constexpr (!kApprox) lo[tb][s2] = *reinterpret_cast<const bf16x8*>(rp + 256 * s2 + 64);
          }
        }
      }
      f32x4 acc[TBM], acc2[TBM];
#pragma unroll
      for (int tb = 0; tb < TBM; ++tb) {
        acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc2[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[tb][s2], qb[0][s2], acc[tb], 0, 0, 0);
          if constexpr (kApprox) {
            // |hi| and |q|: clear the bf16 sign bits (|q| formed at each use)
            u32x4 qa = __builtin_bit_cast(u32x4, qb[0][s2]);
            asm volatile("" : "+v"(qa));
            qa &= 0x7FFF7FFFu;
            const u32x4 ha = __builtin_bit_cast(u32x4, hi[tb][s2]) & 0x7FFF7FFFu;
            acc2[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ha),
                                                               __builtin_bit_cast(bf16x8, qa), acc2[tb], 0, 0, 0);
          } else {
            acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[tb][s2], qb[0][s2], acc[tb], 0, 0, 0);
          }
        }
      }
      // this lane's tile in each run of four tiles of the batch (if any): j = jo (mod 4)
#pragma unroll
      for (int sb = 0; sb < (TBM + 3) / 4; ++sb) {
        const int jj = (jo - j0) & 3;
        const int j = j0 + 4 * sb + jj;
        const bool mine = jj < (TBM < 4 ? TBM : 4) && j < ntiles;
        f32x4 a = acc[4 * sb], a2 = acc2[4 * sb];
#pragma unroll
        for (int tb = 1; tb < (TBM < 4 ? TBM : 4); ++tb) {
          a = jj == tb ? acc[4 * sb + tb] : a;
          a2 = jj == tb ? acc2[4 * sb + tb] : a2;
        }
        float lse[2], err[2];
        int node[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int x = 2 * j + p;  // candidate owning result rows 4kg + 2p, +1
          node[p] = (mine && gown < GPW && x < nx) ? Xs[gown * CW + x] : -1;
          float y[2], bnd[2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int ch = node[p] >= 0 ? 2 * node[p] + c : -1;
            const bool vis = child_visible(ch, nchild, cshift, bq);
            y[c] = vis ? a[2 * p + c] : -INFINITY;
            bnd[c] = vis ? a2[2 * p + c] : 0.f;
          }
          const float va = fmaxf(y[0], y[1]), vb = fminf(y[0], y[1]);
          const float vv = geo.scorer == PISA_LSE ? va + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(vb - va))
                                                  : pair_trunc(va, vb, 1.f, trunc_c2(geo.scorer, true));
          lse[p] = node[p] >= 0 ? vv : 0.f;
          // the pair LSE moves by at most the larger child error; 2^-20 |score| more covers
          // the differing fp32 rounding of the two evaluations
          err[p] = node[p] >= 0 ? kLoBound * fmaxf(bnd[0], bnd[1]) + 9.6e-7f * fabsf(vv) : 0.f;
        }
        lse[0] = group_sum<G>(lse[0]);
        lse[1] = group_sum<G>(lse[1]);
        if constexpr (kApprox) {
          err[0] = group_sum<G>(err[0]);
          err[1] = group_sum<G>(err[1]);
        }
        if (r == 0 && gown < GPW && mine) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int x = 2 * j + p;
            if (x < nx) {
              keys[gown * CW + x] = node[p] >= 0 ? cand_key(lse[p], node[p]) : 0ull;
              if constexpr (kApprox) {
                sc[gown * CW + x] = lse[p];
                er[gown * CW + x] = err[p];
              }
            }
          }
        }
      }
    }
    wave_sync();
  }

  template <bool kApprox>
  __device__ void score(const Geo& geo, int bq, int l, int nx, const int32_t* Xs, uint64_t* keys, float* sc,
                        float* er, int lane) const {
    if constexpr (kMixed) {
      if (l - 1 >= stage_lo)
        score_m<true, kApprox>(geo, bq, l, nx, Xs, keys, sc, er, lane);
      else
        score_m<false, kApprox>(geo, bq, l, nx, Xs, keys, sc, er, lane);
    } else {
      if (l - 1 >= stage_lo)
        score_t<true, kApprox>(geo, bq, l, nx, Xs, keys, sc, er, lane);
      else
        score_t<false, kApprox>(geo, bq, l, nx, Xs, keys, sc, er, lane);
    }
  }

  // Fills X with the visible nodes of level `l` (a prefix of the level) and returns nx.
  __device__ int init_level(const Geo& geo, int bq, int l, WalkLdsM<GPW>* w, int lane) const {
    const int xl = lane % CW, gl = lane / CW;
    const int nx = l == 1 ? bq + 1 : min(geo.n[l], (bq >> (l - 1)) + 1);
    if (xl < nx) w->X[gl * CW + xl] = xl;
    wave_sync();
    return nx;
  }

  // Walks levels l_top down to l_bot (>= 2): score, keep Top-K, expand.  X must hold the
  // candidates of level l_top (nx slots per group).  On return X[g*CW + 0..nx) holds the
  // candidates of level l_bot - 1 and the function returns their slot count (<= 2K).
  //
  // kApprox (LSE scorer only): each level is first scored from the hi halves with error
  // bounds (score_t<., true>).  A candidate is surely kept when fewer than K others could
  // score above it within the bounds, surely dropped when K others surely score above it,
  // and uncertain otherwise; only the uncertain ones are scored again exactly (hi + lo),
  // and the K - (surely kept) best of them by exact score are kept.  The kept set is the
  // one exact scoring gives, at about half the gathered bytes.
  template <bool kApprox = false>
  __device__ int walk_levels(const Geo& geo, int bq, int l_top, int l_bot, int nx, WalkLdsM<GPW>* w,
                             int lane) const {
    const int K = geo.K;
    const int gl = lane / CW, xl = lane % CW;
    int* Xg = w->X + gl * CW;
    const bool approx = kApprox && geo.scorer == PISA_LSE;
    for (int l = l_top; l >= l_bot; --l) {
      const uint64_t* kg = w->key + gl * CW;
      uint64_t my;
      int rank = 0;
      if (approx) {
        score<true>(geo, bq, l, nx, w->X, w->key, w->sc, w->er, lane);
        const float* sg = w->sc + gl * CW;
        const float* eg = w->er + gl * CW;
        my = xl < nx ? kg[xl] : 0ull;
        const float lo_x = xl < nx ? sg[xl] - eg[xl] : 0.f, up_x = xl < nx ? sg[xl] + eg[xl] : 0.f;
        int may = 0, sure = 0;  // others that may / surely score above this candidate
#pragma unroll 8
        for (int y = 0; y < nx; ++y) {  // branch-free and unrolled: the LDS reads go out together
          const bool other = y != xl && kg[y] != 0ull;
          const float sy = sg[y], ey = eg[y];
          may += other && sy + ey >= lo_x;
          sure += other && sy - ey > up_x;
        }
        const int cls = my == 0ull ? -1 : (may < K ? 2 : (sure >= K ? 0 : 1));
        const unsigned long long unc = __ballot(cls == 1);
        if (unc) {
          // compact each group's uncertain candidates and score them exactly
          const unsigned long long gm = (GPW == 1) ? ~0ull : (((1ull << CW) - 1ull) << (gl * CW));
          const int pos = (int)__popcll(unc & gm & ((1ull << lane) - 1ull));
          int nu = 0;
#pragma unroll
          for (int g = 0; g < GPW; ++g) {
            const unsigned long long gmg = (GPW == 1) ? ~0ull : (((1ull << CW) - 1ull) << (g * CW));
            nu = max(nu, (int)__popcll(unc & gmg));
          }
          w->U[lane] = -1;
          wave_sync();
          if (cls == 1) w->U[gl * CW + pos] = Xg[xl];
          wave_sync();
          score<false>(geo, bq, l, nu, w->U, w->key2, nullptr, nullptr, lane);
          if (cls == 1) my = w->key2[gl * CW + pos];
        }
        w->cls[lane] = cls;
        wave_sync();
        w->key[lane] = xl < nx ? my : 0ull;
        wave_sync();
        const int32_t* cg = w->cls + gl * CW;
#pragma unroll 8
        for (int y = 0; y < nx; ++y) rank += cg[y] > cls || (cg[y] == cls && kg[y] > my);
      } else {
        score<false>(geo, bq, l, nx, w->X, w->key, nullptr, nullptr, lane);
        my = xl < nx ? kg[xl] : 0ull;
#pragma unroll 8
        for (int y = 0; y < nx; ++y) rank += kg[y] > my;  // unrolled: the LDS reads go out together
      }
      const int myid = xl < nx ? Xg[xl] : -1;
      const unsigned long long live = __ballot(my != 0ull);
      int nkg = 0, nmax = 0;
#pragma unroll
      for (int g = 0; g < GPW; ++g) {
        const unsigned long long gm = (GPW == 1) ? ~0ull : (((1ull << CW) - 1ull) << (g * CW));
        const int kept = min(K, (int)__popcll(live & gm));
        if (g == gl) nkg = kept;
        nmax = max(nmax, kept);
      }
      wave_sync();
      const int nchild = geo.n[l - 1];
      const int cshift = l - 2;
      if (my != 0ull && rank < K) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int ch = 2 * myid + c;
          Xg[2 * rank + c] = child_visible(ch, nchild, cshift, bq) ? ch : -1;
        }
      }
      if (xl >= 2 * nkg && xl < 2 * nmax) Xg[xl] = -1;
      nx = 2 * nmax;
      wave_sync();
    }
    return nx;
  }

  // The whole walk, levels L..2; returns the leaf-candidate slot count.
  __device__ int walk(const Geo& geo, int bq, WalkLdsM<GPW>* w, int lane) const {
    const int nx = init_level(geo, bq, geo.L, w, lane);
    return geo.L == 1 ? nx : walk_levels(geo, bq, geo.L, 2, nx, w, lane);
  }

  // One query group per wavefront (decode): levels l and l - 1 (l >= 3) from one gather.
  // A pyramid node is the plain mean of its children, so q.(child mean) is the mean of q
  // over the grandchildren's means: the dots of the four level-(l-2) grandchildren
  // 4y .. 4y+3 of every level-l candidate y give its score (LSE over its two children's
  // averaged dots) and the scores of both of its children (LSE over their own children's
  // dots), so the level-l Top-K and the level-(l-1) Top-K over the kept nodes' children
  // need one round of gathers instead of two.  Tile t holds in row block rb the four
  // grandchildren of candidate 4t + rb; lane (column m = head, row block kg) then holds
  // candidate 4t + kg's four dots for head m.  X holds the level-l candidates on entry
  // (nx slots) and the level-(l-2) candidates (children of the level-(l-1) nodes kept) on
  // return; the function returns their slot count.  Uses key, sc, er, key2 and U of w.
  template <bool kLds>
  __device__ int pair_step(const Geo& geo, int bq, int l, int nx, WalkLdsM<GPW>* w, int lane) const {
    static_assert(GPW == 1, "one query group per wavefront");
    constexpr int PT = 4;  // tiles (16 candidates) per batch of gathers
    const int K = geo.K;
    const int lb = l - 2;  // level of the gathered nodes (>= 1)
    const int nb = geo.n[lb];
    const int sh = lb - 1;  // a level-lb node g covers leaf blocks from g << sh
    const char* Lc = kLds ? lds + (int64_t)(geo.off[lb] - stage_base) * kRecLds : nullptr;
    const int m = lane & 15, kg = lane >> 4;
    const int rb = m >> 2, v = m & 3;  // loads: row block (candidate of the tile), grandchild
    const float c2 = trunc_c2(geo.scorer, true);
    const bool lse = geo.scorer == PISA_LSE;
    auto pair = [&](float y0, float y1) {  // y0: a visible child's dot; y1: -inf if absent
      const float a = fmaxf(y0, y1), b = fminf(y0, y1);
      return lse ? a + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(b - a)) : pair_trunc(a, b, 1.f, c2);
    };
    const int ntiles = (nx + 3) >> 2;
    for (int t0 = 0; t0 < ntiles; t0 += PT) {
      bf16x8 hi[PT][KS], lo[PT][KS];
      int ye[PT];  // epilogue: candidate 4 (t0 + tb) + kg of this lane, read with the loads
#pragma unroll
      for (int tb = 0; tb < PT; ++tb) {
        const int xe = 4 * (t0 + tb) + kg;
        ye[tb] = xe < nx ? w->X[xe] : -1;
        const int x = 4 * (t0 + tb) + rb;
        const int y = x < nx ? w->X[x] : -1;
        const int gc = y >= 0 ? 4 * y + v : -1;
        const int ca = (gc >= 0 && gc < nb) ? gc : 0;  // a missing grandchild reads node 0, never used
        if constexpr (kLds) {
          const char* rp = Lc + (int64_t)ca * kRecLds + 16 * kg;
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            hi[tb][s] = *reinterpret_cast<const bf16x8*>(rp + 128 * s);
            lo[tb][s] = *reinterpret_cast<const bf16x8*>(rp + 128 * s + 64);
          }
        } else {
          const bf16* rp = R + rc_node(geo.off[lb] + ca, D) + rc_piece(kg);  // piece 4 s + kg
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            hi[tb][s] = *reinterpret_cast<const bf16x8*>(rp + 256 * s);
            lo[tb][s] = *reinterpret_cast<const bf16x8*>(rp + 256 * s + 64);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // the whole batch in flight before the first product
      // every tile of the batch (those past the candidates gathered node 0 and are never
      // written), with no branch between them so that their MFMA chains and epilogues
      // interleave
      f32x4 acc[PT];
#pragma unroll
      for (int tb = 0; tb < PT; ++tb) {
        acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[tb][s], qb[0][s], acc[tb], 0, 0, 0);
          acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[tb][s], qb[0][s], acc[tb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int tb = 0; tb < PT; ++tb) {
        const f32x4 a = acc[tb];
        const int x = 4 * (t0 + tb) + kg;
        const int y = ye[tb];
        const int g0 = 4 * y;
        const bool e1 = g0 + 1 < nb, e2 = g0 + 2 < nb, e3 = g0 + 3 < nb;
        const bool v1 = e1 && ((int64_t)(g0 + 1) << sh) <= bq;
        const bool v2 = e2 && ((int64_t)(g0 + 2) << sh) <= bq;
        const bool v3 = e3 && ((int64_t)(g0 + 3) << sh) <= bq;
        // children 2y and 2y+1 (the latter exists iff 4y+2 does, is visible iff 4y+2 is):
        // their dots are the means of their existing children's dots
        const float d0 = e1 ? 0.5f * (a[0] + a[1]) : a[0];
        const float d1 = e3 ? 0.5f * (a[2] + a[3]) : a[2];
        const float sl = group_sum<G>(pair(d0, v2 ? d1 : -INFINITY));  // y at level l
        const float s0 = group_sum<G>(pair(a[0], v1 ? a[1] : -INFINITY));  // 2y at level l - 1
        const float s1 = group_sum<G>(pair(a[2], v3 ? a[3] : -INFINITY));  // 2y+1 (if v2)
        if (m == 0 && x < nx) {
          w->key[x] = y >= 0 ? cand_key(sl, y) : 0ull;
          w->sc[x] = s0;
          w->er[x] = s1;
        }
      }
    }
    w->key2[lane] = 0ull;
    w->U[lane] = -1;
    wave_sync();
    // Top-K of level l; the kept node of rank r opens level-(l-1) slots 2r, 2r+1 (key[x] for
    // x in [nx, nx rounded up to even) is 0 here or holds a candidate past nx: never larger)
    {
      const uint64_t my = lane < nx ? w->key[lane] : 0ull;
      int rank = 0;
#pragma unroll 4
      for (int y = 0; y < nx; y += 2) {
        const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(w->key + y);
        rank += (kk.x > my) + (y + 1 < nx && kk.y > my);
      }
      if (my != 0ull && rank < K) {
        const int y = w->X[lane];
        const bool vis1 = child_visible(2 * y + 1, geo.n[l - 1], l - 2, bq);
        w->U[2 * rank] = 2 * y;
        w->key2[2 * rank] = cand_key(w->sc[lane], 2 * y);
        w->U[2 * rank + 1] = vis1 ? 2 * y + 1 : -1;
        w->key2[2 * rank + 1] = vis1 ? cand_key(w->er[lane], 2 * y + 1) : 0ull;
      }
    }
    wave_sync();
    // Top-K of level l - 1; the kept node of rank r opens level-(l-2) slots 2r, 2r+1
    const uint64_t my = w->key2[lane];
    int rank = 0;
#pragma unroll 4
    for (int y = 0; y < 2 * K && y < kMaxCand; y += 2) {
      const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(w->key2 + y);
      rank += (kk.x > my) + (kk.y > my);
    }
    const int z = w->U[lane];
    const int nk = min(K, (int)__popcll(__ballot(my != 0ull)));
    w->X[lane] = -1;
    wave_sync();
    if (my != 0ull && rank < K) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ch = 2 * z + c;
        w->X[2 * rank + c] = child_visible(ch, geo.n[l - 2], l - 3, bq) ? ch : -1;
      }
    }
    wave_sync();
    return 2 * nk;
  }

  // pair_step spread over the workgroup (decode): wavefronts 0 .. kWalkWaves-1 score tiles
  // wave, wave + kWalkWaves, ... (one tile of four candidates at a time, each wavefront with
  // its own copy of the query fragments), so a step's products and epilogues run four at
  // a time; wavefront 0 then runs both Top-Ks.  Every wavefront of the workgroup must call
  // it (it holds three workgroup barriers); the returned count is the same in all of them.
  static constexpr int kWalkWaves = 4;
  template <bool kLds>
  __device__ int pair_step_mw(const Geo& geo, int bq, int l, int nx, WalkLdsM<GPW>* w, int lane, int wave) const {
    static_assert(GPW == 1, "one query group per workgroup");
    const int K = geo.K;
    const int lb = l - 2;  // level of the gathered nodes (>= 1)
    const int nb = geo.n[lb];
    const int sh = lb - 1;  // a level-lb node g covers leaf blocks from g << sh
    const char* Lc = kLds ? lds + (int64_t)(geo.off[lb] - stage_base) * kRecLds : nullptr;
    const int m = lane & 15, kg = lane >> 4;
    const int rb = m >> 2, v = m & 3;
    const float c2 = trunc_c2(geo.scorer, true);
    const bool lse = geo.scorer == PISA_LSE;
    auto pair = [&](float y0, float y1) {  // y0: a visible child's dot; y1: -inf if absent
      const float a = fmaxf(y0, y1), b = fminf(y0, y1);
      return lse ? a + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(b - a)) : pair_trunc(a, b, 1.f, c2);
    };
    const int ntiles = (nx + 3) >> 2;
    if (wave < kWalkWaves) {
      for (int t = wave; t < ntiles; t += kWalkWaves) {
        bf16x8 hi[KS], lo[KS];
        const int xe = 4 * t + kg;
        const int ye = xe < nx ? w->X[xe] : -1;  // epilogue: candidate 4t + kg of this lane
        const int x = 4 * t + rb;
        const int y = x < nx ? w->X[x] : -1;
        const int gc = y >= 0 ? 4 * y + v : -1;
        const int ca = (gc >= 0 && gc < nb) ? gc : 0;  // a missing grandchild reads node 0, never used
        if constexpr (kLds) {
          const char* rp = Lc + (int64_t)ca * kRecLds + 16 * kg;
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            hi[s] = *reinterpret_cast<const bf16x8*>(rp + 128 * s);
            lo[s] = *reinterpret_cast<const bf16x8*>(rp + 128 * s + 64);
          }
        } else {
          const bf16* rp = R + rc_node(geo.off[lb] + ca, D) + rc_piece(kg);  // piece 4 s + kg
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            hi[s] = *reinterpret_cast<const bf16x8*>(rp + 256 * s);
            lo[s] = *reinterpret_cast<const bf16x8*>(rp + 256 * s + 64);
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // the tile's loads in flight before its first product
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[s], qb[0][s], a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[s], qb[0][s], a, 0, 0, 0);
        }
        const int g0 = 4 * ye;
        const bool e1 = g0 + 1 < nb, e2 = g0 + 2 < nb, e3 = g0 + 3 < nb;
        const bool v1 = e1 && ((int64_t)(g0 + 1) << sh) <= bq;
        const bool v2 = e2 && ((int64_t)(g0 + 2) << sh) <= bq;
        const bool v3 = e3 && ((int64_t)(g0 + 3) << sh) <= bq;
        // children 2y and 2y+1 of candidate y (the latter exists iff 4y+2 does, is visible
        // iff 4y+2 is): their dots are the means of their existing children's dots
        const float d0 = e1 ? 0.5f * (a[0] + a[1]) : a[0];
        const float d1 = e3 ? 0.5f * (a[2] + a[3]) : a[2];
        const float sl = group_sum<G>(pair(d0, v2 ? d1 : -INFINITY));  // y at level l
        const float s0 = group_sum<G>(pair(a[0], v1 ? a[1] : -INFINITY));  // 2y at level l - 1
        const float s1 = group_sum<G>(pair(a[2], v3 ? a[3] : -INFINITY));  // 2y+1 (if v2)
        if (m == 0 && xe < nx) {
          w->key[xe] = ye >= 0 ? cand_key(sl, ye) : 0ull;
          w->sc[xe] = s0;
          w->er[xe] = s1;
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      w->key2[lane] = 0ull;
      w->U[lane] = -1;
      wave_sync();
      // Top-K of level l; the kept node of rank r opens level-(l-1) slots 2r, 2r+1
      {
        const uint64_t my = lane < nx ? w->key[lane] : 0ull;
        int rank = 0;
#pragma unroll 4
        for (int y = 0; y < nx; y += 2) {
          const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(w->key + y);
          rank += (kk.x > my) + (y + 1 < nx && kk.y > my);
        }
        if (my != 0ull && rank < K) {
          const int y = w->X[lane];
          const bool vis1 = child_visible(2 * y + 1, geo.n[l - 1], l - 2, bq);
          w->U[2 * rank] = 2 * y;
          w->key2[2 * rank] = cand_key(w->sc[lane], 2 * y);
          w->U[2 * rank + 1] = vis1 ? 2 * y + 1 : -1;
          w->key2[2 * rank + 1] = vis1 ? cand_key(w->er[lane], 2 * y + 1) : 0ull;
        }
      }
      wave_sync();
      // Top-K of level l - 1; the kept node of rank r opens level-(l-2) slots 2r, 2r+1
      const uint64_t my = w->key2[lane];
      int rank = 0;
#pragma unroll 4
      for (int y = 0; y < 2 * K && y < kMaxCand; y += 2) {
        const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(w->key2 + y);
        rank += (kk.x > my) + (kk.y > my);
      }
      const int z = w->U[lane];
      const int nk = min(K, (int)__popcll(__ballot(my != 0ull)));
      w->X[lane] = -1;
      wave_sync();
      if (my != 0ull && rank < K) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int ch = 2 * z + c;
          w->X[2 * rank + c] = child_visible(ch, geo.n[l - 2], l - 3, bq) ? ch : -1;
        }
      }
      if (lane == 0) w->nx_shared = 2 * nk;
    }
    __syncthreads();
    return w->nx_shared;
  }

  // The walk spread over the workgroup: pair_step_mw while at least two routing levels
  // remain, the top level's set-up and a last single level on wavefront 0.  Every
  // wavefront calls it; all of them return the count of level-1 candidates in X.
  __device__ int walk_pairs_mw(const Geo& geo, int bq, WalkLdsM<GPW>* w, int lane, int wave) const {
    if (wave == 0) {
      const int n0 = init_level(geo, bq, geo.L, w, lane);
      if (lane == 0) w->nx_shared = n0;
    }
    __syncthreads();
    int nx = w->nx_shared;
    int l = geo.L;
    for (; l >= 3; l -= 2)
      nx = l - 2 >= stage_lo ? pair_step_mw<true>(geo, bq, l, nx, w, lane, wave)
                             : pair_step_mw<false>(geo, bq, l, nx, w, lane, wave);
    if (l == 2) {
      __syncthreads();  // every wavefront has read nx before wavefront 0 writes it again
      if (wave == 0) {
        const int n1 = walk_levels(geo, bq, 2, 2, nx, w, lane);
        if (lane == 0) w->nx_shared = n1;
      }
      __syncthreads();
      nx = w->nx_shared;
    }
    return nx;
  }

  // The whole walk for one query group per wavefront, two levels per gather while at
  // least two routing levels remain (pair_step), then the last one alone.
  __device__ int walk_pairs(const Geo& geo, int bq, WalkLdsM<GPW>* w, int lane) const {
    int nx = init_level(geo, bq, geo.L, w, lane);
    int l = geo.L;
    for (; l >= 3; l -= 2)
      nx = l - 2 >= stage_lo ? pair_step<true>(geo, bq, l, nx, w, lane) : pair_step<false>(geo, bq, l, nx, w, lane);
    return l == 2 ? walk_levels(geo, bq, 2, 2, nx, w, lane) : nx;
  }
};

// Leaf scores of tiles j[0..NT) for one query group on the matrix cores (decode): A = 16 raw
// keys x 32 dims of a tile (bf16 inputs are exact), B = the group's G head columns in the
// MfmaWalk<D, G, 1> layout (column n = head n; k-step s, lane group kg = lane >> 4 <-> dims
// 32s + 8kg .. +8; columns >= G are zero), four row blocks of 16 keys.  Lane l then holds
// head l & 15 for keys 16rb + 4(l >> 4) + v.  out[u] = the head-summed causal LSE over the
// keys t <= i (t < N) of block j[u], in natural units, in every lane (a tile with j[u] < 0
// reads block 0 and its result is meaningless).  Every tile's loads go out before the
// first product, so the NT tiles cost one round trip.
template <int D, int NT>
__device__ __forceinline__ void load_key_tiles(const bf16* __restrict__ keys, const int (&jt)[NT], int N, int C, int lane,
                                               bf16x8 (&a)[NT][4][D / 32]) {
  constexpr int KS = D / 32;
  const int m = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int j = jt[u] >= 0 ? jt[u] : 0;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int t = min(j * C + 16 * rb + m, N - 1);  // rows past N read a real key; masked below
#pragma unroll
      for (int k = 0; k < KS; ++k) a[u][rb][k] = *reinterpret_cast<const bf16x8*>(keys + (int64_t)t * D + 32 * k + 8 * kg);
    }
  }
}

// The scores of tiles already loaded by load_key_tiles.
template <int D, int G, int NT>
__device__ __forceinline__ void score_loaded_tiles(const bf16x8 (&a)[NT][4][D / 32], const int (&jt)[NT], int i, int N,
                                                   int C, const bf16x8 (&qb)[D / 32], int lane, float s, float s_log2e,
                                                   float (&out)[NT]) {
  constexpr int KS = D / 32;
  const int kg = lane >> 4;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int j = jt[u] >= 0 ? jt[u] : 0;
    f32x4 acc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][rb][k], qb[k], acc[rb], 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = j * C + 16 * rb + 4 * kg + v;
        if (t > i || t >= N) acc[rb][v] = -INFINITY;
        mx = fmaxf(mx, acc[rb][v]);
      }
    // lane bits 4 and 5 hold the other keys of the column: combined in registers
    // (v_permlane16/32_swap), not through LDS
    mx = xor32_max(xor16_max(mx));  // key jC <= i is live, so mx is finite
    const float ms = mx * s_log2e;
    float sum = 0.f;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) sum += __builtin_amdgcn_exp2f(fmaf(acc[rb][v], s_log2e, -ms));
    sum = xor32_sum(xor16_sum(sum));
    // sum >= 1 (the max key contributes 2^0): log2 times ln 2 needs no range handling
    const float lse = group_sum<G>(s * mx + 0.6931471805599453f * __builtin_amdgcn_logf(sum));
    out[u] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(lse)));  // lanes 0 .. G-1: the group's heads
  }
}

template <int D, int G, int NT>
__device__ __forceinline__ void score_tiles_mfma(const bf16* __restrict__ keys, const int (&jt)[NT], int i, int N,
                                                 int C, const bf16x8 (&qb)[D / 32], int lane, float s, float s_log2e,
                                                 float (&out)[NT]) {
  bf16x8 a[NT][4][D / 32];
  load_key_tiles<D, NT>(keys, jt, N, C, lane, a);
  // the tiles' loads in flight before the first product (G <= 4: with more heads the
  // decode kernel would spill)
  if constexpr (G <= 4) __builtin_amdgcn_sched_barrier(0);
  score_loaded_tiles<D, G, NT>(a, jt, i, N, C, qb, lane, s, s_log2e, out);
}

template <int D, int G>
__device__ __forceinline__ float score_tile_mfma(const bf16* __restrict__ keys, int j, int i, int N, int C,
                                                 const bf16x8 (&qb)[D / 32], int lane, float s, float s_log2e) {
  const int jt[1] = {j};
  float out[1];
  score_tiles_mfma<D, G, 1>(keys, jt, i, N, C, qb, lane, s, s_log2e, out);
  return out[0];
}

// ---------------------------------------------------------------- VALU scorer
template <int D, int G>
struct ValuScorer {
  const float* P;   // fp32 means of this (b, h)'s pyramid
  const float* qs;  // LDS: G rows of D (+kQPad) floats

  __device__ void score(const Geo& geo, int bq, int l, int nx, WalkLds* w, int lane) const {
    const float* Pc = P + (int64_t)geo.off[l - 1] * D;
    const int nchild = geo.n[l - 1];
    const int cshift = l - 2;
    const int half = lane >> 5;
    for (int base = 0; base < 2 * nx; base += 32) {
      const int slot = base + (lane & 31);
      const int x = slot >> 1;
      const int node = x < nx ? w->X[x] : -1;
      const int c = node >= 0 ? 2 * node + (slot & 1) : -1;
      const bool valid = child_visible(c, nchild, cshift, bq);
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
        // (Odd slots' sums are never written.)
        sc += geo.scorer == PISA_LSE ? m + logf(expf(y - m) + expf(y2 - m))
                                     : pair_trunc(m, fminf(y, y2), 0.6931471805599453f, trunc_c2(geo.scorer, false));
      }
      if (lane < 32 && (slot & 1) == 0 && x < nx) w->cs[x] = node >= 0 ? sc : -INFINITY;
    }
    wave_sync();
  }
};

// Runs the walk; on return w->X[0..nx) holds the leaf candidates (ids or -1) and the
// function returns nx (<= 2K).
template <class Scorer>
__device__ int route_walk(const Geo& geo, const Scorer& sc, int bq, WalkLds* w, int lane) {
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
    sc.score(geo, bq, l, nx, w, lane);
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
    const int nchild = geo.n[l - 1];
    const int cshift = l - 2;
    if (myid >= 0 && rank < K) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ch = 2 * myid + c;
        w->X[2 * rank + c] = child_visible(ch, nchild, cshift, bq) ? ch : -1;
      }
    }
    nx = 2 * nkept;
    wave_sync();
  }
  return nx;
}

// Loads the G query rows of one group into LDS as fp32 (VALU scorer).
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
