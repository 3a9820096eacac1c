// Leaf scoring on the matrix cores (stage two of the two-stage prefill) and the forced
// local blocks plus final Top-K.
//
// "Block Sparse Attention with Log-Linear Complexity": rcap.io explainer, kernel
// paragraph: the second stage gathers the queries routed to a leaf block, so one load of
// its key tile serves all of them); agihunt.info summary, LSE and forced-block paragraph
// (leaf LSE over raw keys; first, previous and current blocks forced in) and kernels
// paragraph (GQA heads share the selection).
//
// The pages reuse a key tile across up to four queries.  Here the routed candidates are
// grouped by level-2 node (its two children are adjacent leaf blocks, routed together): a
// workgroup stages the node's two 64 x d bf16 key tiles in LDS and streams the entries of
// that node's list through v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims from LDS,
// B = 16 dims x 32 columns where a column is one (query, head) pair of a listed entry
// (32/G entries per column group), so every MFMA is dense.  The epilogue takes a 64-key
// LSE per column and child in registers (one cross-lane exchange), sums the G heads of an
// entry with DPP moves and writes the two scores to the entry's slots.
//
// MFMA operand layout (v_mfma_f32_32x32x16_bf16, wave64): lane l supplies row (l & 31)
// of A and column (l & 31) of B, each with the 8 consecutive k of group (l >> 5); the
// 16 results of lane l are column (l & 31), rows 8(v/4) + 4(l >> 5) + (v & 3).  The head
// dimension is walked as k-step s, group hh -> dims 16s + 8hh .. +8, the same map for A
// and B, so the two lanes of a column read 32 contiguous bytes of its query row per load.
#include "final_dev.h"

namespace pisa {

namespace {

// Workgroup = one chunk of a level-2 node's list (QC = 4 kLeafColGroups 32/G entries):
// the node's two leaf blocks (128 keys) are staged in LDS once, and each wavefront scores
// kLeafColGroups column groups of 32 (entry, head) columns against both, loading the next
// group's query fragments while it scores the current one.  A query that routed through
// the node needs both children unless one is forced (scored elsewhere) or not visible;
// both are scored, and the final Top-K reads only the slots that hold a routed block, so
// one gather of the query rows serves two leaf scores.
//
// Chunks run in list order (one KV head's nodes at a time, siblings adjacent) across all
// XCDs at once.  A query's kept level-2 nodes cluster under few ancestors, so its rows are
// read again by nearby lists while they still sit in the shared MALL: measured at 256K,
// this order beat giving each XCD a contiguous chunk range (so that a node's key tiles are
// fetched by one L2 only) by 13%, and non-temporal query loads cost 60%.
template <int D, int G>
__global__ __launch_bounds__(256) void leaf_pair_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                        Geo geo, const int32_t* __restrict__ off,
                                                        const int32_t* __restrict__ choff,
                                                        const int32_t* __restrict__ entries, int32_t M,
                                                        float* __restrict__ lscore, const bf16* __restrict__ qg) {
  constexpr int CPG = 32 / G;  // entries per column group
  constexpr int NCG = kLeafColGroups;
  constexpr int QC = 4 * NCG * CPG;
  constexpr int KS = D / 16;
  constexpr int LDSR = D + 8;
  constexpr int EPT = QC / 256;  // chunk entries per thread
  static_assert(QC % 256 == 0, "the chunk's entries split evenly over the threads");
  __shared__ __attribute__((aligned(16))) bf16 kt[2 * kLeaf * LDSR];
  __shared__ int32_t ents[QC];  // the chunk's entries (-1 past its end)

  const int c = blockIdx.x;
  if (c >= choff[M]) return;  // uniform: the grid is an upper bound on the chunk count
  const int list = find_chunk_list(choff, 0, M, c, threadIdx.x & 63);
  const int bh = list / geo.n1p, m = list % geo.n1p;
  const int e0 = off[list] + (c - choff[list]) * QC;
  const int e1 = min(e0 + QC, off[list + 1]);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int r = col % G;
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  // The lane's query rows (head h G + r of each entry's query), dims 16 s + 8 hh of k-step
  // s: from the regrouped copy when the dense launch wrote one (the group's heads adjacent
  // per 8-dim piece, so G consecutive lanes read G * 16 contiguous bytes), else from q.
  const bf16* qh = qg ? qg + (int64_t)bh * geo.N * (G * D) + (hh * G + r) * 8
                      : q + ((int64_t)b * geo.Hq + h * G + r) * geo.N * D + 8 * hh;
  const int64_t qrow = qg ? G * D : D;
  const int qstep = qg ? 16 * G : 16;
  // entry of this lane's column in column group u of the wavefront (-1: none; the column
  // then scores the rows of query 0 and its results are never stored): the first
  // from global memory, the others from the chunk's copy in LDS (loaded with the key
  // tiles, so no column group waits on a global round trip for its entry index)
  auto entry = [&](int u) {
    const int e = e0 + (u * 4 + wave) * CPG + col / G;
    return e < e1 ? entries[e] : -1;
  };
  int ent = entry(0);
  bf16x8 bq[KS];
  // query fragments first: their latency overlaps the key-tile staging
  load_bfrag_step<D>(qh + max(ent >> 6, 0) * qrow, qstep, bq);
  int ev[EPT];
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    const int t = threadIdx.x + 256 * x;
    ev[x] = e0 + t < e1 ? entries[e0 + t] : -1;
  }

  const bf16* kb = k + (int64_t)bh * geo.N * D;
  const bool two = 2 * m + 1 < geo.n1;  // the node's second child exists
  KeyTile<D> ta, tb;  // both tiles' loads in flight before either is stored
  ta.load(kb, 2 * m * kLeaf, geo.N);
  if (two) tb.load(kb, (2 * m + 1) * kLeaf, geo.N);
  ta.store(kt);
  if (two) tb.store(kt + kLeaf * LDSR);
#pragma unroll
  for (int x = 0; x < EPT; ++x) ents[threadIdx.x + 256 * x] = ev[x];
  __syncthreads();
  // keys present in each child (>= 1); only a short last block masks
  const int live0 = min(kLeaf, geo.N - 2 * m * kLeaf);
  const int live1 = two ? min(kLeaf, geo.N - (2 * m + 1) * kLeaf) : 0;
  const int twoK = 2 * geo.K;

  // column group u scores with cur while the next group's query fragments load into nxt;
  // two groups per iteration swap the roles, so no fragment is copied between registers
  auto step = [&](int u, const bf16x8 (&cur)[KS], bf16x8 (&nxt)[KS]) {
    if (e0 + (u * 4 + wave) * CPG >= e1) return false;  // uniform across the wavefront
    const int ent_n = u + 1 < NCG ? ents[((u + 1) * 4 + wave) * CPG + col / G] : -1;
    load_bfrag_step<D>(qh + max(ent_n >> 6, 0) * qrow, qstep, nxt);

    f32x16 acc0, acc1;
    tile_mfma32<D>(kt, cur, lane, acc0, acc1);
    if (live0 < kLeaf) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if (key_row(v, hh) >= live0) acc0[v] = -INFINITY;
        if (32 + key_row(v, hh) >= live0) acc1[v] = -INFINITY;
      }
    }
    const float lse0 = group_sum<G>(column_lse32(acc0, acc1, geo.s, geo.s_log2e));
    float lse1 = 0.f;
    if (two) {
      tile_mfma32<D>(kt + kLeaf * LDSR, cur, lane, acc0, acc1);
      if (live1 < kLeaf) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if (key_row(v, hh) >= live1) acc0[v] = -INFINITY;
          if (32 + key_row(v, hh) >= live1) acc1[v] = -INFINITY;
        }
      }
      lse1 = group_sum<G>(column_lse32(acc0, acc1, geo.s, geo.s_log2e));
    }
    if (hh == 0 && r == 0 && ent >= 0) {
      float* dst = lscore + ((int64_t)bh * geo.N + (ent >> 6)) * twoK + 2 * (ent & 63);
      dst[0] = lse0;
      if (two) dst[1] = lse1;
    }
    ent = ent_n;
    return true;
  };
  static_assert(NCG % 2 == 0, "column groups come in pairs");
  bf16x8 bqn[KS];
  for (int u = 0; u < NCG; u += 2) {
    if (!step(u, bq, bqn)) break;
    if (!step(u + 1, bqn, bq)) break;
  }
}

// Workgroup = one leaf block of queries (64) of one (b, h): stages the forced blocks'
// key tiles (0, bq - 1, bq) in LDS, scores them for the block's 64 x G (query, head)
// columns (32 per MFMA tile; the query fragments of the next column group are loaded
// while the current one is scored), then each wavefront finalizes 16 of the queries.
template <int D, int G, int SL>
__global__ __launch_bounds__(256) void forced_final_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                           Geo geo, const int32_t* __restrict__ cand,
                                                           const float* __restrict__ lscore,
                                                           int32_t* __restrict__ out_idx,
                                                           float* __restrict__ out_score) {
  constexpr int KS = D / 16;
  constexpr int LDSR = D + 8;
  constexpr int NQ = 64 / SL;          // query groups finalized per pass
  constexpr int PASSES = 16 / NQ;      // passes for a wavefront's 16 queries
  __shared__ __attribute__((aligned(16))) bf16 kt[3][kLeaf * LDSR];
  __shared__ float fs[kLeaf][4];
  __shared__ __attribute__((aligned(16))) uint64_t kx_all[4][64];
  __shared__ __attribute__((aligned(16))) int32_t lx_all[4][64];

  const int bq = blockIdx.x, bh = blockIdx.y;
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  int F[3];
  const int nf = forced_blocks(bq, F);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int twoK = 2 * geo.K;
  const int slot = lane % SL, qq = lane / SL;

  // Routed candidates and their leaf scores for this wavefront's queries
  // ql = wave + 4 (p NQ + qq), loaded up front.
  int cl[PASSES];
  float cv[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    // the slot's candidate and score loaded together (the score is only used where the
    // slot holds a candidate; elsewhere it reads an in-bounds stale value)
    const int i = bq * kLeaf + wave + 4 * (p * NQ + qq);
    const bool in = i < geo.N && slot < twoK;
    const int64_t e = in ? ((int64_t)bh * geo.N + i) * twoK + slot : 0;
    const int c = cand[e];
    const float v = lscore[e];
    cl[p] = in ? c : -1;
    cv[p] = cl[p] >= 0 ? v : -INFINITY;
  }

  // 64 queries x G heads = 2G groups of 32 columns; this wavefront takes cg = wave + 4m
  auto qrow = [&](int cg) {
    const int gc = cg * 32 + col;
    return q + (((int64_t)b * geo.Hq + h * G + gc % G) * geo.N + bq * kLeaf + gc / G) * D;
  };
  auto qvalid = [&](int cg) { return cg < 2 * G && bq * kLeaf + (cg * 32 + col) / G < geo.N; };
  bf16x8 bfr[KS];
  load_bfrag<D>(qrow(wave), qvalid(wave), hh, bfr);

  const bf16* kb = k + (int64_t)bh * geo.N * D;
  {  // the forced tiles' loads all in flight before the first is stored
    KeyTile<D> tl[3];
#pragma unroll
    for (int f = 0; f < 3; ++f)
      if (f < nf) tl[f].load(kb, F[f] * kLeaf, geo.N);
#pragma unroll
    for (int f = 0; f < 3; ++f)
      if (f < nf) tl[f].store(kt[f]);
  }
  __syncthreads();

  for (int cg = wave; cg < 2 * G; cg += 4) {
    bf16x8 bfn[KS];
    load_bfrag<D>(qrow(cg + 4), qvalid(cg + 4), hh, bfn);
    const int gc = cg * 32 + col;
    const int ql = gc / G, r = gc % G;
    const int i = bq * kLeaf + ql;
    const bool valid = i < geo.N;
    for (int f = 0; f < nf; ++f) {
      f32x16 acc0, acc1;
      tile_mfma32<D>(kt[f], bfr, lane, acc0, acc1);
      const int t0 = F[f] * kLeaf;
      // only the current block (and a short tail block) needs a mask
      if (F[f] == bq || t0 + kLeaf > geo.N) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ta = t0 + key_row(v, hh), tb = ta + 32;
          if (ta > i || ta >= geo.N) acc0[v] = -INFINITY;
          if (tb > i || tb >= geo.N) acc1[v] = -INFINITY;
        }
      }
      // columns past N (last query block only) still see live keys, so no NaN arises
      float lse = column_lse32(acc0, acc1, geo.s, geo.s_log2e);
      lse = group_sum<G>(lse);
      if (hh == 0 && r == 0 && valid) fs[ql][f] = lse;
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) bfr[s] = bfn[s];
  }
  __syncthreads();

#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int ql = wave + 4 * (p * NQ + qq);
    const int i = bq * kLeaf + ql;
    const bool live = i < geo.N;
    const int64_t row = (int64_t)bh * geo.N + (live ? i : 0);
    finalize_rows<SL>(cl[p], cv[p], F, nf, fs[ql], geo.K, lane, live, kx_all[wave], lx_all[wave],
                      out_idx + row * geo.K, out_score + row * geo.K);
  }
}

// Final selection for problems whose forced blocks the dense routing launch scored (fsc:
// the forced blocks' scores of each query group, ascending): workgroup = 4 QW queries of
// one leaf block of one (b, h) (64 / (4 QW) workgroups per leaf block); each wavefront
// finalizes QW of them, 64/SL per pass.  With 2K > 16 slots a query fills SL = 32 or 64
// lanes, so QW = 4 (SL = 32) or 2 (SL = 64) keeps the passes per wavefront (each an LDS
// round trip) few and the launch wide (16K, K = 32: 74 us at QW = 16, 62 at 4, 59 at 2,
// 60 at 1).
template <int SL, int QW>
__global__ __launch_bounds__(256) void final_kernel(Geo geo, const int32_t* __restrict__ cand,
                                                    const float* __restrict__ lscore, const float* __restrict__ fsc,
                                                    int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  constexpr int NQ = 64 / SL;      // query groups finalized per pass
  constexpr int PASSES = QW / NQ;  // passes for a wavefront's QW queries
  constexpr int SUB = 16 / QW;     // workgroups per leaf block
  static_assert(QW % NQ == 0 && 16 % QW == 0, "whole passes, whole leaf blocks");
  __shared__ __attribute__((aligned(16))) uint64_t kx_all[4][64];
  __shared__ __attribute__((aligned(16))) int32_t lx_all[4][64];
  const int bq = blockIdx.x / SUB, q0 = bq * kLeaf + (blockIdx.x % SUB) * 4 * QW, bh = blockIdx.y;
  int F[3];
  const int nf = forced_blocks(bq, F);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int twoK = 2 * geo.K;
  const int slot = lane % SL, qq = lane / SL;
  int cl[PASSES];
  float cv[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    // the slot's candidate and score loaded together (the score is only used where the
    // slot holds a candidate; elsewhere it reads an in-bounds stale value)
    const int i = q0 + wave + 4 * (p * NQ + qq);
    const bool in = i < geo.N && slot < twoK;
    const int64_t e = in ? ((int64_t)bh * geo.N + i) * twoK + slot : 0;
    const int c = cand[e];
    const float v = lscore[e];
    cl[p] = in ? c : -1;
    cv[p] = cl[p] >= 0 ? v : -INFINITY;
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int i = q0 + wave + 4 * (p * NQ + qq);
    const bool live = i < geo.N;
    const int64_t row = (int64_t)bh * geo.N + (live ? i : 0);
    finalize_rows<SL>(cl[p], cv[p], F, nf, fsc + row * 3, geo.K, lane, live, kx_all[wave], lx_all[wave],
                      out_idx + row * geo.K, out_score + row * geo.K);
  }
}

template <int D>
int leaf_d(const Geo& g, const void* q, const void* k, const void* qg, const int32_t* off, const int32_t* choff,
           const int32_t* entries, int32_t M, float* lscore, hipStream_t st) {
  const int qc = chunk_entries(g.G);
  const int64_t pairs = (int64_t)g.B * g.Hkv * g.N * g.K;
  const int64_t grid = (pairs + qc - 1) / qc + M;  // bound on the sum over lists of ceil(count / qc)
  const bf16* qq = (const bf16*)q;
  const bf16* kk = (const bf16*)k;
  switch (g.G) {
    case 1: leaf_pair_kernel<D, 1><<<(unsigned)grid, 256, 0, st>>>(qq, kk, g, off, choff, entries, M, lscore, (const bf16*)qg); break;
    case 2: leaf_pair_kernel<D, 2><<<(unsigned)grid, 256, 0, st>>>(qq, kk, g, off, choff, entries, M, lscore, (const bf16*)qg); break;
    case 4: leaf_pair_kernel<D, 4><<<(unsigned)grid, 256, 0, st>>>(qq, kk, g, off, choff, entries, M, lscore, (const bf16*)qg); break;
    case 8: leaf_pair_kernel<D, 8><<<(unsigned)grid, 256, 0, st>>>(qq, kk, g, off, choff, entries, M, lscore, (const bf16*)qg); break;
    case 16: leaf_pair_kernel<D, 16><<<(unsigned)grid, 256, 0, st>>>(qq, kk, g, off, choff, entries, M, lscore, (const bf16*)qg); break;
    default: return PISA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

template <int D, int SL>
int forced_sl(const Geo& g, const bf16* q, const bf16* k, const int32_t* cand, const float* lscore, int32_t* oi,
              float* os, hipStream_t st) {
  dim3 grid(g.n1, g.B * g.Hkv);
  switch (g.G) {
    case 1: forced_final_kernel<D, 1, SL><<<grid, 256, 0, st>>>(q, k, g, cand, lscore, oi, os); break;
    case 2: forced_final_kernel<D, 2, SL><<<grid, 256, 0, st>>>(q, k, g, cand, lscore, oi, os); break;
    case 4: forced_final_kernel<D, 4, SL><<<grid, 256, 0, st>>>(q, k, g, cand, lscore, oi, os); break;
    case 8: forced_final_kernel<D, 8, SL><<<grid, 256, 0, st>>>(q, k, g, cand, lscore, oi, os); break;
    case 16: forced_final_kernel<D, 16, SL><<<grid, 256, 0, st>>>(q, k, g, cand, lscore, oi, os); break;
    default: return PISA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

template <int D>
int forced_d(const Geo& g, const void* q, const void* k, const int32_t* cand, const float* lscore, int32_t* oi,
             float* os, hipStream_t st) {
  const bf16* qq = (const bf16*)q;
  const bf16* kk = (const bf16*)k;
  // slots per query group: 2K rounded up to a power of two (at least 16)
  if (2 * g.K <= 16) return forced_sl<D, 16>(g, qq, kk, cand, lscore, oi, os, st);
  if (2 * g.K <= 32) return forced_sl<D, 32>(g, qq, kk, cand, lscore, oi, os, st);
  return forced_sl<D, 64>(g, qq, kk, cand, lscore, oi, os, st);
}

}  // namespace

int launch_leaf_mfma(const Geo& g, const void* q, const void* k, const void* qg, const int32_t* off,
                     const int32_t* choff, const int32_t* entries, int32_t M, float* lscore, hipStream_t st) {
  if (g.d == 128) return leaf_d<128>(g, q, k, qg, off, choff, entries, M, lscore, st);
  if (g.d == 64) return leaf_d<64>(g, q, k, qg, off, choff, entries, M, lscore, st);
  return PISA_ERR_UNSUPPORTED;
}

int launch_final(const Geo& g, const int32_t* cand, const float* lscore, const float* fsc, int32_t* out_idx,
                 float* out_score, hipStream_t st) {
  const unsigned bh = (unsigned)(g.B * g.Hkv);
  if (2 * g.K <= 16)
    final_kernel<16, 16><<<dim3(g.n1, bh), 256, 0, st>>>(g, cand, lscore, fsc, out_idx, out_score);
  else if (2 * g.K <= 32)
    final_kernel<32, 4><<<dim3(4 * g.n1, bh), 256, 0, st>>>(g, cand, lscore, fsc, out_idx, out_score);
  else
    final_kernel<64, 2><<<dim3(8 * g.n1, bh), 256, 0, st>>>(g, cand, lscore, fsc, out_idx, out_score);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

int launch_forced_final(const Geo& g, const void* q, const void* k, const int32_t* cand, const float* lscore,
                        int32_t* out_idx, float* out_score, hipStream_t st) {
  if (g.d == 128) return forced_d<128>(g, q, k, cand, lscore, out_idx, out_score, st);
  if (g.d == 64) return forced_d<64>(g, q, k, cand, lscore, out_idx, out_score, st);
  return PISA_ERR_UNSUPPORTED;
}

}  // namespace pisa
