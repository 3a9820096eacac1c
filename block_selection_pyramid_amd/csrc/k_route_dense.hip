// Prefill routing, upper pyramid levels (L down to l_bot >= 3, while the levels are small),
// scored densely.
//
// What is computed is the top-down walk of "Block Sparse Attention with Log-Linear
// Complexity" (rcap.io explainer, top-down walk and scoring paragraphs; agihunt.info
// summary, kernels paragraph for the GQA head sum): at each level a candidate's score is
// the sum over the G heads of the LogSumExp of s*q.child over its visible children, the
// Top-K candidates (score descending, lower index first) are kept, and their children are
// the next level's candidates.
//
// How it is computed differs from a per-query gather.  The queries of one leaf block see
// the same prefix of every level, and at the upper levels that prefix is small, so a
// workgroup scores every visible child of a level against all of its queries: a dense
// contraction on the matrix cores (v_mfma_f32_32x32x16_bf16, A = 32 child summaries from
// the hi/lo routing copy staged in LDS once per workgroup, B = 32 (query, head) columns
// held in registers; the routing copy is pre-scaled by s log2(e), so the products are the
// scores in log2 units).  The epilogue forms the pair LSE of each node's two children (or,
// for the PISA-1 / PISA-2 ablations, its truncation about their mean) and the head sum,
// and each wavefront keeps only the scores of its own queries' candidates.  Because a
// node's dot is the mean of its children's dots, one sweep over the tiles of level l - 2
// scores both level l - 1 (pairs of tile nodes) and level l (pairs of those pair means):
// the levels are scored two per sweep, so the tiles of every other level are never read.
// The staged tiles do not depend on the walk, so the next tile is fetched straight into
// the other LDS buffer (no registers in flight) while the current one is scored, across
// level boundaries too.
//
// Output: per query group, the 2K candidate slots of level l_bot - 1 (children of the Top-K
// nodes of level l_bot, -1 where a child does not exist or is not visible), the input of
// the gather routing launch; for l_bot = 2 the leaf candidates themselves, forced blocks
// also -1.  The same workgroup then scores its queries' forced leaf blocks
// ("Block Sparse Attention with Log-Linear Complexity", agihunt.info summary, LSE and
// forced-block paragraph: first, previous and current block; leaf score = causal LSE over
// the block's raw keys, summed over the G heads) with the query rows it already holds:
// each forced key tile is staged in LDS once and contracted on the matrix cores.
#include <type_traits>

#include "final_dev.h"
#include "route_dev.h"
#include "tile_dev.h"

namespace pisa {

namespace {

template <int D, int G, int KC>
constexpr size_t dense_lds_bytes() {
  return 2 * (size_t)(2 * (D / 16) * 1024) + (size_t)kDenseWaves * DenseShape<G>::QPW * (96 + 20 * KC);
}

// Forced key tile f (64 raw keys) into fragment-major LDS: fragment fi = rb KS + ks holds
// keys 64 f + 32 rb + (lane & 31), dims 16 ks + 8 (lane >> 5) .. +8; keys past N read
// zeros (the row index is clamped and the value replaced, so no load sits behind a branch).
template <int D, int NU>
__device__ __forceinline__ void dense_load_keys(const bf16* kb, int N, int f, int wave, int lane, u32x4 (&stg)[NU]) {
  constexpr int KS = D / 16;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int fi = wave + kDenseWaves * u, rb = fi / KS, ks = fi % KS;
    const int key = 64 * f + 32 * rb + (lane & 31);
    const u32x4 v = *reinterpret_cast<const u32x4*>(kb + (int64_t)min(key, N - 1) * D + 16 * ks + 8 * (lane >> 5));
    stg[u] = key < N ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

// KC >= K: capacity of kept nodes per query (the 2*KC candidate slots hold 2K in use).
// K <= 8 asks for three wavefronts per SIMD: the few registers this costs spill only in
// the phases after the routing loop.  TRUNC selects the PISA-1 / PISA-2 node scores (a
// separate instantiation keeps the LSE kernel's register allocation as it is).
template <int D, int G, int KC, bool TRUNC>
__global__ __launch_bounds__(256, KC <= 8 ? 3 : 2) void route_dense_kernel(const bf16* __restrict__ q, const float* __restrict__ pyr,
                                                          const bf16* __restrict__ k, Geo geo, int32_t l_bot,
                                                          int32_t* __restrict__ x2, float* __restrict__ fsc,
                                                          bf16* __restrict__ qg) {
  constexpr int NCG = DenseShape<G>::NCG, QPW = DenseShape<G>::QPW;
  constexpr int KS = D / 16;         // k-steps of 16 dims
  constexpr int F = 2 * KS;          // 1 KB fragments of a staged child tile (hi, lo per k-step)
  constexpr int TILE = F * 1024;     // bytes of one staged tile of 32 children
  constexpr int ITEMS = QPW * KC;    // (query, kept-node rank) items of a wavefront
  constexpr int M = (ITEMS + 63) / 64;
  constexpr int SLOTS = 2 * KC;
  static_assert(F % kDenseWaves == 0, "fragments split evenly over the wavefronts");
  static_assert((KC & (KC - 1)) == 0, "items index queries by it / KC");

  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  char* wl = lds + 2 * TILE + wave * (QPW * (96 + 20 * KC));
  float* Sx = reinterpret_cast<float*>(wl);                             // [QPW][24] node scores
  uint64_t* key = reinterpret_cast<uint64_t*>(wl + QPW * 96);           // [QPW][SLOTS]
  int32_t* np = reinterpret_cast<int32_t*>(wl + QPW * (96 + 16 * KC));  // [QPW][KC]

  const int N = geo.N, K = geo.K, L = geo.L;
  constexpr int C = kLeaf;  // leaf block size (the only one the kernels support)
  constexpr bool trunc = TRUNC;
  const float c2 = trunc_c2(geo.scorer, true);
  const int BH = geo.B * geo.Hkv;
  const int bh = blockIdx.x % BH;  // workgroups of one XCD (w mod 8) share few heads
  // longest visible prefixes (highest leaf blocks) first, so the heaviest workgroups do not
  // form the launch's tail (64K: 0.74 -> ~0.69 ms)
  const int nwg = (geo.N + kDenseWaves * QPW - 1) / (kDenseWaves * QPW);
  const int iwg = (nwg - 1 - (int)(blockIdx.x / BH)) * (kDenseWaves * QPW);
  const int iw = iwg + wave * QPW;
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  const int bqmax = (min(N, iwg + kDenseWaves * QPW) - 1) / C;
  const char* Rb = reinterpret_cast<const char*>(pyr + geo.means_floats()) + (int64_t)bh * geo.Tp * (4 * D);

  // B operand: lane column j <-> (query j / G, head j % G) of column group cg, dims
  // 16 ks + 8 hh .. +8 of k-step ks.
  const int j = lane & 31, hh = lane >> 5;
  bf16x8 qf[NCG][KS];
  int bqc[NCG];
  const int bqw = min(iw, N - 1) / C;  // bq of this wavefront's first (smallest) query
  load_query_cols<D, G, NCG>(q, geo, b, h, iw, lane, qf, bqc);
  // The regrouped query copy for the gather and leaf launches: query i's G heads of every
  // 8-dim piece adjacent, [b, h, i][piece][head][8 dims]; lane (j, hh) holds pieces
  // 2 ks + hh of column j, so each G consecutive lanes write G * 16 contiguous bytes.
  if (qg) {
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const int i = iw + cg * (32 / G) + j / G;
      if (i < N) {
        bf16* dst = qg + ((int64_t)bh * N + i) * (G * D) + (hh * G + j % G) * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) *reinterpret_cast<bf16x8*>(dst + ks * 16 * G) = qf[cg][ks];
      }
    }
  }

  // Walk state.  Item (query iq, rank r) = lane + 64 m holds the node ip kept at rank r one
  // level up; its candidates are ip's two children, with scores sc.  At the top level the
  // candidates are the visible prefix of level L, i.e. "children" of a virtual node r.
  int ip[M], ibq[M];
  float sc[M][2];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int it = lane + 64 * m;
    const int iq = it / KC, ir = it % KC;
    ibq[m] = min(iw + iq, N - 1) / C;
    const int nvis = min(geo.n[L], (ibq[m] >> (L - 1)) + 1);
    ip[m] = (it < ITEMS && 2 * ir < nvis) ? ir : -1;
    sc[m][0] = sc[m][1] = 0.f;
  }

  // Passes.  A pair pass scores levels l and l - 1 from one sweep over the tiles of level
  // l - 2: a node's dot is the mean of its children's dots, so the sweep's products give the
  // level-(l-1) dots (pair means, over the children that exist) and with them both levels'
  // scores, and the level-(l - 1) candidates (children of the level-l nodes kept) are
  // children of level-l candidates, whose scores the items pick up in the same sweep.  A
  // single pass scores level l from the tiles of level l - 1.  Pair passes cost the tiles of
  // every other level only; when the dense levels are odd in number the single pass is the
  // top one, whose tiles are the fewest, and the pairs end at l_bot.
  auto is_pair = [&](int lv) { return ((lv - l_bot) & 1) && lv >= 3; };
  auto tile_level = [&](int lv) { return is_pair(lv) ? lv - 2 : lv - 1; };
  auto ntiles = [&](int lt) {  // tiles of the visible prefix of level lt
    const int nv = min(geo.n[lt], (bqmax >> (lt - 1)) + 1);
    return (nv + 31) >> 5;
  };
  // pair pass: an item keeps the scores of the level-(l-1) nodes 4 ip .. 4 ip + 3 in its two
  // key slots (16 bytes, free until the pass's Top-K), not in registers

  int l = L, t = 0, buf = 0;
  int nt = ntiles(tile_level(L));
  dense_fetch_tile<D>(Rb, geo, tile_level(L) + 1, 0, wave, lane, lds, 0);
  dense_fetch_wait();
  __syncthreads();
  for (;;) {
    const bool pr = is_pair(l);
    const int lt = pr ? l - 2 : l - 1;  // level of this pass's tiles
    int ln = l, tn = t + 1;
    if (tn == nt) {
      ln = l - (pr ? 2 : 1);
      tn = 0;
    }
    const bool more = ln >= l_bot;
    const int ltn = more ? tile_level(ln) : lt;

    // ---- products of the 32 level-lt nodes of tile t with this wavefront's queries
    // the level size the epilogue needs, loaded (and waited for) before the products: a
    // scalar load in flight among the fragment reads makes every LDS wait a full drain
    int ntn = geo.n[lt];
    asm volatile("" : "+s"(ntn));
    const char* Tt = lds + buf * TILE;
    f32x16 acc[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[cg][v] = 0.f;
    // A fragments one k-step ahead: the reads of step ks + 1 are in flight while step ks's
    // products issue, so no k-step waits out a full LDS round trip
    bf16x8 fa[2][2];
    auto read_a = [&](int ks, bf16x8 (&f)[2]) {
      f[0] = *reinterpret_cast<const bf16x8*>(Tt + ((2 * ks) * 64 + lane) * 16);
      f[1] = *reinterpret_cast<const bf16x8*>(Tt + ((2 * ks + 1) * 64 + lane) * 16);
    };
    read_a(0, fa[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) read_a(ks + 1, fa[(ks + 1) & 1]);
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        acc[cg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][0], qf[cg][ks], acc[cg], 0, 0, 0);
        acc[cg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks & 1][1], qf[cg][ks], acc[cg], 0, 0, 0);
      }
    }
    // keep that order through scheduling: step 0's two reads, then per step the next step's
    // two reads ahead of this step's products (the register-pressure scheduler would
    // otherwise wait for each step's reads right before its products)
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NCG, 0);
    }
    // the next tile goes straight into the other buffer, which every wavefront finished
    // reading before the previous step's barrier; issued after the fragment reads, since
    // with a transfer into LDS in flight the reads' waits can no longer be counted
    if (more) dense_fetch_tile<D>(Rb, geo, ltn + 1, tn, wave, lane, lds, buf ^ 1);
    // Epilogue.  Result row (tile node) 8a + 4hh + v sits in acc[4a + v]: the lane holds
    // the four nodes 8a + 4hh .. +3, i.e. the children of the two level-(lt+1) nodes
    // 4a + 2hh + p of the tile (p = 0, 1), which are the children of level-(lt+2) node
    // 2a + hh.  Pair LSE per head: max(y0, y1) and f = 1 + 2^-|y0 - y1| in [1, 2]; the head
    // reduction is sum(max) and prod(f), and the node score (log2 units) = sum(max) +
    // log2 prod(f).  The reductions are scattered over the G lanes of a query, each lane
    // finishing a share of the values.  A node whose first child is visible has a finite
    // max; other nodes are never read, so only second children are masked (-inf: max = y0,
    // f = 1), and only in the tile that holds the end of the visible prefix: the others take
    // a path without masks.  (fmed3 against +inf is the max without canonicalising the raw
    // MFMA results first.)
    const int base = 32 * t;
    const int vsh = lt - 1;  // a level-lt node c is visible to leaf block bq iff c <= bq >> vsh
    const int lim = min(ntn - 1, bqw >> vsh) - base;  // visible rows of the wavefront's leaf block: <= lim
    const int elim = ntn - 1 - base;                  // existing rows: <= elim
    const int r = j % G;
    // +inf in a register the compiler cannot see through: fmed3 against a literal +inf is
    // rewritten into a max that canonicalises both raw MFMA results first (three operations)
    float pinf = INFINITY;
    asm volatile("" : "+s"(pinf));
    auto epilogue = [&](auto maskedc) {
      constexpr bool MASKED = decltype(maskedc)::value;
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        const int qi = cg * (32 / G) + j / G;
        if (pr) {  // the 8 level-(lt+2) nodes: slots 16..23 (first: this reads acc, the values
                   // below consume it)
          // a level-(lt+1) node's dot is the mean of its existing children's dots; these are
          // twice the means, the factor 1/2 is taken after the head sum.  The node's second
          // child (level lt+1) is visible iff that child's first child is.
          float mxs[4], prd[4];
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int r0 = 8 * a + 4 * hh;
            const float y0 = acc[cg][4 * a], y1 = acc[cg][4 * a + 1];
            const float y2 = acc[cg][4 * a + 2], y3 = acc[cg][4 * a + 3];
            float d0 = y0 + y1, d1 = y2 + y3;
            if constexpr (MASKED) {
              d0 = r0 + 1 <= elim ? d0 : 2.f * y0;
              d1 = r0 + 3 <= elim ? d1 : 2.f * y2;
              d1 = r0 + 2 <= lim ? d1 : -INFINITY;
            }
            if constexpr (!trunc) {
              mxs[a] = __builtin_amdgcn_fmed3f(d0, d1, pinf);
              prd[a] = 1.f + __builtin_amdgcn_exp2f(-fabsf(0.5f * (d0 - d1)));
            } else {
              mxs[a] = 2.f * pair_trunc(0.5f * d0, 0.5f * d1, 1.f, c2);
              prd[a] = 1.f;
            }
          }
          group_reduce_scatter<G, 4, false>(mxs, r);
          if constexpr (!trunc) group_reduce_scatter<G, 4, true>(prd, r);
          constexpr int GE = G < 4 ? G : 4, VPL = 4 / GE;
#pragma unroll
          for (int u = 0; u < VPL; ++u) {  // value e: node 2e + hh
            const int e = (r % GE) * VPL + u;
            const float out = trunc ? 0.5f * mxs[u] : fmaf(0.5f, mxs[u], __builtin_amdgcn_logf(prd[u]));
            if (r < GE) Sx[qi * 24 + 16 + 2 * e + hh] = out;
          }
        }
        {  // the 16 level-(lt+1) nodes of the tile: slots 0..15
          float mxs[8], prd[8];
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const float y0 = acc[cg][4 * a + 2 * p];
              float y1 = acc[cg][4 * a + 2 * p + 1];
              if constexpr (MASKED) y1 = 8 * a + 4 * hh + 2 * p + 1 <= lim ? y1 : -INFINITY;
              if constexpr (!trunc) {
                mxs[2 * a + p] = __builtin_amdgcn_fmed3f(y0, y1, pinf);
                prd[2 * a + p] = 1.f + __builtin_amdgcn_exp2f(-fabsf(y0 - y1));
              } else {
                mxs[2 * a + p] = pair_trunc(y0, y1, 1.f, c2);
                prd[2 * a + p] = 1.f;
              }
            }
          group_reduce_scatter<G, 8, false>(mxs, r);
          if constexpr (!trunc) group_reduce_scatter<G, 8, true>(prd, r);
          constexpr int GE = G < 8 ? G : 8, VPL = 8 / GE;
#pragma unroll
          for (int u = 0; u < VPL; ++u) {  // value e = 2a + p: node 4a + 2hh + p
            const int e = (r % GE) * VPL + u;
            const float out = trunc ? mxs[u] : mxs[u] + __builtin_amdgcn_logf(prd[u]);
            if (r < GE) Sx[qi * 24 + 4 * (e >> 1) + 2 * hh + (e & 1)] = out;
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // one column group's epilogue at a time
      }
    };
    if (lim >= 31)
      epilogue(std::false_type{});
    else
      epilogue(std::true_type{});
    wave_sync();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int iq = (lane + 64 * m) / KC;
      if (pr) {
        // candidates 2 ip, 2 ip + 1 (level l) and their children 4 ip .. 4 ip + 3 (level l - 1)
        if (ip[m] >= 4 * t && ip[m] < 4 * t + 4) {
          const int o = ip[m] - 4 * t;
          const float2 v = *reinterpret_cast<const float2*>(Sx + iq * 24 + 16 + 2 * o);
          const float4 w4 = *reinterpret_cast<const float4*>(Sx + iq * 24 + 4 * o);
          sc[m][0] = v.x;
          sc[m][1] = v.y;
          *reinterpret_cast<float4*>(key + 2 * (lane + 64 * m)) = w4;
        }
      } else if (ip[m] >= 8 * t && ip[m] < 8 * t + 8) {
        const float2 v = *reinterpret_cast<const float2*>(Sx + iq * 24 + 2 * (ip[m] - 8 * t));
        sc[m][0] = v.x;
        sc[m][1] = v.y;
      }
    }
    wave_sync();

    if (t == nt - 1) {
      // ---- Top-K of level l per query; the kept node of rank r becomes item r's parent
      // (single pass) or opens the level-(l-1) slots 2r, 2r+1 (pair pass)
      const int nl = geo.n[l];
      int kr[M][2];  // rank of the item's two candidates (>= K: not kept)
      float c1[M][4];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int it = lane + 64 * m;
        const float4 w4 = pr && it < ITEMS ? *reinterpret_cast<const float4*>(key + 2 * it) : float4{0.f, 0.f, 0.f, 0.f};
        c1[m][0] = w4.x;
        c1[m][1] = w4.y;
        c1[m][2] = w4.z;
        c1[m][3] = w4.w;
      }
      wave_sync();
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int it = lane + 64 * m;
        kr[m][0] = kr[m][1] = K;
        if (it < ITEMS) {
          // item it = (query it / KC, rank it % KC): key slots 2 it, 2 it + 1 (SLOTS = 2 KC)
          const int n0 = 2 * ip[m], n1 = n0 + 1;
          const bool v0 = ip[m] >= 0;
          const bool v1 = v0 && n1 < nl && ((int64_t)n1 << (l - 1)) <= ibq[m];
          key[2 * it] = v0 ? cand_key(sc[m][0], n0) : 0ull;
          key[2 * it + 1] = v1 ? cand_key(sc[m][1], n1) : 0ull;
          np[it] = -1;
        }
      }
      wave_sync();
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int it = lane + 64 * m;
        if (it < ITEMS) {
          const uint64_t* kq = key + (it & ~(KC - 1)) * 2;  // the query's SLOTS keys
          const uint64_t k0 = key[2 * it], k1 = key[2 * it + 1];
          int r0 = 0, r1 = 0;
#pragma unroll 4
          for (int s = 0; s < SLOTS; s += 2) {
            const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(kq + s);
            r0 += (kk.x > k0) + (kk.y > k0);
            r1 += (kk.x > k1) + (kk.y > k1);
          }
          if (k0 != 0ull && r0 < K) kr[m][0] = r0;
          if (k1 != 0ull && r1 < K) kr[m][1] = r1;
          if (!pr) {
            if (kr[m][0] < K) np[(it & ~(KC - 1)) + r0] = 2 * ip[m];
            if (kr[m][1] < K) np[(it & ~(KC - 1)) + r1] = 2 * ip[m] + 1;
          }
        }
      }
      wave_sync();
      if (pr) {
        // ---- Top-K of level l - 1 over the kept nodes' children: kept node x of rank r
        // fills slots 2r, 2r+1 with its children 2x, 2x+1 (keys of the level-(l-1) scores
        // picked up during the sweep)
        const int nc = geo.n[l - 1];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const int it = lane + 64 * m;
          if (it < ITEMS) {
            key[2 * it] = 0ull;
            key[2 * it + 1] = 0ull;
          }
        }
        wave_sync();
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const int it = lane + 64 * m;
          if (it < ITEMS) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              if (kr[m][c] < K) {
                const int x = 2 * ip[m] + c;
                const int ch1 = 2 * x + 1;
                const bool vis1 = ch1 < nc && ((int64_t)ch1 << (l - 2)) <= ibq[m];
                uint64_t* dst = key + (it & ~(KC - 1)) * 2 + 2 * kr[m][c];
                dst[0] = cand_key(c1[m][2 * c], 2 * x);
                dst[1] = vis1 ? cand_key(c1[m][2 * c + 1], ch1) : 0ull;
              }
            }
          }
        }
        wave_sync();
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const int it = lane + 64 * m;
          if (it < ITEMS) {
            const uint64_t* kq = key + (it & ~(KC - 1)) * 2;
            const uint64_t k0 = key[2 * it], k1 = key[2 * it + 1];
            int r0 = 0, r1 = 0;
#pragma unroll 4
            for (int s = 0; s < SLOTS; s += 2) {
              const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(kq + s);
              r0 += (kk.x > k0) + (kk.y > k0);
              r1 += (kk.x > k1) + (kk.y > k1);
            }
            // the node of a key: its low word holds the complemented index
            if (k0 != 0ull && r0 < K) np[(it & ~(KC - 1)) + r0] = (int)~(uint32_t)k0;
            if (k1 != 0ull && r1 < K) np[(it & ~(KC - 1)) + r1] = (int)~(uint32_t)k1;
          }
        }
        wave_sync();
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int it = lane + 64 * m;
        if (it < ITEMS) ip[m] = np[it];
      }
      wave_sync();
    }

    if (more) dense_fetch_wait();
    __syncthreads();
    if (!more) break;
    if (ln != l) nt = ntiles(ltn);
    l = ln;
    t = tn;
    buf ^= 1;
  }
  // the passes end at level l_bot: ip holds its kept nodes

  // ---- level l_bot - 1 candidates: the children of each kept node, 2K slots per query
  const int lc = l_bot - 1, twoK = 2 * K;
  // the item indices are formed again from an opaque copy of the lane: carried across the
  // passes they would cost registers the tile loop needs
  int lp = lane;
  asm volatile("" : "+v"(lp));
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int it = lp + 64 * m;
    const int iq = it / KC, ir = it % KC, i = iw + iq;
    if (it < ITEMS && ir < K && i < N) {
      const int p = ip[m];
      int c0 = p >= 0 ? 2 * p : -1;
      int c1 = (p >= 0 && 2 * p + 1 < geo.n[lc] && ((int64_t)(2 * p + 1) << (lc - 1)) <= ibq[m]) ? 2 * p + 1 : -1;
      if (lc == 1) {  // leaf candidates: the forced blocks are scored on their own
        if (c0 >= 0 && is_forced(c0, ibq[m])) c0 = -1;
        if (c1 >= 0 && is_forced(c1, ibq[m])) c1 = -1;
      }
      int32_t* dst = x2 + ((int64_t)bh * N + i) * twoK + 2 * ir;
      __builtin_nontemporal_store(c0, dst);
      __builtin_nontemporal_store(c1, dst + 1);
    }
  }

  // ---- forced leaf blocks {0, bw - 1, bw} of this wavefront's queries (one leaf block bw:
  // QPW divides C).  The workgroup's tiles are 0 and bfirst - 1 .. bqmax (at most 4).
  static_assert(kLeaf % QPW == 0, "a wavefront's queries share one leaf block");
  const int bfirst = iwg / C;
  int ft[4];
  int nft = 0;
  ft[nft++] = 0;
  for (int f = max(1, bfirst - 1); f <= bqmax && nft < 4; ++f) ft[nft++] = f;
  const bf16* kb = k + (int64_t)bh * N * D;
  u32x4 stg[F / kDenseWaves];
  __syncthreads();  // the staging buffers are free again
  dense_load_keys<D>(kb, N, ft[0], wave, lane, stg);
  dense_store_tile<D>(lds, 0, wave, lane, stg);
  __syncthreads();
  int nfw = 0;  // |F| of this wavefront's leaf block
  {
    int Fw[3];
    nfw = forced_blocks(bqw, Fw);
  }
  for (int x = 0; x < nft; ++x) {
    const int f = ft[x];
    dense_load_keys<D>(kb, N, ft[min(x + 1, nft - 1)], wave, lane, stg);  // next tile (or this one again)
    const bool mine = iw < N && (f == 0 || f == bqw - 1 || f == bqw);
    if (mine) {
      const int fidx = f == 0 ? 0 : (f == bqw - 1 ? 1 : nfw - 1);  // position in F (ascending)
      const char* Tt = lds + (x & 1) * TILE;
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        f32x16 a0, a1;
#pragma unroll
        for (int v = 0; v < 16; ++v) a0[v] = a1[v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          // fragments read per k-step (and per column group): this phase runs once, and
          // holding all of them would cost the routing loop a wavefront per SIMD
          const bf16x8 f0 = *reinterpret_cast<const bf16x8*>(Tt + (ks * 64 + lane) * 16);
          const bf16x8 f1 = *reinterpret_cast<const bf16x8*>(Tt + ((KS + ks) * 64 + lane) * 16);
          a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0, qf[cg][ks], a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1, qf[cg][ks], a1, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        const int i = iw + cg * (32 / G) + j / G;  // this lane's column's query
        if (f == bqw || 64 * f + 64 > N) {          // causal mask: only the current (or a short) block
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int ta = 64 * f + key_row(v, hh), tb = ta + 32;
            if (ta > i || ta >= N) a0[v] = -INFINITY;
            if (tb > i || tb >= N) a1[v] = -INFINITY;
          }
        }
        // columns past N still see live keys (ta <= N - 1 < i), so no NaN arises
        float lse = column_lse32(a0, a1, geo.s, geo.s_log2e);
        lse = group_sum<G>(lse);
        if (hh == 0 && j % G == 0 && i < N) fsc[((int64_t)bh * N + i) * 3 + fidx] = lse;
        // one column group at a time: overlapping them would raise the kernel's register
        // count above what three wavefronts per SIMD allow
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (x + 1 < nft) dense_store_tile<D>(lds, (x + 1) & 1, wave, lane, stg);
    __syncthreads();
  }
}

template <int D, int G, int KC>
int dense_launch(const Geo& g, const bf16* q, const float* pyr, const bf16* k, int32_t* x2, float* fsc,
                 bf16* qg, hipStream_t st) {
  constexpr int QW = kDenseWaves * DenseShape<G>::QPW;  // queries per workgroup
  const unsigned grid = (unsigned)(g.B * g.Hkv * ((g.N + QW - 1) / QW));
  if (g.scorer == PISA_LSE)
    route_dense_kernel<D, G, KC, false>
        <<<grid, 64 * kDenseWaves, dense_lds_bytes<D, G, KC>(), st>>>(q, pyr, k, g, dense_bottom(g), x2, fsc, qg);
  else
    route_dense_kernel<D, G, KC, true>
        <<<grid, 64 * kDenseWaves, dense_lds_bytes<D, G, KC>(), st>>>(q, pyr, k, g, dense_bottom(g), x2, fsc, qg);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

template <int D, int G>
int dense_k(const Geo& g, const bf16* q, const float* pyr, const bf16* k, int32_t* x2, float* fsc, bf16* qg,
            hipStream_t st) {
  if (g.K <= 8) return dense_launch<D, G, 8>(g, q, pyr, k, x2, fsc, qg, st);
  if (g.K <= 16) return dense_launch<D, G, 16>(g, q, pyr, k, x2, fsc, qg, st);
  return dense_launch<D, G, 32>(g, q, pyr, k, x2, fsc, qg, st);
}

template <int D>
int dense_g(const Geo& g, const bf16* q, const float* pyr, const bf16* k, int32_t* x2, float* fsc, bf16* qg,
            hipStream_t st) {
  switch (g.G) {
    case 1: return dense_k<D, 1>(g, q, pyr, k, x2, fsc, qg, st);
    case 2: return dense_k<D, 2>(g, q, pyr, k, x2, fsc, qg, st);
    case 4: return dense_k<D, 4>(g, q, pyr, k, x2, fsc, qg, st);
    case 8: return dense_k<D, 8>(g, q, pyr, k, x2, fsc, qg, st);
    case 16: return dense_k<D, 16>(g, q, pyr, k, x2, fsc, qg, st);
    default: return PISA_ERR_UNSUPPORTED;
  }
}

}  // namespace

int launch_route_upper_dense(const Geo& g, const void* q, const float* pyr, const void* k, int32_t* x2, float* fsc,
                              void* qg, hipStream_t st) {
  if (g.L < 3 || g.K > 32) return PISA_ERR_UNSUPPORTED;
  if (g.d == 128) return dense_g<128>(g, (const bf16*)q, pyr, (const bf16*)k, x2, fsc, (bf16*)qg, st);
  if (g.d == 64) return dense_g<64>(g, (const bf16*)q, pyr, (const bf16*)k, x2, fsc, (bf16*)qg, st);
  return PISA_ERR_UNSUPPORTED;
}

}  // namespace pisa
