// Prefill routing of the lowest routing levels (3 and 2, or 2 alone) from the leaf-block
// means under each query group's kept nodes, in one gather.
//
// What is computed is the top-down walk of "Block Sparse Attention with Log-Linear
// Complexity" (rcap.io explainer, top-down walk and scoring-rule paragraphs; agihunt.info
// summary, pyramid paragraph and kernels paragraph for the GQA head sum): a candidate's
// score is the sum over the G heads of the LogSumExp of s*q.child over its visible
// children, the Top-K candidates are kept (score descending, lower index first) and their
// children become the next level's candidates.
//
// How it is computed.  A pyramid node is the plain mean of its children, so q.P_2[m] is the
// mean of q.P_1 over the (one or two) leaf blocks of level-2 node m.  The 2K level-3
// candidates of a query group are the children of its K kept level-4 nodes; dotting q
// with the leaf-block means under each of them -- four per level-3 candidate, 8K in all --
// therefore gives every dot that levels 3 and 2 of the walk need: the level-2 dots (means
// of leaf pairs) that score the level-3 candidates, and the leaf dots that score whichever
// level-2 candidates the level-3 Top-K then opens.  That is as many dot products as the
// walk's two levels, but all of them are known before the first one is needed, so one
// burst of independent, contiguous gathers (4 leaf means = 2 KB per level-3 candidate)
// replaces two dependent rounds.  With the dense launch stopping one level lower (level-2
// candidates in), each of the K kept level-3 nodes contributes its four leaf means and
// only level 2 is walked here.
//
// Matrix cores: v_mfma_f32_16x16x32_bf16 over the level-1 routing copy's hi halves, four
// query groups of one leaf block per wavefront, B = their 16 (group, head) query columns.
// At d = 128 the products of the lo halves come from a compact fp8 copy that lo8_kernel
// writes into the workspace: each leaf's lo halves in e4m3 under a power-of-two scale that
// the E8M0 scale operand of v_mfma_scale_f32_16x16x128_f8f6f4 undoes, against the query
// columns in e5m2.  The lo product is itself ~2^-9 of a dot, so its fp8 rounding (~2^-4 of
// it) leaves the dots ~1e-5 from exact in score units, and a leaf costs 384 instead of 512
// bytes; at d = 64 the bf16 lo halves are multiplied as they are.  Tile j holds in row
// block rb the four leaf means of level-3 node Y[(rb + j) mod 4][j], so every lane's B
// operand is its own query fragment and each result lane finds its own group's rows in one
// tile of every four (mixed-row tiles; G = 4 only).
#include "route_dev.h"

namespace pisa {

namespace {

constexpr int kSubQueries = 512;  // queries per workgroup
// Tiles per batch of gathers (256K, levels 3-2: 1, 2 and 4 tiles took 1.49, 1.51 and
// 1.51 ms at 4, 3 and 2 wavefronts per SIMD).
constexpr int kSubTB = 1;

template <int KC, int NLEV>
struct SubLds {
  static constexpr int NT = NLEV == 2 ? 2 * KC : KC;  // tiles (level-3 nodes) per group
  int32_t Y[4][NT];         // level-3 node of tile j, -1 for none
  uint64_t k3[4][2 * KC];   // level-3 candidate keys (NLEV == 2)
  float s2[4][2 * NT];      // scores of the two level-2 children of tile j's node (NLEV == 2)
  uint64_t k2[4][2 * KC];   // level-2 candidate keys
  int32_t X2[4][2 * KC];    // level-2 candidates: slot 2r + c = child c of the kept level-3 node of rank r
  int32_t Lf[4][2 * KC];    // leaf candidates out
};

typedef int v8i __attribute__((ext_vector_type(8)));

// fp8 correction record of leaf n (d = 128): quads of four leaves, then the lane k-group kg,
// then the leaf in the quad; 32 bytes, byte 8 s + e holding dim 32 s + 8 kg + e -- the dims
// a route_sub lane holds in its query fragments, in the same order, so that four lanes of
// one k-group read one 128-byte line.
__device__ __forceinline__ int64_t lo8_piece(int64_t n, int kg) { return (n >> 2) * 512 + kg * 128 + (n & 3) * 32; }

// Thread = (leaf n, k-group kg), four consecutive lanes per leaf: the 32 lo halves of its
// dims from the level-1 routing copy, scaled by 2^S (S per leaf: the largest |lo| lands in
// [128, 256), inside e4m3's range), rounded to e4m3; the leaf's E8M0 byte 127 - S follows
// the records.  Leaves n1 .. n1q-1 get zeros (the level-2 launch never reads them).
__global__ __launch_bounds__(256) void lo8_kernel(const float* __restrict__ pyr, Geo geo, uint8_t* __restrict__ lo8) {
  constexpr int D = 128;
  const int bh = blockIdx.y;
  const int n1q = (geo.n1 + 3) & ~3;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int n = t >> 2, kg = t & 3;
  if (n >= n1q) return;  // all four lanes of a leaf alike
  const bf16* R1 = reinterpret_cast<const bf16*>(pyr + geo.means_floats()) + (int64_t)bh * geo.Tp * 2 * D;
  float r[32];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    // lo half of 8-dim piece 4 s + kg (leaf 0's when n is past n1; zeroed below)
    const uint4 u = *reinterpret_cast<const uint4*>(R1 + rc_node(n < geo.n1 ? n : 0, D) + rc_piece(4 * s + kg) + 64);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      r[8 * s + 2 * h] = n < geo.n1 ? bf2f(w[h] & 0xFFFFu) : 0.f;
      r[8 * s + 2 * h + 1] = n < geo.n1 ? bf2f(w[h] >> 16) : 0.f;
    }
  }
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) mx = fmaxf(mx, fabsf(r[e]));
  mx = fmaxf(mx, __shfl_xor(mx, 1));
  mx = fmaxf(mx, __shfl_xor(mx, 2));
  // mx < 2^E with E = biased exponent - 126; below 2^-100 the record stays zero
  const uint32_t eb = __float_as_uint(mx) >> 23;
  const bool tiny = eb < 27;
  const int S = tiny ? 0 : 134 - (int)eb;  // 8 - E
  int w[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const float a = tiny ? 0.f : ldexpf(r[4 * v], S), b = tiny ? 0.f : ldexpf(r[4 * v + 1], S);
    const float c = tiny ? 0.f : ldexpf(r[4 * v + 2], S), d = tiny ? 0.f : ldexpf(r[4 * v + 3], S);
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w[v] = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, x, true);
  }
  uint8_t* rec = lo8 + (int64_t)bh * n1q * D + lo8_piece(n, kg);
  reinterpret_cast<uint4*>(rec)[0] = uint4{(uint32_t)w[0], (uint32_t)w[1], (uint32_t)w[2], (uint32_t)w[3]};
  reinterpret_cast<uint4*>(rec)[1] = uint4{(uint32_t)w[4], (uint32_t)w[5], (uint32_t)w[6], (uint32_t)w[7]};
  if (kg == 0) lo8[(int64_t)geo.B * geo.Hkv * n1q * D + (int64_t)bh * n1q + n] = (uint8_t)(127 - S);
}

template <bool TRUNC>
__device__ __forceinline__ float sub_pair(float y0, float y1, float c2) {
  // y0: a visible child's dot; y1: the other child's, -inf when missing or not visible
  const float mx = fmaxf(y0, y1), mn = fminf(y0, y1);
  if constexpr (TRUNC)
    return pair_trunc(mx, mn, 1.f, c2);
  else
    return mx + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(mn - mx));
}

// NLEV = 2: x2 holds the 2K level-3 candidates per query group (slots 2r, 2r+1 = children of
// the kept level-4 node of rank r, -1 where missing or not visible); levels 3 and 2 are
// walked.  NLEV = 1: x2 holds the 2K level-2 candidates (children of the K kept level-3
// nodes); level 2 is walked.  Writes the 2K leaf candidates per query group that are not
// forced blocks (-1 elsewhere; slots 2r, 2r+1 = children of the kept level-2 node of rank r)
// and histograms the (query group, level-2 node) pairs into cnt.
template <int D, int KC, int NLEV, bool TRUNC>
__global__ __launch_bounds__(256, NLEV == 2 ? 4 : 3) void route_sub_kernel(const bf16* __restrict__ q, const float* __restrict__ pyr,
                                                        Geo geo, const int32_t* __restrict__ x2,
                                                        int32_t* __restrict__ cand, int32_t* __restrict__ cnt,
                                                        const bf16* __restrict__ qg, const uint8_t* __restrict__ lo8) {
  constexpr int G = 4, KS = D / 32;
  constexpr bool LO8 = D == 128;  // lo products from the fp8 records
  using S = SubLds<KC, NLEV>;
  extern __shared__ __attribute__((aligned(16))) int hist[];
  __shared__ S sl_all[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int BH = geo.B * geo.Hkv;
  const int bh = blockIdx.x % BH;  // the workgroups of one XCD (w mod 8) gather from few heads
  const int qr0 = (blockIdx.x / BH) * kSubQueries;
  const bool lhist = geo.n1p <= kHistMaxBins;
  if (lhist) {
    for (int t = threadIdx.x; t < geo.n1p; t += 256) hist[t] = 0;
    __syncthreads();
  }
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  S* w = &sl_all[wave];
  // routing copy of this (b, h); level 1 comes first, so leaf c is node c
  const bf16* R1 = reinterpret_cast<const bf16*>(pyr + geo.means_floats()) + (int64_t)bh * geo.Tp * 2 * D;
  const int N = geo.N, K = geo.K, twoK = 2 * K, n1 = geo.n[1];
  const int n1q = (n1 + 3) & ~3;
  const uint8_t* L8 = LO8 ? lo8 + (int64_t)bh * n1q * D : nullptr;                                // records
  const uint8_t* S8 = LO8 ? lo8 + (int64_t)geo.B * geo.Hkv * n1q * D + (int64_t)bh * n1q : nullptr;  // scales
  const int ntile = NLEV == 2 ? twoK : K;
  const float c2 = trunc_c2(geo.scorer, true);
  const int m = lane & 15, kg = lane >> 4;
  const int gown = m >> 2, r = m & 3;  // query column: group, head
  const int rb = m >> 2, v = m & 3;    // A row: row block, row in it
  const int jo = (gown - kg) & 3;      // result tiles j = jo (mod 4) hold this lane's rows
  const int gl = lane >> 4, xl = lane & 15;  // ranking: group, slot lane
  const int64_t qbase = ((int64_t)b * geo.Hq + h * G) * N;

  // Query fragments (column (gown, r), dims 32 s + 8 kg .. +8) and the tiles' level-3 nodes
  // (lane (gl, xl): tiles xl, xl + 16, ...) of quad qd, loaded one quad ahead so that their
  // HBM latency overlaps the current quad's gathers.
  constexpr int YPL = (S::NT + 15) / 16;
  auto fetch = [&](int qd, bf16x8 (&qf)[KS], int (&yf)[YPL]) {
    const int f0 = qr0 + qd * 4;
    const int ii = f0 + gown;
    if (qd < kSubQueries / 4 && ii < N) {
      // piece 4 s + kg of head r: from the regrouped copy (the group's heads adjacent per
      // piece) when the dense launch wrote one, else from q's own rows
      const bf16* p = qg ? qg + ((int64_t)bh * N + ii) * (G * D) + (kg * G + r) * 8
                         : q + (qbase + (int64_t)r * N + ii) * D + 8 * kg;
      const int step = qg ? 32 * G : 32;
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p + step * s));
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)0.f;
    }
    const int fi = f0 + gl;
    const int64_t frow = (int64_t)bh * N + fi;
#pragma unroll
    for (int u = 0; u < YPL; ++u) {
      const int j = xl + 16 * u;
      int y = -1;
      if (qd < kSubQueries / 4 && fi < N && j < ntile) {
        if constexpr (NLEV == 2) {
          y = __builtin_nontemporal_load(&x2[frow * twoK + j]);
        } else {
          const int c = __builtin_nontemporal_load(&x2[frow * twoK + 2 * j]);
          y = c >= 0 ? c >> 1 : -1;
        }
      }
      yf[u] = y;
    }
  };
  // Gathers of tiles t0 .. t0+TB-1 (a batch: 2 TB KS loads per lane, all issued before the
  // first MFMA that needs them: left to itself the compiler keeps two in flight and waits
  // on each, a dependent chain of L2 round trips).
  auto load_batch = [&](int t0, bf16x8 (&hi)[kSubTB][KS], bf16x8 (&lo)[kSubTB][KS], v8i (&l8)[kSubTB],
                        int (&sc)[kSubTB]) {
#pragma unroll
    for (int u = 0; u < kSubTB; ++u) {
      const int j = t0 + u;
      const int y = j < ntile ? w->Y[(rb + j) & 3][j] : -1;
      const int leaf = 4 * y + v;
      // a missing leaf (or an empty tile) reads leaf 0 instead; its rows are never used
      // k-step s, lane group kg <-> 8-dim piece 4 s + kg (hi, then lo 64 bf16 later)
      const int lf = (y >= 0 && leaf < n1) ? leaf : 0;
      const bf16* rp = R1 + rc_node(lf, D) + rc_piece(kg);
      if constexpr (LO8) {
        // this lane's A row is leaf lf: its record piece for k-group kg and its scale
        // (loaded first: the fp8 product opens the tile's accumulation)
        l8[u] = *reinterpret_cast<const v8i*>(L8 + lo8_piece(lf, kg));
        sc[u] = S8[lf];
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) hi[u][s] = *reinterpret_cast<const bf16x8*>(rp + 256 * s);
      if constexpr (!LO8) {
#pragma unroll
        for (int s = 0; s < KS; ++s) lo[u][s] = *reinterpret_cast<const bf16x8*>(rp + 256 * s + 64);
      }
    }
  };

  bf16x8 qb[KS], qn[KS];
  int yn[YPL];
  fetch(wave, qn, yn);

#pragma unroll 1
  for (int quad = wave; quad < kSubQueries / 4; quad += 4) {
    const int i0 = qr0 + quad * 4;
    if (i0 >= N) break;          // uniform across the wavefront
    const int bq = i0 / kLeaf;   // four consecutive queries share one leaf block (C = kLeaf)
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = qn[s];
    // the query columns in e5m2 for the fp8 lo products, in the records' dim order (byte
    // 8 s + e = dim 32 s + 8 kg + e); |q| past e5m2's largest finite value is clamped to it
    v8i q8;
    if constexpr (LO8) {
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int s = v >> 1, e = 4 * (v & 1);
        float c[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) c[h] = __builtin_amdgcn_fmed3f((float)qb[s][e + h], -57344.f, 57344.f);
        const int x = __builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], 0, false);
        q8[v] = __builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], x, true);
      }
    }
#pragma unroll
    for (int u = 0; u < YPL; ++u)
      if (xl + 16 * u < S::NT) w->Y[gl][xl + 16 * u] = yn[u];
    fetch(quad + 4, qn, yn);  // the next quad's query fragments and tile nodes
    const int i = i0 + gl;  // the query of this lane's ranking group
    const int64_t row = (int64_t)bh * N + i;
    for (int x = xl; x < 2 * KC; x += 16) {
      w->k2[gl][x] = 0ull;
      w->X2[gl][x] = -1;
      w->Lf[gl][x] = -1;
    }
    wave_sync();

    for (int t0 = 0; t0 < ntile; t0 += 4) {
      f32x4 acc[4];
#pragma unroll
      for (int t1 = 0; t1 < 4; t1 += kSubTB) {
        bf16x8 hi[kSubTB][KS], lo[kSubTB][KS];
        v8i l8[kSubTB];
        int sc[kSubTB];
        load_batch(t0 + t1, hi, lo, l8, sc);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kSubTB; ++u) {
          acc[t1 + u] = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (LO8) {
            // the lo products first (their record registers free at once): A = e4m3
            // records (format 0) with their E8M0 scales, B = e5m2 queries (format 1)
            acc[t1 + u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(l8[u], q8, acc[t1 + u], 0, 1, 0, sc[u], 0, 127);
          }
#pragma unroll
          for (int s = 0; s < KS; ++s)
            acc[t1 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[u][s], qb[s], acc[t1 + u], 0, 0, 0);
          if constexpr (!LO8) {
#pragma unroll
            for (int s = 0; s < KS; ++s)
              acc[t1 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[u][s], qb[s], acc[t1 + u], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // this lane's tile of the four: leaf dots a[0..3] of leaves 4y .. 4y+3, head r
      f32x4 a = acc[0];
      a = jo == 1 ? acc[1] : a;
      a = jo == 2 ? acc[2] : a;
      a = jo == 3 ? acc[3] : a;
      const int jt = t0 + jo;
      const int y = jt < ntile ? w->Y[gown][jt] : -1;
      const int l0 = 4 * y;
      const bool e1 = l0 + 1 < n1, e2 = l0 + 2 < n1, e3 = l0 + 3 < n1;
      const bool v1 = e1 && l0 + 1 <= bq, v2 = e2 && l0 + 2 <= bq, v3 = e3 && l0 + 3 <= bq;
      // scores of level-2 nodes 2y (leaves l0, l0+1) and 2y+1 (leaves l0+2, l0+3; exists iff e2)
      float s2a = sub_pair<TRUNC>(a[0], v1 ? a[1] : -INFINITY, c2);
      float s2b = sub_pair<TRUNC>(a[2], v3 ? a[3] : -INFINITY, c2);
      float s3 = 0.f;
      if constexpr (NLEV == 2) {
        // level-3 node y: its level-2 children's dots are the means of their leaves' dots
        const float d2a = e1 ? 0.5f * (a[0] + a[1]) : a[0];
        const float d2b = e3 ? 0.5f * (a[2] + a[3]) : a[2];
        s3 = group_sum<G>(sub_pair<TRUNC>(d2a, v2 ? d2b : -INFINITY, c2));
      }
      s2a = group_sum<G>(s2a);
      s2b = group_sum<G>(s2b);
      if (r == 0 && jt < ntile) {
        if constexpr (NLEV == 2) {
          w->k3[gown][jt] = y >= 0 ? cand_key(s3, y) : 0ull;
          w->s2[gown][2 * jt] = s2a;
          w->s2[gown][2 * jt + 1] = s2b;
        } else {  // tile jt = the kept level-3 node of rank jt: level-2 slots 2jt, 2jt+1
          w->k2[gown][2 * jt] = y >= 0 ? cand_key(s2a, 2 * y) : 0ull;
          w->k2[gown][2 * jt + 1] = (y >= 0 && v2) ? cand_key(s2b, 2 * y + 1) : 0ull;
          w->X2[gown][2 * jt] = y >= 0 ? 2 * y : -1;
          w->X2[gown][2 * jt + 1] = (y >= 0 && v2) ? 2 * y + 1 : -1;
        }
      }
    }
    wave_sync();

    if constexpr (NLEV == 2) {
      // Top-K of level 3; the kept node of rank r opens level-2 slots 2r, 2r+1
      for (int x = xl; x < twoK; x += 16) {
        const uint64_t my = w->k3[gl][x];
        int rank = 0;
#pragma unroll 8
        for (int y2 = 0; y2 < twoK; ++y2) rank += w->k3[gl][y2] > my;
        if (my != 0ull && rank < K) {
          const int y = w->Y[gl][x];
          const bool v2 = 4 * y + 2 < n1 && 4 * y + 2 <= bq;
          w->X2[gl][2 * rank] = 2 * y;
          w->k2[gl][2 * rank] = cand_key(w->s2[gl][2 * x], 2 * y);
          w->X2[gl][2 * rank + 1] = v2 ? 2 * y + 1 : -1;
          w->k2[gl][2 * rank + 1] = v2 ? cand_key(w->s2[gl][2 * x + 1], 2 * y + 1) : 0ull;
        }
      }
      wave_sync();
    }

    // Top-K of level 2; the kept node of rank r gives leaf slots 2r, 2r+1
    for (int x = xl; x < twoK; x += 16) {
      const uint64_t my = w->k2[gl][x];
      int rank = 0;
#pragma unroll 8
      for (int y2 = 0; y2 < twoK; ++y2) rank += w->k2[gl][y2] > my;
      if (my != 0ull && rank < K) {
        const int mn = w->X2[gl][x];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int leaf = 2 * mn + c;
          const bool ok = leaf < n1 && leaf <= bq && !is_forced(leaf, bq);
          w->Lf[gl][2 * rank + c] = ok ? leaf : -1;
        }
      }
    }
    wave_sync();

    if (i < N) {
      for (int x = xl; x < twoK; x += 16) {
        const int leaf = w->Lf[gl][x];
        __builtin_nontemporal_store(leaf, &cand[row * twoK + x]);
        if ((x & 1) == 0) {
          const int sib = w->Lf[gl][x + 1];
          if (leaf >= 0 || sib >= 0) {
            const int node = (leaf >= 0 ? leaf : sib) >> 1;
            if (lhist)
              atomicAdd(&hist[node], 1);
            else
              atomicAdd(&cnt[bh * geo.n1p + node], 1);
          }
        }
      }
    }
    wave_sync();
  }
  if (lhist) {
    __syncthreads();
    for (int t = threadIdx.x; t < geo.n1p; t += 256)
      if (hist[t]) atomicAdd(&cnt[bh * geo.n1p + t], hist[t]);
  }
}

template <int D, int KC, int NLEV>
int sub_launch(const Geo& g, const void* q, const float* pyr, const int32_t* x2, int32_t* cand, int32_t* cnt,
               const void* qg, uint8_t* lo8, hipStream_t st) {
  if constexpr (D == 128) {
    if (!lo8) return PISA_ERR_INTERNAL;
    const int n1q = (g.n1 + 3) & ~3;
    lo8_kernel<<<dim3((unsigned)((4 * n1q + 255) / 256), (unsigned)(g.B * g.Hkv)), 256, 0, st>>>(pyr, g, lo8);
    if (hipGetLastError() != hipSuccess) return PISA_ERR_HIP;
  }
  const unsigned grid = (unsigned)(g.B * g.Hkv * ((g.N + kSubQueries - 1) / kSubQueries));
  const size_t hbytes = g.n1p <= kHistMaxBins ? sizeof(int) * (size_t)g.n1p : 0;
  if (g.scorer == PISA_LSE)
    route_sub_kernel<D, KC, NLEV, false><<<grid, 256, hbytes, st>>>((const bf16*)q, pyr, g, x2, cand, cnt, (const bf16*)qg, lo8);
  else
    route_sub_kernel<D, KC, NLEV, true><<<grid, 256, hbytes, st>>>((const bf16*)q, pyr, g, x2, cand, cnt, (const bf16*)qg, lo8);
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

template <int D, int NLEV>
int sub_k(const Geo& g, const void* q, const float* pyr, const int32_t* x2, int32_t* cand, int32_t* cnt,
          const void* qg, uint8_t* lo8, hipStream_t st) {
  if (g.K <= 8) return sub_launch<D, 8, NLEV>(g, q, pyr, x2, cand, cnt, qg, lo8, st);
  if (g.K <= 16) return sub_launch<D, 16, NLEV>(g, q, pyr, x2, cand, cnt, qg, lo8, st);
  return sub_launch<D, 32, NLEV>(g, q, pyr, x2, cand, cnt, qg, lo8, st);
}

}  // namespace

bool route_sub_supported(const Geo& g, int l_x) {
  return g.G == 4 && g.L >= 3 && g.C % 4 == 0 && g.K <= 32 && (l_x == 2 || l_x == 3) && (g.d == 64 || g.d == 128);
}

int launch_route_sub(const Geo& g, int l_x, const void* q, const float* pyr, const int32_t* x2, int32_t* cand,
                     int32_t* cnt, const void* qg, uint8_t* lo8, hipStream_t st) {
  if (!route_sub_supported(g, l_x)) return PISA_ERR_UNSUPPORTED;
  if (g.d == 128)
    return l_x == 3 ? sub_k<128, 2>(g, q, pyr, x2, cand, cnt, qg, lo8, st) : sub_k<128, 1>(g, q, pyr, x2, cand, cnt, qg, lo8, st);
  return l_x == 3 ? sub_k<64, 2>(g, q, pyr, x2, cand, cnt, qg, lo8, st) : sub_k<64, 1>(g, q, pyr, x2, cand, cnt, qg, lo8, st);
}

}  // namespace pisa
