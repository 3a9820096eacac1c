// Block-sparse attention over the selected blocks, the consumer of the selection
// ("Block Sparse Attention with Log-Linear Complexity": agihunt.info summary, opening
// paragraph: each query reads only its Top-K tiles of C keys, so the attention pass is
// linear in N; rcap.io explainer, first paragraphs: attention over the original keys of
// the picked blocks).  Per query head: out = sum_t softmax_t(s q.k_t) v_t over the causal
// keys of its row's selected blocks (shared by the GQA group), lse = log sum_t exp(s q.k_t).
//
// Query-major: one wavefront per query group walks the group's <= K selected blocks with
// an online softmax in the log2 domain.  Per block, lane t scores key t of the block
// against the G query rows (fp32 in LDS), the wavefront takes the block max and sum, and
// the value tile is read as 16-byte row pieces (lane = (row group, 8 or 4 dims)) and
// accumulated with the probabilities broadcast from LDS; the row groups are summed once at
// the end.  Every (query group, block) pair reads its key and value tiles (2 C d elements),
// which is the pass's traffic: there is no reuse between query groups that picked the same
// block.
#include "final_dev.h"
#include "route_dev.h"

namespace pisa {

namespace {

template <typename T>
__device__ __forceinline__ void store_out(T* p, const float* x, int n);
template <>
__device__ __forceinline__ void store_out<float>(float* p, const float* x, int n) {
  for (int e = 0; e < n; e += 4) *reinterpret_cast<float4*>(p + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
}
template <>
__device__ __forceinline__ void store_out<bf16>(bf16* p, const float* x, int n) {
  for (int e = 0; e < n; e += 8) {
    u32x4 u;
#pragma unroll
    for (int w = 0; w < 4; ++w) u[w] = f2bf_rne(x[e + 2 * w]) | (f2bf_rne(x[e + 2 * w + 1]) << 16);
    *reinterpret_cast<u32x4*>(p + e) = u;
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void attn_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, Geo geo, const int32_t* __restrict__ idx,
                                                   int32_t decode, T* __restrict__ out, float* __restrict__ lse) {
  constexpr int DPL = Vec<T>::N;    // dims per 16-byte value piece
  constexpr int LPR = D / DPL;      // lanes per value row
  constexpr int RG = 64 / LPR;      // value rows read together
  __shared__ float qs_all[4][G * (D + kQPad)];
  __shared__ float pl_all[4][G][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = geo.N, C = geo.C, K = geo.K;
  const int nq = decode ? 1 : N;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= (int64_t)geo.B * geo.Hkv * nq) return;  // whole wavefront; no workgroup barrier follows
  const int bh = (int)(row / nq);
  const int i = decode ? N - 1 : (int)(row % nq);
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  const int bq = i / C;
  float* qs = qs_all[wave];
  float(*pl)[64] = pl_all[wave];

  const T* rows[G];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const int64_t hq = (int64_t)b * geo.Hq + h * G + r;
    rows[r] = q + (decode ? hq * D : (hq * N + i) * D);
  }
  load_qrows<T, D, G>(rows, qs, lane);
  const int my_blk = lane < K ? idx[row * K + lane] : -1;
  wave_sync();

  const T* kb = k + (int64_t)bh * N * D;
  const T* vb = v + (int64_t)bh * N * D;
  const float sl = geo.s_log2e;
  const int rg = lane / LPR, dg = lane % LPR;
  float m2[G], l[G], acc[G][DPL];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    m2[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[r][e] = 0.f;
  }

  for (int u = 0; u < K; ++u) {
    const int j = __shfl(my_blk, u);
    if (j < 0 || j > bq) continue;  // uniform: padding, or a block after the query's own
    // scores of the block's keys (lane = key); a selected block j <= b always has key jC <= i
    const int t = j * C + lane;
    const bool valid = lane < C && t <= i;
    float dot[G];
#pragma unroll
    for (int r = 0; r < G; ++r) dot[r] = 0.f;
    if (valid) {
      const T* kr = kb + (int64_t)t * D;
#pragma unroll 4
      for (int e = 0; e < D; e += DPL) {
        float x[DPL];
        Vec<T>::load(kr + e, x);
#pragma unroll
        for (int r = 0; r < G; ++r)
#pragma unroll
          for (int w = 0; w < DPL; ++w) dot[r] += x[w] * qs[r * (D + kQPad) + e + w];
      }
    }
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const float x = valid ? dot[r] * sl : -INFINITY;
      const float mnew = fmaxf(m2[r], wave_max(x));
      const float scale = __builtin_amdgcn_exp2f(m2[r] - mnew);  // 0 on the first block
      const float p = valid ? __builtin_amdgcn_exp2f(x - mnew) : 0.f;
      l[r] = l[r] * scale + wave_sum(p);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[r][e] *= scale;
      m2[r] = mnew;
      pl[r][lane] = p;
    }
    wave_sync();
    // values: row group rg takes rows rg, rg + RG, ...; rows past the query read row i
    // with probability 0
#pragma unroll 4
    for (int kr = rg; kr < C; kr += RG) {
      const int tv = min(j * C + kr, i);
      float x[DPL];
      Vec<T>::load(vb + (int64_t)tv * D + dg * DPL, x);
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const float p = pl[r][kr];
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[r][e] += p * x[e];
      }
    }
    wave_sync();
  }

  // sum the row groups, normalise, write
#pragma unroll
  for (int r = 0; r < G; ++r)
#pragma unroll
    for (int e = 0; e < DPL; ++e)
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) acc[r][e] += __shfl_xor(acc[r][e], o);
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const int64_t hq = (int64_t)b * geo.Hq + h * G + r;
    const int64_t orow = decode ? hq : hq * N + i;
    const float inv = l[r] > 0.f ? 1.f / l[r] : 0.f;
    if (rg == 0) {
      float y[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) y[e] = acc[r][e] * inv;
      store_out<T>(out + orow * D + dg * DPL, y, DPL);
    }
    if (lse && lane == 0) lse[orow] = l[r] > 0.f ? (m2[r] + __builtin_amdgcn_logf(l[r])) * 0.6931471805599453f : -INFINITY;
  }
}

template <typename T, int D>
int attn_g(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx, int decode, void* out,
           float* lse, hipStream_t st) {
  const int64_t rows = (int64_t)g.B * g.Hkv * (decode ? 1 : g.N);
  const unsigned grid = (unsigned)((rows + 3) / 4);
  const T *qq = (const T*)q, *kk = (const T*)k, *vv = (const T*)v;
  T* oo = (T*)out;
  switch (g.G) {
    case 1: attn_kernel<T, D, 1><<<grid, 256, 0, st>>>(qq, kk, vv, g, idx, decode, oo, lse); break;
    case 2: attn_kernel<T, D, 2><<<grid, 256, 0, st>>>(qq, kk, vv, g, idx, decode, oo, lse); break;
    case 4: attn_kernel<T, D, 4><<<grid, 256, 0, st>>>(qq, kk, vv, g, idx, decode, oo, lse); break;
    case 8: attn_kernel<T, D, 8><<<grid, 256, 0, st>>>(qq, kk, vv, g, idx, decode, oo, lse); break;
    case 16: attn_kernel<T, D, 16><<<grid, 256, 0, st>>>(qq, kk, vv, g, idx, decode, oo, lse); break;
    default: return PISA_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? PISA_OK : PISA_ERR_HIP;
}

// ---- key-major form (bf16 prefill) ----
//
// The (query group, selected block) pairs are sorted by block (counting sort), so each
// block's key and value tiles are staged in LDS once per chunk of 4 kAttnColGroups 32/G
// pairs (four wavefronts x kAttnColGroups column groups of 32 (pair, head) columns) instead
// of being gathered for every pair.  Per chunk, on
// v_mfma_f32_32x32x16_bf16: S = K Q^T (rows = 64 keys, columns = 32 (pair, head) per
// wavefront), the block softmax in registers, then O^T = V^T P with the keys of each k-step
// taken in the order the lane already holds its probabilities (k-step s, lane half hh,
// element e <-> key 32 (s >> 1) + 16 (s & 1) + 8 (e >> 2) + 4 hh + (e & 3)), the value tile
// staged transposed so that those keys are two 8-byte LDS reads.  The transposed product
// leaves each lane four consecutive dims of its own column's output row per result group:
// each pair's block-normalised output (bf16) is staged in LDS in 8-byte pieces and leaves
// in 16-byte pieces, with its log2-sum-exp.  The forced blocks {0, b-1, b} of leaf block b
// are shared by all its queries: they are left out of the pairs and attended per leaf block
// by attn_forced_kernel, which writes one combined partial per (query, head).  One
// wavefront per query group then merges that partial with its other slots' partials.

// Candidate array of the pairs (per_row = K slots per query group, -1 where the slot is
// padding, names a block after the query's own or one of its forced blocks) and their
// count per list (range, b h, block): query i belongs to range i / R (R a multiple of
// kLeafQueries, so a workgroup's queries share one range).
__global__ __launch_bounds__(256) void attn_cand_kernel(const int32_t* __restrict__ idx, Geo geo, int32_t R,
                                                        int32_t* __restrict__ cand, int32_t* __restrict__ cnt) {
  extern __shared__ __attribute__((aligned(16))) int hist[];
  const int BH = geo.B * geo.Hkv, K = geo.K;
  const int bh = blockIdx.x % BH;
  const int q0 = (blockIdx.x / BH) * kLeafQueries, q1 = min(geo.N, q0 + kLeafQueries);
  const int lrow = (q0 / R) * BH + bh;  // this workgroup's lists: lrow * n1 + block
  const bool lhist = geo.n1 <= kHistMaxBins;
  if (lhist) {
    for (int t = threadIdx.x; t < geo.n1; t += 256) hist[t] = 0;
    __syncthreads();
  }
  const int64_t base = ((int64_t)bh * geo.N + q0) * K;
  const int n = (q1 - q0) * K;
  for (int t = threadIdx.x; t < n; t += 256) {
    const int i = q0 + t / K;
    const int j = idx[base + t];
    // the forced blocks of the query's leaf block are attended densely (attn_forced_kernel)
    const bool ok = j >= 0 && j <= i / geo.C && !is_forced(j, i / geo.C);
    cand[base + t] = ok ? j : -1;
    if (ok) {
      if (lhist) atomicAdd(&hist[j], 1);
      else atomicAdd(&cnt[lrow * geo.n1 + j], 1);
    }
  }
  if (lhist) {
    __syncthreads();
    for (int t = threadIdx.x; t < geo.n1; t += 256)
      if (hist[t]) atomicAdd(&cnt[lrow * geo.n1 + t], hist[t]);
  }
}

// Column groups of 32 (pair, head) columns each wavefront attends per chunk: the staged key
// and value tiles serve 4 kAttnColGroups column groups of a block's list (256K, chunk
// kernel plus merge: 1, 2, 4, 8 and 16 groups took 8.84, 8.46, 7.49, 6.98 and 6.71 ms; with
// the transposed value product, 16 and 32 groups 6.37 and 6.20 ms).
constexpr int kAttnColGroups = 32;

template <int D, int G>
__global__ __launch_bounds__(256) void attn_chunk_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                         const bf16* __restrict__ v, Geo geo,
                                                         const int32_t* __restrict__ off,
                                                         const int32_t* __restrict__ choff,
                                                         const int32_t* __restrict__ entries, int32_t Mlo,
                                                         int32_t Mhi, int32_t i0, int32_t R,
                                                         float* __restrict__ plse, bf16* __restrict__ po) {
  // one query range: lists [Mlo, Mhi) (those of queries i0 .. i0 + R - 1); the partials of
  // query i of (b, h) sit at row b h * R + (i - i0) of the range's partial buffers
  constexpr int EW = 32 / G;                    // pairs per column group
  constexpr int NCG = kAttnColGroups;
  constexpr int QC = 4 * NCG * EW;              // pairs per chunk (workgroup)
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int VTR = kLeaf + 8;  // padded row (keys) of the transposed value tile
  constexpr int OSR = D + 8;      // padded row of a wavefront's staged output
  // the chunk's entries (-1 past its end) in LDS while they take at most 4 KB (G >= 4); with
  // fewer heads per group the chunk is longer and its copy would cost a workgroup per CU
  constexpr bool kLdsEnt = QC <= 1024;
  constexpr int EPT = kLdsEnt ? QC / 256 : 1;
  static_assert(!kLdsEnt || QC % 256 == 0, "the chunk's entries split evenly over the threads");
  __shared__ int32_t ents[kLdsEnt ? QC : 1];
  __shared__ __attribute__((aligned(16))) bf16 kt[kLeaf * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 vt[D * VTR];
  __shared__ __attribute__((aligned(16))) bf16 os_all[4][32 * OSR];
  __shared__ int64_t px_all[4][32];

  const int c = choff[Mlo] + blockIdx.x;
  if (c >= choff[Mhi]) return;  // uniform: grid is an upper bound on the range's chunk count
  const int list = find_chunk_list(choff, Mlo, Mhi, c, threadIdx.x & 63);  // largest list whose first chunk is <= c
  const int bh = (list / geo.n1) % (geo.B * geo.Hkv), j = list % geo.n1;
  const int e0 = off[list] + (c - choff[list]) * QC;
  const int e1 = min(e0 + QC, off[list + 1]);
  const int N = geo.N, K = geo.K;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int r = col % G;
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  const bf16* qh = q + ((int64_t)b * geo.Hq + h * G + r) * N * D;
  // entry of this lane's column in column group u of the wavefront (-1: none): the first
  // from global memory, the others from the chunk's copy in LDS (loaded with the tiles, so
  // no column group waits on a global round trip for its entry index)
  auto entry = [&](int u) {
    const int e = e0 + (u * 4 + wave) * EW + col / G;
    return e < e1 ? entries[e] : -1;
  };
  int ent = entry(0);
  bf16x8 bq[KS];
  load_bfrag<D>(qh + (int64_t)max(ent >> 6, 0) * D, ent >= 0, hh, bq);
  int ev[EPT];
  if constexpr (kLdsEnt) {
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int t = threadIdx.x + 256 * x;
      ev[x] = e0 + t < e1 ? entries[e0 + t] : -1;
    }
  }

  stage_tile<D>(k + (int64_t)bh * N * D, j * kLeaf, N, kt);
  {  // value tile, transposed: vt[dim][key] (zeros past N)
    const bf16* vb = v + (int64_t)bh * N * D;
    for (int t = threadIdx.x; t < kLeaf * (D / 8); t += 256) {
      const int key = t / (D / 8), d8 = (t % (D / 8)) * 8;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j * kLeaf + key < N) x = *reinterpret_cast<const u32x4*>(vb + (int64_t)(j * kLeaf + key) * D + d8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vt[(d8 + 2 * w) * VTR + key] = (bf16)(x[w] & 0xFFFFu);
        vt[(d8 + 2 * w + 1) * VTR + key] = (bf16)(x[w] >> 16);
      }
    }
  }
  if constexpr (kLdsEnt) {
#pragma unroll
    for (int x = 0; x < EPT; ++x) ents[threadIdx.x + 256 * x] = ev[x];
  }
  __syncthreads();

  int64_t* px = px_all[wave];
  bf16* os = os_all[wave];
  const float sl = geo.s_log2e;
  for (int u = 0; u < NCG; ++u) {
    if (e0 + (u * 4 + wave) * EW >= e1) break;  // uniform across the wavefront
    int ent_n = -1;
    if (u + 1 < NCG) ent_n = kLdsEnt ? ents[((u + 1) * 4 + wave) * EW + col / G] : entry(u + 1);
    bf16x8 bqn[KS];
    load_bfrag<D>(qh + (int64_t)max(ent_n >> 6, 0) * D, ent_n >= 0, hh, bqn);
    const bool valid = ent >= 0;
    const int i = valid ? ent >> 6 : 0, slot = valid ? ent & 63 : 0;

    f32x16 s0, s1;
    tile_mfma32<D>(kt, bq, lane, s0, s1);
    // block softmax of the column in log2 units; keys after the query or past N are masked
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int t0 = j * kLeaf + key_row(w, hh), t1 = t0 + 32;
      s0[w] = (t0 <= i && t0 < N) ? s0[w] * sl : -INFINITY;
      s1[w] = (t1 <= i && t1 < N) ? s1[w] * sl : -INFINITY;
      mx = fmaxf(mx, fmaxf(s0[w], s1[w]));
    }
    mx = xor32_max(mx);  // key 64 j <= i is live for a valid pair
    if (!valid) mx = 0.f;                // padding columns: all probabilities 0, never written
    float sum = 0.f;
    bf16x8 pa[4];
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const float p0 = __builtin_amdgcn_exp2f(s0[w] - mx), p1 = __builtin_amdgcn_exp2f(s1[w] - mx);
      sum += p0 + p1;
      pa[w >> 3][w & 7] = (__bf16)p0;
      pa[2 + (w >> 3)][w & 7] = (__bf16)p1;
    }
    sum = xor32_sum(sum);

    f32x16 ao[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int w = 0; w < 16; ++w) ao[db][w] = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16* vr = vt + (32 * db + col) * VTR + 32 * (s >> 1) + 16 * (s & 1) + 4 * hh;
        const uint2 x0 = *reinterpret_cast<const uint2*>(vr), x1 = *reinterpret_cast<const uint2*>(vr + 8);
        const u32x4 xv = {x0.x, x0.y, x1.x, x1.y};
        ao[db] = mfma32(__builtin_bit_cast(bf16x8, xv), pa[s], ao[db]);
      }
    }

    // O^T: lane (col, hh) holds dims 32 db + 8 a + 4 hh .. +3 of its own column's output
    // row in ao[db][4a .. 4a+3]
    if (hh == 0) {
      const int64_t pi = ((((int64_t)bh * R + (i - i0)) * K + slot) * G + r);
      px[col] = valid ? pi : -1;
      if (valid) plse[pi] = mx + __builtin_amdgcn_logf(sum);
    }
    // the normalised rows go through this wavefront's LDS staging (8-byte pieces in) so that
    // they leave in 16-byte pieces
    {
      const float inv = valid ? 1.f / sum : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          uint2 o;
          o.x = f2bf_rne(ao[db][4 * a] * inv) | (f2bf_rne(ao[db][4 * a + 1] * inv) << 16);
          o.y = f2bf_rne(ao[db][4 * a + 2] * inv) | (f2bf_rne(ao[db][4 * a + 3] * inv) << 16);
          *reinterpret_cast<uint2*>(os + col * OSR + 32 * db + 8 * a + 4 * hh) = o;
        }
    }
    wave_sync();
#pragma unroll
    for (int t = lane; t < 32 * (D / 8); t += 64) {
      const int m = t / (D / 8), c8 = (t % (D / 8)) * 8;
      const int64_t pi = px[m];
      // streamed out (read back once, by the merge): non-temporal stores keep the key and
      // value tiles and query rows in the caches (256K attention 6.20 -> 5.73 ms)
      if (pi >= 0)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(os + m * OSR + c8),
                                    reinterpret_cast<u32x4*>(po + pi * D + c8));
    }
    wave_sync();  // px and os are rewritten by the next column group
    ent = ent_n;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) bq[s2] = bqn[s2];
  }
}

// The forced blocks {0, b-1, b} of leaf block b, shared by its 64 queries.  Workgroup = a
// run of consecutive leaf blocks of one (b, h), eight wavefronts: key tiles and
// transposed value tiles live in LDS slots, tile 0 in slot 0 for the whole run and tile j >= 1
// in slot 1 + j % 3, so that moving from block b to b + 1 stages one new tile (b + 1), whose
// global loads are issued into registers before block b is computed and written to its slot
// (that of b - 2, no longer read) after it.  Each wavefront takes column groups of 32
// (query, head) columns (the next group's query fragments loaded ahead) and runs an online
// softmax over the block's forced tiles (a tile the query's selection does not name, and
// keys after the query, are masked), with S = K Q^T and O^T = V^T P as in
// attn_chunk_kernel.  Writes one combined partial per (query, head): the output over its
// forced keys normalised by their sum (bf16) and their log2-sum-exp (-inf without such keys).
// Run length: about two workgroups per compute unit (one fits, by LDS), at most 32 blocks
// (256K, runs of 4, 8, 16 and 32 blocks: attention 5.07, 5.02, 5.01 and 4.98 ms).
constexpr int kForcedMaxRun = 32;
inline int forced_run(const Geo& g) {
  const int64_t lists = (int64_t)g.B * g.Hkv * g.n1;
  return (int)std::max<int64_t>(1, std::min<int64_t>(kForcedMaxRun, lists / 512));
}

template <int D>
struct ForcedTile {
  static constexpr int PER = kLeaf * (D / 8) / 512;  // 16-byte pieces per thread and tensor
  u32x4 kx[PER], vx[PER];
  __device__ __forceinline__ void load(const bf16* kb, const bf16* vb, int f, int N) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int t = threadIdx.x + 512 * p;
      const int key = t / (D / 8), d8 = (t % (D / 8)) * 8;
      kx[p] = {0u, 0u, 0u, 0u};
      vx[p] = {0u, 0u, 0u, 0u};
      if (f * kLeaf + key < N) {
        kx[p] = *reinterpret_cast<const u32x4*>(kb + (int64_t)(f * kLeaf + key) * D + d8);
        vx[p] = *reinterpret_cast<const u32x4*>(vb + (int64_t)(f * kLeaf + key) * D + d8);
      }
    }
  }
  __device__ __forceinline__ void store(bf16* kt, bf16* vt) const {
    constexpr int VTR = kLeaf + 8;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int t = threadIdx.x + 512 * p;
      const int key = t / (D / 8), d8 = (t % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&kt[key * (D + 8) + d8]) = kx[p];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vt[(d8 + 2 * w) * VTR + key] = (bf16)(vx[p][w] & 0xFFFFu);
        vt[(d8 + 2 * w + 1) * VTR + key] = (bf16)(vx[p][w] >> 16);
      }
    }
  }
};

__device__ __forceinline__ int forced_slot(int j) { return j == 0 ? 0 : 1 + j % 3; }

template <int D, int G>
__global__ __launch_bounds__(512) void attn_forced_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                          const bf16* __restrict__ v, Geo geo,
                                                          const int32_t* __restrict__ idx, int run, int b0,
                                                          int b1, int i0, int R, float* __restrict__ pfl,
                                                          bf16* __restrict__ pfo) {
  // one query range: leaf blocks [b0, b1) (queries i0 .. i0 + R - 1); the partial of query i
  // of (b, h) sits at row b h * R + (i - i0) of the range's buffers
  static_assert(D % 64 == 0, "ForcedTile spreads a tile over 512 threads in whole pieces");
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int VTR = kLeaf + 8;
  __shared__ __attribute__((aligned(16))) bf16 kt[4][kLeaf * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 vt[4][D * VTR];
  __shared__ uint32_t pres[2][kLeaf];  // bit x: the query's selection names forced block x
  const int nruns = (b1 - b0 + run - 1) / run;
  const int bh = blockIdx.x / nruns;  // one-dimensional grid: B * Hkv may exceed a y extent
  const int N = geo.N, K = geo.K;
  const int b = bh / geo.Hkv, h = bh % geo.Hkv;
  const int bs = b0 + (blockIdx.x % nruns) * run, be = min(bs + run, b1);
  const bf16* kb = k + (int64_t)bh * N * D;
  const bf16* vb = v + (int64_t)bh * N * D;
  auto presence = [&](int bq, uint32_t* dst) {
    if (threadIdx.x < kLeaf) {
      const int i = bq * kLeaf + threadIdx.x;
      uint32_t pm = 0;
      if (i < N) {
        const int32_t* sel = idx + ((int64_t)bh * N + i) * K;
        for (int u = 0; u < K; ++u) {
          const int j = sel[u];
          pm |= (j == 0 ? 1u : 0u) | (bq >= 2 && j == bq - 1 ? 2u : 0u) | (bq >= 1 && j == bq ? 4u : 0u);
        }
      }
      dst[threadIdx.x] = pm;
    }
  };
  {  // the run's first block: tiles 0, bs - 1 and bs
    ForcedTile<D> t;
    t.load(kb, vb, 0, N);
    t.store(kt[0], vt[0]);
    if (bs >= 2) {
      t.load(kb, vb, bs - 1, N);
      t.store(kt[forced_slot(bs - 1)], vt[forced_slot(bs - 1)]);
    }
    if (bs >= 1) {
      t.load(kb, vb, bs, N);
      t.store(kt[forced_slot(bs)], vt[forced_slot(bs)]);
    }
    presence(bs, pres[bs & 1]);
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const float sl = geo.s_log2e;
  // query fragments of column group cg of block bq (zeros past N)
  auto load_q = [&](int bq, int cg, bf16x8* dst) {
    const int gc = cg * 32 + col;
    const int i = bq * kLeaf + gc / G, r = gc % G;
    const bool valid = i < N;
    load_bfrag<D>(q + (((int64_t)b * geo.Hq + h * G + r) * N + (valid ? i : 0)) * D, valid, hh, dst);
  };
  bf16x8 bqf[KS];
  if (wave < 2 * G) load_q(bs, wave, bqf);
  for (int bq = bs; bq < be; ++bq) {
    const bool more = bq + 1 < be;
    ForcedTile<D> nt;
    if (more) {
      nt.load(kb, vb, bq + 1, N);
      presence(bq + 1, pres[(bq + 1) & 1]);
    }
    int F[3];
    const int nf = forced_blocks(bq, F);
    for (int cg = wave; cg < 2 * G; cg += 8) {
      // the next column group of this wavefront, in this block or the next
      const int ncg = cg + 8 < 2 * G ? cg + 8 : wave;
      const int nbq = cg + 8 < 2 * G ? bq : bq + 1;
      bf16x8 bqn[KS];
      if (nbq < be) load_q(nbq, ncg, bqn);
      const int gc = cg * 32 + col;
      const int ql = gc / G, r = gc % G;
      const int i = bq * kLeaf + ql;
      const bool valid = i < N;
      const uint32_t pm = valid ? pres[bq & 1][ql] : 0u;
      float mrun = -INFINITY, lrun = 0.f;
      f32x16 ao[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int w = 0; w < 16; ++w) ao[db][w] = 0.f;
      for (int x = 0; x < nf; ++x) {
        const int f = x == 0 ? F[0] : (x == 1 ? F[1] : F[2]);
        const int fs = forced_slot(f);
        // presence bit of block f: 0 -> bit 0, bq - 1 -> bit 1, bq -> bit 2
        const bool named = (pm >> (f == 0 ? 0 : (f == bq ? 2 : 1))) & 1u;
        f32x16 s0, s1;
        tile_mfma32<D>(kt[fs], bqf, lane, s0, s1);
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
          const int t0 = f * kLeaf + key_row(w, hh), t1 = t0 + 32;
          s0[w] = (named && t0 <= i && t0 < N) ? s0[w] * sl : -INFINITY;
          s1[w] = (named && t1 <= i && t1 < N) ? s1[w] * sl : -INFINITY;
          mx = fmaxf(mx, fmaxf(s0[w], s1[w]));
        }
        mx = xor32_max(mx);
        const float mnew = fmaxf(mrun, mx);
        // running maximum still -inf: every key so far is masked and contributes nothing
        const float base = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - base);
        float sum = 0.f;
        bf16x8 pa[4];
#pragma unroll
        for (int w = 0; w < 16; ++w) {
          const float p0 = __builtin_amdgcn_exp2f(s0[w] - base), p1 = __builtin_amdgcn_exp2f(s1[w] - base);
          sum += p0 + p1;
          pa[w >> 3][w & 7] = (__bf16)p0;
          pa[2 + (w >> 3)][w & 7] = (__bf16)p1;
        }
        sum = xor32_sum(sum);
        lrun = lrun * alpha + sum;
        mrun = mnew;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int w = 0; w < 16; ++w) ao[db][w] *= alpha;
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            const bf16* vr = &vt[fs][(32 * db + col) * VTR + 32 * (s2 >> 1) + 16 * (s2 & 1) + 4 * hh];
            const uint2 x0 = *reinterpret_cast<const uint2*>(vr), x1 = *reinterpret_cast<const uint2*>(vr + 8);
            const u32x4 xv = {x0.x, x0.y, x1.x, x1.y};
            ao[db] = mfma32(__builtin_bit_cast(bf16x8, xv), pa[s2], ao[db]);
          }
        }
      }
      if (valid) {
        const int64_t prow = ((int64_t)bh * R + (i - i0)) * G + r;
        if (hh == 0) pfl[prow] = lrun > 0.f ? mrun + __builtin_amdgcn_logf(lrun) : -INFINITY;
        const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
        bf16* dst = pfo + prow * D + 4 * hh;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            uint2 o;
            o.x = f2bf_rne(ao[db][4 * a] * inv) | (f2bf_rne(ao[db][4 * a + 1] * inv) << 16);
            o.y = f2bf_rne(ao[db][4 * a + 2] * inv) | (f2bf_rne(ao[db][4 * a + 3] * inv) << 16);
            *reinterpret_cast<uint2*>(dst + 32 * db + 8 * a) = o;
          }
      }
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) bqf[s2] = bqn[s2];
    }
    // slot of bq + 1 = slot of bq - 2, read last by the previous block (before the barrier)
    if (more) nt.store(kt[forced_slot(bq + 1)], vt[forced_slot(bq + 1)]);
    __syncthreads();
  }
}

// One wavefront per query group: merges, for each of its G heads, the forced blocks'
// combined partial and the partials of the other selected blocks.  A head's row is D / 8
// lanes x 16 bytes, so one pass covers HP = 64 / (D / 8) heads and each slot's partial rows
// of those heads (contiguous: partials are slot-major, head-minor) come in one 16-byte load
// per lane, the K slots' loads all in flight together.  Lane t < K G first reads the
// log2-sum-exp of partial t (slot t / G, head t % G); each lane then takes its head's
// weights by shuffles.  A slot without a partial (forced, padding, or after the query's
// block) gets weight 0 and is not loaded, so no stale value reaches the sum.
template <int D, int G>
__global__ __launch_bounds__(256) void attn_merge_kernel(const int32_t* __restrict__ idx, Geo geo,
                                                         const float* __restrict__ plse,
                                                         const bf16* __restrict__ po,
                                                         const float* __restrict__ pfl,
                                                         const bf16* __restrict__ pfo, bf16* __restrict__ out,
                                                         float* __restrict__ lse, int i0, int nq, int R) {
  // one query range: queries i0 .. i0 + nq - 1 of every (b, h); their partials sit at rows
  // b h * R + (i - i0) of the range's buffers
  constexpr int LPH = D / 8;       // lanes per head row (16 bytes each)
  constexpr int HP = 64 / LPH;     // heads per pass
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = geo.N, K = geo.K;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= (int64_t)geo.B * geo.Hkv * nq) return;  // whole wavefront; no barrier follows
  const int bh = (int)(w / nq), i = i0 + (int)(w % nq);
  const int64_t row = (int64_t)bh * N + i;       // the selection's row
  const int64_t prow = (int64_t)bh * R + (i - i0);  // the partials' row
  const int b = bh / geo.Hkv, h = bh % geo.Hkv, bq = i / geo.C;
  const int KG = K * G;
  const float* lrow = plse + prow * KG;
  float x0 = -INFINITY, x1 = -INFINITY;
  if (lane < KG) {
    const int jb = idx[row * K + lane / G];
    if (jb >= 0 && jb <= bq && !is_forced(jb, bq)) x0 = lrow[lane];
  }
  if (lane + 64 < KG) {
    const int jb = idx[row * K + (lane + 64) / G];
    if (jb >= 0 && jb <= bq && !is_forced(jb, bq)) x1 = lrow[lane + 64];
  }
  // partial t's log2-sum-exp for this lane (t may differ between lanes)
  auto xat = [&](int t) -> float {
    const float a = __shfl(x0, t & 63), c = __shfl(x1, t & 63);
    if (t < 64) return a;
    if (t < 128) return c;
    const int jb = idx[row * K + t / G];
    return (jb >= 0 && jb <= bq && !is_forced(jb, bq)) ? lrow[t] : -INFINITY;
  };
  const int hl = lane / LPH, dl = (lane % LPH) * 8;  // head within the pass, first dim
#pragma unroll 1
  for (int r0 = 0; r0 < G; r0 += HP) {
    const int r = r0 + hl;
    const bool live = r < G;
    const int rr = live ? r : 0;  // idle lanes shadow head 0 so every lane takes part in the shuffles
    // the forced blocks' combined partial of this head (attn_forced_kernel)
    const float lf = pfl[prow * G + rr];
    const u32x4 fr = *reinterpret_cast<const u32x4*>(pfo + (prow * G + rr) * D + dl);
    float mx = lf;
    for (int u = 0; u < K; ++u) mx = fmaxf(mx, xat(u * G + rr));
    float l = 0.f, acc[8];
    {
      const float wf = lf > -INFINITY ? __builtin_amdgcn_exp2f(lf - mx) : 0.f;
      l = wf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = wf > 0.f ? wf * bf2f(fr[e] & 0xFFFFu) : 0.f;
        acc[2 * e + 1] = wf > 0.f ? wf * bf2f(fr[e] >> 16) : 0.f;
      }
    }
#pragma unroll 8
    for (int u = 0; u < K; ++u) {
      const int t = u * G + rr;
      const float xt = xat(t);
      const float wu = xt > -INFINITY ? __builtin_amdgcn_exp2f(xt - mx) : 0.f;
      l += wu;
      // slots without a partial (forced blocks, padding, blocks after the query's) are not
      // read: the slot's block is the same for every lane, so this is uniform in practice
      u32x4 pr = {0u, 0u, 0u, 0u};
      if (wu > 0.f) pr = *reinterpret_cast<const u32x4*>(po + (prow * KG + t) * D + dl);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf2f(pr[e] & 0xFFFFu), hi = bf2f(pr[e] >> 16);
        acc[2 * e] += wu > 0.f ? wu * lo : 0.f;
        acc[2 * e + 1] += wu > 0.f ? wu * hi : 0.f;
      }
    }
    if (live) {
      const int64_t orow = ((int64_t)b * geo.Hq + h * G + r) * N + i;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = f2bf_rne(acc[2 * e] * inv) | (f2bf_rne(acc[2 * e + 1] * inv) << 16);
      *reinterpret_cast<u32x4*>(out + orow * D + dl) = o;
      if (lse && lane % LPH == 0)
        lse[orow] = l > 0.f ? (mx + __builtin_amdgcn_logf(l)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

template <int D, int G>
int attn_km_g(const Geo& g, const bf16* q, const bf16* k, const bf16* v, const int32_t* idx, const AttnWs& w,
              char* ws, bf16* out, float* lse, hipStream_t st) {
  int32_t* cand = (int32_t*)(ws + w.cand);
  int32_t* cnt = (int32_t*)(ws + w.cnt);
  int32_t* cursor = (int32_t*)(ws + w.cursor);
  int32_t* off = (int32_t*)(ws + w.off);
  int32_t* choff = (int32_t*)(ws + w.choff);
  int32_t* entries = (int32_t*)(ws + w.entries);
  float* plse = (float*)(ws + w.plse);
  bf16* po = (bf16*)(ws + w.po);
  float* pfl = (float*)(ws + w.pfl);
  bf16* pfo = (bf16*)(ws + w.pfo);
  const int BH = g.B * g.Hkv, R = w.R;
  int rc;
  if ((rc = launch_zero(cnt, (int64_t)(w.off - w.cnt) / (int64_t)sizeof(int32_t), st)) != PISA_OK) return rc;
  const unsigned cgrid = (unsigned)(BH * ((g.N + kLeafQueries - 1) / kLeafQueries));
  const size_t hbytes = g.n1 <= kHistMaxBins ? sizeof(int) * (size_t)g.n1 : 0;
  attn_cand_kernel<<<cgrid, 256, hbytes, st>>>(idx, g, R, cand, cnt);
  if (hipGetLastError() != hipSuccess) return PISA_ERR_HIP;
  const int qc = 4 * kAttnColGroups * 32 / G;  // pairs per chunk
  if ((rc = launch_scan(cnt, w.M, qc, off, choff, st)) != PISA_OK) return rc;
  if ((rc = launch_scatter(g, g.K, R, cand, off, cursor, entries, st)) != PISA_OK) return rc;
  const int run = forced_run(g);
  // one pass per query range (one in all with the full workspace): the chunk kernel writes
  // the range's pair partials, the forced kernel its forced partials, the merge its output
  for (int i0 = 0; i0 < g.N; i0 += R) {
    const int i1 = std::min(g.N, i0 + R), nq = i1 - i0;
    const int32_t Mlo = (i0 / R) * BH * g.n1, Mhi = Mlo + BH * g.n1;
    // chunks of the range: at most its pairs / qc plus one per list that can be non-empty
    // (blocks up to the range's last query)
    const int64_t lists = (int64_t)BH * std::min(g.n1, (i1 - 1) / kLeaf + 1);
    const int64_t grid = ((int64_t)BH * nq * g.K + qc - 1) / qc + lists;
    attn_chunk_kernel<D, G><<<(unsigned)grid, 256, 0, st>>>(q, k, v, g, off, choff, entries, Mlo, Mhi, i0, R, plse,
                                                            po);
    if (hipGetLastError() != hipSuccess) return PISA_ERR_HIP;
    const int b0 = i0 / kLeaf, b1 = std::min(g.n1, (i1 + kLeaf - 1) / kLeaf);
    const unsigned fgrid = (unsigned)(((b1 - b0 + run - 1) / run) * (int64_t)BH);
    attn_forced_kernel<D, G><<<fgrid, 512, 0, st>>>(q, k, v, g, idx, run, b0, b1, i0, R, pfl, pfo);
    if (hipGetLastError() != hipSuccess) return PISA_ERR_HIP;
    const int64_t rows = (int64_t)BH * nq;
    attn_merge_kernel<D, G><<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(idx, g, plse, po, pfl, pfo, out, lse, i0, nq,
                                                                          R);
    if (hipGetLastError() != hipSuccess) return PISA_ERR_HIP;
  }
  return PISA_OK;
}

template <int D>
int attn_km_d(const Geo& g, const void* q, const void* k, const void* v, const int32_t* idx, void* ws,
              int32_t R, void* out, float* lse, hipStream_t st) {
  const AttnWs w = attention_ws(g, R);
  const bf16 *qq = (const bf16*)q, *kk = (const bf16*)k, *vv = (const bf16*)v;
  bf16* oo = (bf16*)out;
  char* wc = (char*)ws;
  switch (g.G) {
    case 1: return attn_km_g<D, 1>(g, qq, kk, vv, idx, w, wc, oo, lse, st);
    case 2: return attn_km_g<D, 2>(g, qq, kk, vv, idx, w, wc, oo, lse, st);
    case 4: return attn_km_g<D, 4>(g, qq, kk, vv, idx, w, wc, oo, lse, st);
    case 8: return attn_km_g<D, 8>(g, qq, kk, vv, idx, w, wc, oo, lse, st);
    case 16: return attn_km_g<D, 16>(g, qq, kk, vv, idx, w, wc, oo, lse, st);
    default: return PISA_ERR_UNSUPPORTED;
  }
}

}  // namespace

bool attention_key_major(const Geo& g, int dtype, int decode) { return dtype == PISA_BF16 && !decode; }

AttnWs attention_ws(const Geo& g, int32_t R) {
  AttnWs w;
  auto align256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t BH = (int64_t)g.B * g.Hkv;
  w.R = R;
  w.slots = BH * g.N * g.K;
  const int64_t M = ((g.N + R - 1) / R) * BH * g.n1;
  if (R <= 0 || M >= (int64_t)1 << 30) {  // list indices must stay int32: too many ranges
    w.M = 0;
    w.total = SIZE_MAX;
    return w;
  }
  w.M = (int32_t)M;
  size_t o = 0;
  w.cand = o;    o = align256(o + sizeof(int32_t) * w.slots);
  w.cnt = o;     o = align256(o + sizeof(int32_t) * w.M);
  w.cursor = o;  o = align256(o + sizeof(int32_t) * w.M);
  w.off = o;     o = align256(o + sizeof(int32_t) * (w.M + 1));
  w.choff = o;   o = align256(o + sizeof(int32_t) * (w.M + 1));
  w.entries = o; o = align256(o + sizeof(int32_t) * w.slots);
  const size_t rows = (size_t)BH * R;  // one range's (b h, query) rows
  w.plse = o;    o = align256(o + sizeof(float) * rows * g.K * g.G);
  w.po = o;      o = align256(o + sizeof(uint16_t) * rows * g.K * g.G * g.d);
  w.pfl = o;     o = align256(o + sizeof(float) * rows * g.G);
  w.pfo = o;     o = align256(o + sizeof(uint16_t) * rows * g.G * g.d);
  w.total = o;
  return w;
}

int32_t attention_full_range(const Geo& g) {
  return (int32_t)(((int64_t)g.N + kLeafQueries - 1) / kLeafQueries * kLeafQueries);
}

int32_t attention_range(const Geo& g, size_t bytes) {
  int lo = 0, hi = attention_full_range(g) / kLeafQueries;  // largest m with total(m * kLeafQueries) <= bytes
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (attention_ws(g, mid * kLeafQueries).total <= bytes) lo = mid; else hi = mid - 1;
  }
  return lo * kLeafQueries;
}

int launch_attention(const Geo& g, int dtype, const void* q, const void* k, const void* v, const int32_t* idx,
                     int decode, void* ws, size_t ws_bytes, void* out, float* lse, hipStream_t st) {
  if (attention_key_major(g, dtype, decode)) {
    const int32_t R = attention_range(g, ws_bytes);  // as many queries per pass as the workspace holds
    if (R <= 0) return PISA_ERR_WORKSPACE;
    if (g.d == 128) return attn_km_d<128>(g, q, k, v, idx, ws, R, out, lse, st);
    if (g.d == 64) return attn_km_d<64>(g, q, k, v, idx, ws, R, out, lse, st);
    return PISA_ERR_UNSUPPORTED;
  }
  if (dtype == PISA_BF16) {
    if (g.d == 128) return attn_g<bf16, 128>(g, q, k, v, idx, decode, out, lse, st);
    if (g.d == 64) return attn_g<bf16, 64>(g, q, k, v, idx, decode, out, lse, st);
  } else {
    if (g.d == 128) return attn_g<float, 128>(g, q, k, v, idx, decode, out, lse, st);
    if (g.d == 64) return attn_g<float, 64>(g, q, k, v, idx, decode, out, lse, st);
  }
  return PISA_ERR_UNSUPPORTED;
}

}  // namespace pisa
