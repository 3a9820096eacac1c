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

}  // namespace

int launch_attention(const Geo& g, int dtype, const void* q, const void* k, const void* v, const int32_t* idx,
                     int decode, void* out, float* lse, hipStream_t st) {
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
