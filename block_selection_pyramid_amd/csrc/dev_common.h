// Device helpers shared by the libpisa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pisa_internal.h"

namespace pisa {

using bf16 = uint16_t;  // raw bfloat16 bits

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
// 16 raw bytes as a native vector (HIP's uint4 struct can keep arrays of it in scratch)
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Routing copy of the pyramid: for every node v = fp32(s log2(e) P) split into hi = bf16(v)
// and lo = bf16(v - hi), so that a dot product with a query row is the scaled score in log2
// units.  It follows the fp32 means in the pyramid buffer.  Layout: the nodes of one (b, h)
// (node stride a multiple of 4) form aligned quads 4Q .. 4Q+3, each a record of 8*D bf16;
// for every two 8-dim pieces 2j, 2j+1 (dims 16j .. 16j+15) the record holds a 128-byte hi
// line [piece 2j of nodes 4Q .. 4Q+3 | piece 2j+1 of nodes 4Q .. 4Q+3] (16 bytes per node
// and piece), then the lo line laid out alike.  The matrix cores' operand layout puts
// consecutive nodes on consecutive lanes that each take 16 bytes of one piece, so every
// four consecutive lanes read 64 contiguous bytes and the lanes of two adjacent pieces fill
// whole lines: an L1 pays per line per group of four lanes (L2-resident gathers on this
// chip, this layout's operand loads: 34 TB/s; four lanes on four lines: 9.7).
// rc_node: bf16 offset of node n's hi piece 0; piece p's hi at + 128 (p >> 1) + 32 (p & 1),
// its lo 64 bf16 further.
__host__ __device__ __forceinline__ int64_t rc_node(int64_t n, int D) { return (n >> 2) * 8 * D + (n & 3) * 8; }
__host__ __device__ __forceinline__ int64_t rc_piece(int p) { return 128 * (p >> 1) + 32 * (p & 1); }
__host__ __device__ __forceinline__ int64_t rcopy_index(int64_t node, int e, int D) {
  return rc_node(node, D) + rc_piece(e >> 3) + (e & 7);
}
// Byte offset of 16-byte piece c of node n in the order of a node-contiguous record (the
// layout staged in LDS): d/32 chunks of [hi(32 dims) | lo(32 dims)], 8 pieces each.
__host__ __device__ __forceinline__ int64_t rc_piece_bytes(int64_t n, int c, int D) {
  const int p = 4 * (c >> 3) + (c & 3);  // 8-dim piece
  return 2 * (rc_node(n, D) + rc_piece(p) + 64 * ((c >> 2) & 1));
}
template <int D>
__device__ __forceinline__ void store_rcopy(bf16* R, int64_t node, int e, float v) {
  const uint32_t hi = f2bf_rne(v);
  const float rest = v - bf2f(hi);
  const int64_t i = rcopy_index(node, e, D);
  R[i] = (bf16)hi;
  R[i + 64] = (bf16)f2bf_rne(rest);
}

// Load 16 bytes of input starting at element e of row r and widen to float.
// bf16: 8 elements, fp32: 4 elements.
template <typename T>
struct Vec;
template <>
struct Vec<bf16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void load(const bf16* p, float* out) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    out[0] = bf2f(u.x & 0xFFFFu); out[1] = bf2f(u.x >> 16);
    out[2] = bf2f(u.y & 0xFFFFu); out[3] = bf2f(u.y >> 16);
    out[4] = bf2f(u.z & 0xFFFFu); out[5] = bf2f(u.z >> 16);
    out[6] = bf2f(u.w & 0xFFFFu); out[7] = bf2f(u.w >> 16);
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const float* p, float* out) {
    float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
};

// Orders LDS traffic among the lanes of one wavefront.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// max(a, b, c) in one v_max3_f32.  fmaxf chains become max3 only where the compiler can
// prove its inputs canonical; values that come from v_med3_f32 of raw matrix-core results
// are not, so it would emit a v_max_f32 per pair instead.  Operands are VALU results (no
// matrix-core read hazard to cover).
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// v combined with lane l ^ 32's v, in every lane: v_permlane32_swap exchanges the two
// halves of the wavefront between two copies of v, so each lane then holds both values in
// registers (no LDS crossbar round trip, unlike a shuffle).
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same across lane bit 4 (lane l ^ 16): v_permlane16_swap exchanges the odd 16-lane
// rows of one copy with the even rows of the other.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over each aligned group of G consecutive lanes (G = 1, 2, 4, 8, 16), result in every
// lane of the group.  DPP lane moves within rows of 16 (quad permutes, then the half-row
// and row mirrors, which pair each lane with one of the other half once the halves hold
// equal sums), so no LDS crossbar traffic.
template <int DPP>
__device__ __forceinline__ float dpp_move(float v) {
  // every lane reads a lane of its own row, so bound_ctrl never applies; setting it lets
  // the compiler fold the move into the consuming add or multiply
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), DPP, 0xF, 0xF, true));
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group of 1..16 lanes");
  if constexpr (G >= 2) v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v += dpp_move<0x141>(v);  // row_half_mirror
  if constexpr (G >= 16) v += dpp_move<0x140>(v); // row_mirror
  return v;
}

template <int G>
__device__ __forceinline__ float group_prod(float v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group of 1..16 lanes");
  if constexpr (G >= 2) v *= dpp_move<0xB1>(v);
  if constexpr (G >= 4) v *= dpp_move<0x4E>(v);
  if constexpr (G >= 8) v *= dpp_move<0x141>(v);
  if constexpr (G >= 16) v *= dpp_move<0x140>(v);
  return v;
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

// The largest list l in [lo, hi) whose first chunk choff[l] is <= c, given choff[lo] <= c <
// choff[hi] (choff non-decreasing: empty lists repeat an offset).  A 64-way search: every
// lane of the wavefront probes one offset per round, so 8192 lists take three rounds of
// loads instead of thirteen dependent ones.  Uniform across the wavefront.
__device__ __forceinline__ int find_chunk_list(const int32_t* __restrict__ choff, int lo, int hi, int c, int lane) {
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) >> 6;
    const int idx = lo + step * lane;
    const bool ok = lane == 0 || (idx < hi && choff[idx] <= c);  // a prefix of the lanes
    const unsigned long long bal = __ballot(ok);
    const int t = 63 - __clzll(bal);
    lo += step * t;
    hi = min(hi, lo + step);
  }
  return lo;
}

// Sum (or product) of NV values per lane over the G lanes of a query group, scattered:
// afterwards lane r of the group holds the results for values (r % GE) VPL .. + VPL - 1 in
// v[0 .. VPL), GE = min(G, NV), VPL = NV / GE.  The exchanges run from the highest lane bit
// down: while the group spans more lanes than there are values left to split, both partners
// combine everything; below that each step sends the half of the values the partner keeps
// and combines the half it keeps, so a value crosses lanes once per step, not once per step
// per result.  The partner of lane bit b (quad_perm for bits 0 and 1, half-row and row
// mirrors for bits 2 and 3) agrees with the lane on every higher bit, so both hold the same
// sub-range of values when they exchange.
template <int CTRL, bool PROD>
__device__ __forceinline__ float dpp_combine(float keep, float send) {
  return PROD ? keep * dpp_move<CTRL>(send) : keep + dpp_move<CTRL>(send);
}
template <int G, int NV, bool PROD>
__device__ __forceinline__ void group_reduce_scatter(float (&v)[NV], int r) {
  constexpr int LG = ilog2(G), H = LG < ilog2(NV) ? LG : ilog2(NV);
  static_assert((1 << LG) == G && (1 << ilog2(NV)) == NV, "powers of two");
  auto step = [&](auto bitc) {
    constexpr int b = decltype(bitc)::value;
    constexpr int CTRL = b == 0 ? 0xB1 : b == 1 ? 0x4E : b == 2 ? 0x141 : 0x140;
    if constexpr (b >= H) {
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = dpp_combine<CTRL, PROD>(v[i], v[i]);
    } else {
      constexpr int n = NV >> (H - 1 - b);  // values still held
      const bool up = (r >> b) & 1;
#pragma unroll
      for (int i = 0; i < n / 2; ++i) {
        const float lo = v[i], hi = v[i + n / 2];
        v[i] = dpp_combine<CTRL, PROD>(up ? hi : lo, up ? lo : hi);
      }
    }
  };
  if constexpr (LG > 3) step(std::integral_constant<int, 3>{});
  if constexpr (LG > 2) step(std::integral_constant<int, 2>{});
  if constexpr (LG > 1) step(std::integral_constant<int, 1>{});
  if constexpr (LG > 0) step(std::integral_constant<int, 0>{});
}

// Forced leaf blocks of a query in leaf block bq: {0, bq-1, bq} that exist, ascending.
// (Constant indices only, so the array stays in registers.)
__device__ __forceinline__ int forced_blocks(int bq, int* f) {
  f[0] = 0;
  f[1] = bq >= 2 ? bq - 1 : bq;  // bq = 1: {0, 1}
  f[2] = bq;                      // bq >= 2: {0, bq - 1, bq}
  return bq == 0 ? 1 : (bq == 1 ? 2 : 3);
}
// Routing score of one head for a node with the scaled dots y0 (first child, visible) and
// y1 (second child, -inf when missing or not visible) under the PISA-1 / PISA-2 truncations
// of the pair LSE about the children's mean ("Block Sparse Attention with Log-Linear
// Complexity": agihunt.info summary, LSE paragraph; rcap.io explainer, scoring-rule
// paragraph): log m + mean, plus half the population variance for PISA-2.  With two
// children the variance is (y0 - y1)^2 / 4.  `one` is log(2) in the dots' units and c2 the
// coefficient of (y0 - y1)^2: 0 for PISA-1, 1/8 in natural units, ln(2)/8 in log2 units
// (where a natural-units quantity v reads v / ln 2, so the variance term scales by ln 2).
__device__ __forceinline__ float pair_trunc(float y0, float y1, float one, float c2) {
  const float d = y0 - y1;
  const float v = fmaf(c2 * d, d, one + 0.5f * (y0 + y1));
  return y1 == -INFINITY ? y0 : v;
}
// c2 of pair_trunc for the scorer, in log2 (log2 = true) or natural units.
__host__ __device__ __forceinline__ float trunc_c2(int scorer, bool log2) {
  return scorer == PISA_PISA2 ? (log2 ? 0.6931471805599453f / 8.f : 0.125f) : 0.f;
}

__device__ __forceinline__ bool is_forced(int j, int bq) { return j == 0 || j == bq || j == bq - 1; }

}  // namespace pisa
