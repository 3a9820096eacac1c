// Staging of pyramid tiles for the dense matrix-core kernels (upper-level routing and the
// full-scan BSA selector): 32 consecutive nodes of one level, hi and lo halves of the
// routing copy, moved through registers into fragment-major LDS so that every MFMA
// A-operand read is one conflict-free 16-byte row per lane.  The B operand holds 32
// (query, head) columns per column group, head fastest.
#pragma once

#include "dev_common.h"

namespace pisa {

constexpr int kDenseWaves = 4;

// Columns of the B operand: 32 (query, head) pairs per column group, head fastest.
template <int G>
struct DenseShape {
  static constexpr int NCG = (G <= 2) ? 1 : 2;  // column groups per wavefront
  static constexpr int QPW = 32 * NCG / G;      // queries per wavefront
};

// Staging of child tile t of level l - 1 (children 32t .. 32t+31) into fragment-major LDS:
// fragment f = 2 ks + hi/lo, lane slot = child (lane & 31) and dims 8 (lane >> 5) .. of
// k-step ks, so every MFMA A-operand read is one conflict-free 16-byte row per lane.  The
// wavefronts of the workgroup take fragments wave, wave + 4, ...  A fragment's lane reads
// 8-dim piece 2 ks + (lane >> 5) of its child, so each four consecutive lanes read one node
// quad's 64 contiguous bytes of the routing copy and the two halves of the lanes fill the
// k-step's hi (or lo) lines.
template <int D, int NU>
__device__ __forceinline__ void dense_load_tile(const char* Rb, const Geo& geo, int l, int t, int wave, int lane,
                                                u32x4 (&stg)[NU]) {
  const int node = geo.off[l - 1] + min(32 * t + (lane & 31), geo.n[l - 1] - 1);  // a missing child reads a real node
  // fragment wave + 4 u: k-step 2 u + (wave >> 1), hi / lo = wave & 1
  const char* base = Rb + 2 * rc_node(node, D) + 64 * (lane >> 5) + 256 * (wave >> 1) + 128 * (wave & 1);
#pragma unroll
  for (int u = 0; u < NU; ++u) stg[u] = *reinterpret_cast<const u32x4*>(base + 512 * u);
}
// The same tile straight into LDS buffer buf (global_load_lds_dwordx4: each lane's 16 bytes
// land at the wavefront-uniform fragment base + 16 lane, which is the fragment-major slot),
// so no registers hold the tile in flight.  Completion is counted by vmcnt: wait for
// vmcnt(0) (dense_fetch_wait) before the barrier that publishes the buffer.
template <int D>
__device__ __forceinline__ void dense_fetch_tile(const char* Rb, const Geo& geo, int l, int t, int wave, int lane,
                                                 char* lds, int buf) {
  constexpr int NU = 2 * (D / 16) / kDenseWaves, TILE = 2 * (D / 16) * 1024;
  const int node = geo.off[l - 1] + min(32 * t + (lane & 31), geo.n[l - 1] - 1);
  const char* base = Rb + 2 * rc_node(node, D) + 64 * (lane >> 5) + 256 * (wave >> 1) + 128 * (wave & 1);
#pragma unroll
  for (int u = 0; u < NU; ++u)
    __builtin_amdgcn_global_load_lds(base + 512 * u,
                                     (__attribute__((address_space(3))) void*)(lds + buf * TILE + (wave + kDenseWaves * u) * 1024),
                                     16, 0, 0);
}
__device__ __forceinline__ void dense_fetch_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
template <int D, int NU>
__device__ __forceinline__ void dense_store_tile(char* lds, int buf, int wave, int lane, const u32x4 (&stg)[NU]) {
  constexpr int TILE = 2 * (D / 16) * 1024;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int f = wave + kDenseWaves * u;
    *reinterpret_cast<u32x4*>(lds + buf * TILE + (f * 64 + lane) * 16) = stg[u];
  }
}

// B operand of the queries iw .. iw + QPW - 1 of (b, h): lane column j = lane & 31 of
// column group cg <-> (query iw + cg * 32/G + j / G, head h*G + j % G), dims 16 ks +
// 8 (lane >> 5) .. +8 of k-step ks; zeros for queries past N.  bqc[cg] is the leaf
// block of the lane's query (clamped to the last query).
template <int D, int G, int NCG>
__device__ __forceinline__ void load_query_cols(const bf16* q, const Geo& geo, int b, int h, int iw, int lane,
                                                bf16x8 (&qf)[NCG][D / 16], int (&bqc)[NCG]) {
  constexpr int KS = D / 16;
  const int j = lane & 31, hh = lane >> 5, N = geo.N;
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int i = iw + cg * (32 / G) + j / G;
    bqc[cg] = min(i, N - 1) / kLeaf;  // C = kLeaf
    if (i < N) {
      const bf16* p = q + (((int64_t)b * geo.Hq + h * G + j % G) * N + i) * D + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[cg][ks] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p + 16 * ks));
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[cg][ks][e] = (__bf16)0.f;
    }
  }
}

}  // namespace pisa
