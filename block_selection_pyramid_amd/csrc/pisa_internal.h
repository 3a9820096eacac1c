// Internal declarations of libpisa: problem geometry, workspace layout, kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pisa.h"

namespace pisa {

constexpr int kMaxLevels = PISA_MAX_LEVELS;
constexpr int kWave = 64;
constexpr int kLeaf = 64;     // C supported by the kernels
constexpr int kMaxCand = 64;  // g*K <= 64 candidates per level (one per lane)

// Geometry of one problem, passed by value to every kernel.
struct Geo {
  int32_t B, Hq, Hkv, G, N, d, C, K, g, L, n1, T;
  int32_t Tp;      // node stride of one (b, h) pyramid in the buffer: T rounded up to a multiple of 4
  int32_t n1p;     // ceil(n1 / 2): level-2 nodes as leaf-block pairs (g = 2), one prefill leaf list each
  int32_t scorer;  // enum pisa_scorer of the routing levels
  float s;        // scale applied to every dot product
  float s_log2e;  // s * log2(e), for exp2-based LSE
  int32_t n[kMaxLevels + 2];    // n[0] = N, n[l] nodes at level l (1..L)
  int32_t off[kMaxLevels + 2];  // node offset of level l in one (b, h) pyramid

  // floats of fp32 means before the routing copy in the pyramid buffer
  __host__ __device__ int64_t means_floats() const { return (int64_t)B * Hkv * Tp * d; }
};

// Prefill workspace carve-up (byte offsets, 256-aligned).  qg: the queries regrouped by
// (b, KV head, position) with the G heads of each 8-dim piece adjacent, written by the dense
// routing launch (bf16 with L >= 3) for the gather and leaf launches; total includes it,
// total_min does not (a workspace of at least total_min but less than total runs without
// the copy, reading q itself).
struct PrefillWs {
  size_t cand, lscore, cnt, cursor, off, choff, entries, fsc, lo8, qg, total_min, total;
  int64_t slots;  // B*Hkv*N*2K
  int32_t M;      // B*Hkv*n1p leaf-pair lists
};

int make_geo(const pisa_problem* p, Geo* g);  // PISA_OK or PISA_ERR_INVALID_ARG
int supported(const Geo& g, int dtype, int mode);
PrefillWs prefill_ws(const Geo& g, int dtype);
// Leaf-pair entries (query groups) per chunk of the prefill leaf kernel: four wavefronts,
// kLeafColGroups column groups of 32 (query, head) columns each (256K prefill: 2, 4, 8, 16
// and 32 groups took 2.45, 2.02, 1.82, 1.73 and ~1.69 ms).
constexpr int kLeafColGroups = 32;
inline int chunk_entries(int G) { return 4 * kLeafColGroups * 32 / G; }
// Queries per workgroup of block-sparse attention's candidate pass and scatter, and the
// most the leaf-pair count and scatter take (group_queries); the histograms of those passes
// and of the gather routing launch live in LDS while they have at most kHistMaxBins bins
// (leaf blocks or level-2 nodes).
constexpr int kLeafQueries = 2048;
constexpr int kHistMaxBins = 8192;
// Queries per workgroup of the leaf-pair count and scatter: kLeafQueries, halved (down to
// 64) while that leaves fewer than 1024 workgroups, so small problems fill the chip.
inline int group_queries(const Geo& g) {
  int qpw = kLeafQueries;
  while (qpw > 64 && (int64_t)g.B * g.Hkv * ((g.N + qpw - 1) / qpw) < 1024) qpw >>= 1;
  return qpw;
}
// Query groups one routing wavefront walks together: 2K candidate slots each within 64
// lanes, one MFMA column per (group, head) within 16.
inline int route_groups_per_wave(int G, int K) {
  int gpw = 4;
  while (gpw > 1 && (64 / gpw < 2 * K || G * gpw > 16)) gpw >>= 1;
  return gpw;
}

// ---- launchers (each returns PISA_OK or PISA_ERR_HIP) ----
int launch_build_pyramid(const Geo& g, int dtype, const void* k, float* pyr, hipStream_t st);
// block-sparse attention over selected blocks (decode != 0: one query per sequence at N-1);
// bf16 prefill runs key-major in passes over query ranges of R queries (R a multiple of
// kLeafQueries) and needs the workspace laid out by attention_ws(g, R)
struct AttnWs {
  size_t cand, cnt, cursor, off, choff, entries, plse, po, pfl, pfo, total;
  int64_t slots;  // B*Hkv*N*K
  int32_t M;      // ceil(N / R) * B*Hkv*n1 block lists, numbered (range, b h, block)
  int32_t R;      // queries per range
};
bool attention_key_major(const Geo& g, int dtype, int decode);
AttnWs attention_ws(const Geo& g, int32_t R);
int32_t attention_full_range(const Geo& g);           // one range: N rounded up to kLeafQueries
int32_t attention_range(const Geo& g, size_t bytes);  // largest R whose workspace fits, 0 if none
int launch_attention(const Geo& g, int dtype, const void* q, const void* k, const void* v, const int32_t* idx,
                     int decode, void* ws, size_t ws_bytes, void* out, float* lse, hipStream_t st);
// full-scan BSA selection (bf16): out_idx / out_score [B, Hkv, N, K]
int launch_bsa(const Geo& g, const void* q, const float* pyr, int32_t* out_idx, float* out_score, hipStream_t st);
int launch_zero(int32_t* a, int64_t n, hipStream_t st);
// x2: scratch of B*Hkv*N*2K int32 (level-2 candidates between the two routing launches);
// fsc: forced-block scores, written when route_scores_forced(); mid (may be null) is
// recorded between the upper-level and the level-2 launch
// qg (may be null): the regrouped query copy, written by the dense launch and read by the
// gather launch
// lo8: workspace of lo8_bytes(g) for the level-2 launch's fp8 leaf corrections (d = 128)
int launch_route(const Geo& g, int dtype, const void* q, const void* k, const float* pyr, int32_t* x2,
                 float* fsc, int32_t* cand, int32_t* cnt, void* qg, uint8_t* lo8, hipEvent_t mid, hipStream_t st);
// Levels L..dense_bottom(g) of the bf16 walk (L >= 3), scored densely per leaf block; writes x2 and the
// forced blocks' scores fsc [B*Hkv*N*3] (ascending forced-block order).
int launch_route_upper_dense(const Geo& g, const void* q, const float* pyr, const void* k, int32_t* x2, float* fsc,
                              void* qg, hipStream_t st);
// true when launch_route scores the forced blocks (into fsc) for this problem
inline bool route_scores_forced(const Geo& g, int dtype) { return dtype == PISA_BF16 && g.L >= 3; }
// Dense scoring pays while a level is small: its cost per query grows with the visible
// prefix of the child level, a gather's does not.  The dense launch covers levels L down
// to dense_bottom(g), the highest routing levels whose child level has at most
// kDenseMaxChildren nodes (n[L-1] <= 2gK always qualifies, so L >= 3 implies a dense
// launch); the gather launch walks the levels below, down to 2.  Measured at 256K-1M
// tokens: a level over 2048 children costs a little more dense than gathered, one over
// 1024 children clearly less (the dense cost halves with each level up, a gathered
// level's stays the same).  With at most kDenseMaxChildren leaf blocks level 2 is dense
// too (dense_bottom == 2): the dense launch then writes the leaf candidates itself, a
// counting pass builds the leaf-pair histogram and the gather launch is skipped.
constexpr int kDenseMaxChildren = 1024;
inline int dense_bottom(const Geo& g) {
  int l = 2;
  while (l < g.L && g.n[l - 1] > kDenseMaxChildren) ++l;
  return l;
}
// The gather levels in one launch from leaf-block means (G = 4, gather levels l_x .. 2 with
// l_x = 3 or 2; x2 holds the level-l_x candidates); writes cand and histograms into cnt
// like the gather walk.
bool route_sub_supported(const Geo& g, int l_x);
int launch_route_sub(const Geo& g, int l_x, const void* q, const float* pyr, const int32_t* x2, int32_t* cand,
                     int32_t* cnt, const void* qg, uint8_t* lo8, hipStream_t st);
// Level-1 fp8 corrections that the level-2 launch reads in place of the routing copy's lo
// halves (d = 128): per (b, KV head) n1 rounded up to 4 leaf records of 128 e4m3 bytes,
// then one E8M0 scale byte per leaf (workspace bytes, 0 for other d).
inline size_t lo8_bytes(const Geo& g) {
  return g.d == 128 ? (size_t)g.B * g.Hkv * (size_t)((g.n1 + 3) & ~3) * (g.d + 1) : 0;
}
int launch_scan(const int32_t* cnt, int32_t M, int32_t qc, int32_t* off, int32_t* choff, hipStream_t st);
// histogram of the routed (query group, level-2 node) pairs of the 2K leaf slots per query
// group into cnt [B*Hkv*n1p] (the counts the gather launch keeps when it runs)
int launch_count_pairs(const Geo& g, const int32_t* cand, int32_t* cnt, hipStream_t st);
// scatter of per_row candidate slots per query group (-1 = none) into per-leaf-block lists
// (block-sparse attention's (query group, block) pairs)
int launch_scatter(const Geo& g, int per_row, int32_t R, const int32_t* cand, const int32_t* off, int32_t* cursor,
                   int32_t* entries, hipStream_t st);
// scatter of the 2K routed leaf slots per query group into per-level-2-node lists: slots 2r
// and 2r+1 (children of the kept node of rank r) give one entry (i << 6 | r) when either
// holds a block
int launch_scatter_pairs(const Geo& g, const int32_t* cand, const int32_t* off, int32_t* cursor, int32_t* entries,
                         hipStream_t st);
int launch_leaf_mfma(const Geo& g, const void* q, const void* k, const void* qg, const int32_t* off,
                     const int32_t* choff, const int32_t* entries, int32_t M, float* lscore, hipStream_t st);
int launch_final(const Geo& g, const int32_t* cand, const float* lscore, const float* fsc, int32_t* out_idx,
                 float* out_score, hipStream_t st);
int launch_forced_final(const Geo& g, const void* q, const void* k, const int32_t* cand, const float* lscore,
                        int32_t* out_idx, float* out_score, hipStream_t st);
int launch_qmajor(const Geo& g, int dtype, const void* q, const void* k, const int32_t* cand, int32_t* out_idx,
                  float* out_score, hipStream_t st);
// lengths: nullptr (every sequence holds g.N keys) or device int32 [B] per-sequence lengths
// in a cache of capacity g.N (pyramid in the capacity layout)
int launch_decode(const Geo& g, int dtype, const void* q, const void* k, const float* pyr, const int32_t* lengths,
                  int32_t* out_idx, float* out_score, hipStream_t st);
// incremental pyramid update of sequences growing from old_len[b] to new_len[b] keys
// (capacity geometry g; at most max_new keys per sequence)
int launch_append(const Geo& g, int dtype, const void* k, const int32_t* old_len, const int32_t* new_len,
                  int max_new, float* pyr, hipStream_t st);

}  // namespace pisa
