// libpisa C ABI: argument validation, geometry and workspace layout, kernel orchestration.
// Every check runs on the host before the first HIP call; no call allocates memory or
// synchronises the stream.
#include <math.h>
#include <string.h>

#include <mutex>
#include <new>

#include "pisa_internal.h"

namespace pisa {

int make_geo(const pisa_problem* p, Geo* g) {
  if (!p || !g) return PISA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->seq_len < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1) return PISA_ERR_INVALID_ARG;
  if (p->n_q_heads % p->n_kv_heads) return PISA_ERR_INVALID_ARG;
  if (p->head_dim < 1 || p->block < 1 || p->top_k < 3 || p->branch < 2) return PISA_ERR_INVALID_ARG;
  if (p->dtype != PISA_F32 && p->dtype != PISA_BF16) return PISA_ERR_INVALID_ARG;
  if (p->scorer != PISA_LSE && p->scorer != PISA_PISA1 && p->scorer != PISA_PISA2) return PISA_ERR_INVALID_ARG;
  if (!isfinite(p->scale)) return PISA_ERR_INVALID_ARG;
  if ((int64_t)p->top_k * p->branch > (1 << 20)) return PISA_ERR_INVALID_ARG;
  memset(g, 0, sizeof(*g));
  g->B = p->batch;
  g->Hq = p->n_q_heads;
  g->Hkv = p->n_kv_heads;
  g->G = p->n_q_heads / p->n_kv_heads;
  g->N = p->seq_len;
  g->d = p->head_dim;
  g->C = p->block;
  g->K = p->top_k;
  g->g = p->branch;
  g->scorer = p->scorer;
  g->s = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  g->s_log2e = g->s * 1.4426950408889634f;
  int64_t n = ((int64_t)g->N + g->C - 1) / g->C;
  g->n[0] = g->N;
  g->n[1] = (int32_t)n;
  int L = 1;
  while (n > (int64_t)g->g * g->K) {
    if (L + 1 > kMaxLevels) return PISA_ERR_INVALID_ARG;
    n = (n + g->g - 1) / g->g;
    g->n[++L] = (int32_t)n;
  }
  g->L = L;
  g->n1 = g->n[1];
  g->n1p = (g->n1 + 1) / 2;
  int64_t off = 0;
  for (int l = 1; l <= L; ++l) {
    g->off[l] = (int32_t)off;
    off += g->n[l];
  }
  g->off[L + 1] = (int32_t)off;
  g->T = (int32_t)off;
  g->Tp = (int32_t)((off + 3) & ~(int64_t)3);  // node quads of the routing copy stay within one (b, h)
  return PISA_OK;
}

int supported(const Geo& g, int dtype, int mode) {
  (void)dtype;
  if (mode != PISA_PREFILL && mode != PISA_DECODE) return PISA_ERR_INVALID_ARG;
  if (g.d != 64 && g.d != 128) return PISA_ERR_UNSUPPORTED;
  if (g.C != kLeaf || g.g != 2 || g.K > 32) return PISA_ERR_UNSUPPORTED;
  if (g.G != 1 && g.G != 2 && g.G != 4 && g.G != 8 && g.G != 16) return PISA_ERR_UNSUPPORTED;
  if (mode == PISA_PREFILL) {
    // only the prefill workspace holds per-(query, slot) lists: entries pack (i << 6 | slot)
    // and list offsets are int32
    if (g.N >= (1 << 25)) return PISA_ERR_UNSUPPORTED;
    const int64_t slots = (int64_t)g.B * g.Hkv * g.N * 2 * g.K;
    if (slots >= ((int64_t)1 << 31) - 1) return PISA_ERR_UNSUPPORTED;
  }
  return PISA_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

PrefillWs prefill_ws(const Geo& g, int dtype) {
  PrefillWs w;
  w.slots = (int64_t)g.B * g.Hkv * g.N * 2 * g.K;
  w.M = g.B * g.Hkv * g.n1p;
  size_t o = 0;
  w.cand = o;    o = align256(o + sizeof(int32_t) * w.slots);
  w.lscore = o;  o = align256(o + sizeof(float) * w.slots);
  w.cnt = o;     o = align256(o + sizeof(int32_t) * w.M);
  w.cursor = o;  o = align256(o + sizeof(int32_t) * w.M);
  w.off = o;     o = align256(o + sizeof(int32_t) * (w.M + 1));
  w.choff = o;   o = align256(o + sizeof(int32_t) * (w.M + 1));
  w.entries = o; o = align256(o + sizeof(int32_t) * w.slots);
  w.fsc = o;     o = align256(o + sizeof(float) * 3 * (size_t)g.B * g.Hkv * g.N);
  w.lo8 = o;     o = align256(o + lo8_bytes(g));
  w.total_min = o;
  w.qg = o;
  if (route_scores_forced(g, dtype)) o = align256(o + 2 * (size_t)g.B * g.Hq * g.N * g.d);  // bf16, q's size
  w.total = o;
  return w;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Scratch of pisa_select_prefill_noalloc: one copy per device, held until the process ends.
// In host code `scratch` names a host-side stand-in; kernels get the device address that
// hipGetSymbolAddress returns for the current device (looked up once per device).
static __device__ __align__(256) unsigned char scratch[PISA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void* scratch_dev[kMaxDevices];

// Device address of the current device's scratch, or null (HIP error or device id out of range).
static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_dev[dev] = ptr;
  }
  return scratch_dev[dev];
}
static bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace pisa

using namespace pisa;

extern "C" {

int pisa_levels(const pisa_problem* p, int32_t* n_levels, int64_t* level_nodes, int64_t* level_offset) {
  Geo g;
  const int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (n_levels) *n_levels = g.L;
  if (level_nodes) {
    for (int l = 0; l < PISA_MAX_LEVELS + 2; ++l) level_nodes[l] = l <= g.L ? g.n[l] : 0;
  }
  if (level_offset) {
    for (int l = 0; l < PISA_MAX_LEVELS + 2; ++l) level_offset[l] = (l >= 1 && l <= g.L + 1) ? g.off[l] : 0;
  }
  return PISA_OK;
}

int pisa_pyramid_layout(const pisa_problem* p, int32_t* n_levels, int32_t* nodes, int64_t* node_offset) {
  Geo g;
  const int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (n_levels) *n_levels = g.L;
  if (nodes) {
    for (int i = 0; i < PISA_MAX_LEVELS; ++i) nodes[i] = i < g.L ? g.n[i + 1] : 0;
  }
  if (node_offset) {
    for (int i = 0; i <= PISA_MAX_LEVELS; ++i) node_offset[i] = i <= g.L ? g.off[i + 1] : 0;
  }
  return PISA_OK;
}

int pisa_supported(const pisa_problem* p, int mode) {
  Geo g;
  const int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  return supported(g, p->dtype, mode);
}

size_t pisa_pyramid_bytes(const pisa_problem* p) {
  Geo g;
  if (make_geo(p, &g) != PISA_OK) return 0;
  return 2 * sizeof(float) * (size_t)g.B * g.Hkv * g.Tp * g.d;  // fp32 means + bf16 hi/lo copy
}

size_t pisa_workspace_bytes(const pisa_problem* p, int mode) {
  Geo g;
  if (make_geo(p, &g) != PISA_OK) return 0;
  if (mode == PISA_DECODE) return 0;
  if (mode != PISA_PREFILL) return 0;
  return prefill_ws(g, p->dtype).total;
}

size_t pisa_prefill_workspace_min_bytes(const pisa_problem* p) {
  Geo g;
  if (make_geo(p, &g) != PISA_OK) return 0;
  return prefill_ws(g, p->dtype).total_min;
}

int pisa_build_pyramid(const pisa_problem* p, const void* k, float* pyramid, pisa_stream_t stream) {
  Geo g;
  int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (!k || !pyramid || !aligned16(k) || !aligned16(pyramid)) return PISA_ERR_INVALID_ARG;
  // the build uses no workspace lists: the decode support matrix (no prefill list limits)
  rc = supported(g, p->dtype, PISA_DECODE);
  if (rc != PISA_OK) return rc;
  return launch_build_pyramid(g, p->dtype, k, pyramid, (hipStream_t)stream);
}

static int select_prefill_impl(const pisa_problem* p, const void* q, const void* k, const float* pyramid,
                               void* workspace, size_t workspace_bytes, int32_t* out_idx, float* out_score,
                               void* const* ev, hipStream_t st) {
  Geo g;
  int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (!q || !k || !pyramid || !out_idx || !out_score || !workspace) return PISA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(pyramid) || !aligned16(workspace)) return PISA_ERR_INVALID_ARG;
  rc = supported(g, p->dtype, PISA_PREFILL);
  if (rc != PISA_OK) return rc;
  const PrefillWs w = prefill_ws(g, p->dtype);
  if (workspace_bytes < w.total_min) return PISA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  void* qg = (w.total > w.total_min && workspace_bytes >= w.total) ? ws + w.qg : nullptr;
  int32_t* cand = (int32_t*)(ws + w.cand);
  float* lscore = (float*)(ws + w.lscore);
  int32_t* cnt = (int32_t*)(ws + w.cnt);
  int32_t* cursor = (int32_t*)(ws + w.cursor);
  int32_t* off = (int32_t*)(ws + w.off);
  int32_t* choff = (int32_t*)(ws + w.choff);
  int32_t* entries = (int32_t*)(ws + w.entries);
  float* fsc = (float*)(ws + w.fsc);
  uint8_t* lo8 = (uint8_t*)(ws + w.lo8);
  auto mark = [&](int i) { return ev ? (hipEventRecord((hipEvent_t)ev[i], st) == hipSuccess ? PISA_OK : PISA_ERR_HIP)
                                     : PISA_OK; };

  if ((rc = mark(0)) != PISA_OK) return rc;
  // counters are contiguous: cnt then cursor (each 256-aligned)
  if ((rc = launch_zero(cnt, (int64_t)(w.off - w.cnt) / (int64_t)sizeof(int32_t), st)) != PISA_OK) return rc;
  // the entries region is free until the scatter: it carries the level-2 candidates
  if ((rc = launch_route(g, p->dtype, q, k, pyramid, entries, fsc, cand, cnt, qg, lo8, ev ? (hipEvent_t)ev[1] : nullptr,
                        st)) != PISA_OK)
    return rc;
  if ((rc = mark(2)) != PISA_OK) return rc;
  if (p->dtype == PISA_F32) {
    if ((rc = mark(3)) != PISA_OK) return rc;
    if ((rc = launch_qmajor(g, p->dtype, q, k, cand, out_idx, out_score, st)) != PISA_OK) return rc;
    if ((rc = mark(4)) != PISA_OK) return rc;
    return mark(5);
  }
  if ((rc = launch_scan(cnt, w.M, chunk_entries(g.G), off, choff, st)) != PISA_OK) return rc;
  if ((rc = launch_scatter_pairs(g, cand, off, cursor, entries, st)) != PISA_OK) return rc;
  if ((rc = mark(3)) != PISA_OK) return rc;
  if ((rc = launch_leaf_mfma(g, q, k, qg, off, choff, entries, w.M, lscore, st)) != PISA_OK) return rc;
  if ((rc = mark(4)) != PISA_OK) return rc;
  rc = route_scores_forced(g, p->dtype) ? launch_final(g, cand, lscore, fsc, out_idx, out_score, st)
                                        : launch_forced_final(g, q, k, cand, lscore, out_idx, out_score, st);
  if (rc != PISA_OK) return rc;
  return mark(5);
}

int pisa_select_prefill(const pisa_problem* p, const void* q, const void* k, const float* pyramid, void* workspace,
                        size_t workspace_bytes, int32_t* out_idx, float* out_score, pisa_stream_t stream) {
  return select_prefill_impl(p, q, k, pyramid, workspace, workspace_bytes, out_idx, out_score, nullptr,
                             (hipStream_t)stream);
}

int pisa_select_prefill_staged(const pisa_problem* p, const void* q, const void* k, const float* pyramid,
                               void* workspace, size_t workspace_bytes, int32_t* out_idx, float* out_score,
                               void* const* events, int32_t n_events, pisa_stream_t stream) {
  if (!events || n_events != 6) return PISA_ERR_INVALID_ARG;
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return PISA_ERR_INVALID_ARG;
  return select_prefill_impl(p, q, k, pyramid, workspace, workspace_bytes, out_idx, out_score, events,
                             (hipStream_t)stream);
}

int pisa_select_prefill_noalloc(const pisa_problem* p, const void* q, const void* k, const float* pyramid,
                                int32_t* out_idx, float* out_score, pisa_stream_t stream) {
  Geo g;
  int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (!q || !k || !pyramid || !out_idx || !out_score) return PISA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(pyramid)) return PISA_ERR_INVALID_ARG;
  rc = supported(g, p->dtype, PISA_PREFILL);
  if (rc != PISA_OK) return rc;
  // without room for the regrouped query copy the call reads q itself
  if (prefill_ws(g, p->dtype).total_min > (size_t)PISA_NOALLOC_SCRATCH_BYTES) return PISA_ERR_WORKSPACE;
  void* ws = scratch_address();
  if (!ws) return PISA_ERR_HIP;
  return select_prefill_impl(p, q, k, pyramid, ws, (size_t)PISA_NOALLOC_SCRATCH_BYTES, out_idx, out_score, nullptr,
                             (hipStream_t)stream);
}

int pisa_prefill_routed_pairs(const pisa_problem* p, const void* workspace, size_t workspace_bytes,
                              int64_t* routed_pairs, pisa_stream_t stream) {
  Geo g;
  int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (!workspace || !routed_pairs) return PISA_ERR_INVALID_ARG;
  rc = supported(g, p->dtype, PISA_PREFILL);
  if (rc != PISA_OK) return rc;
  const PrefillWs w = prefill_ws(g, p->dtype);
  if (workspace_bytes < w.total) return PISA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return PISA_ERR_HIP;
  // every routed leaf candidate holds a block id >= 0 in its slot (-1 elsewhere)
  const int32_t* cand = (const int32_t*)((const char*)workspace + w.cand);
  int64_t total = 0;
  const int64_t chunk = 1 << 20;
  int32_t* host = new (std::nothrow) int32_t[chunk];
  if (!host) return PISA_ERR_INTERNAL;
  for (int64_t o = 0; o < w.slots && rc == PISA_OK; o += chunk) {
    const int64_t n = w.slots - o < chunk ? w.slots - o : chunk;
    if (hipMemcpy(host, cand + o, sizeof(int32_t) * n, hipMemcpyDeviceToHost) != hipSuccess) rc = PISA_ERR_HIP;
    for (int64_t t = 0; t < n && rc == PISA_OK; ++t) total += host[t] >= 0;
  }
  delete[] host;
  if (rc == PISA_OK) *routed_pairs = total;
  return rc;
}

int pisa_prefill_dense_levels(const pisa_problem* p, int32_t* dense_top, int32_t* dense_bottom) {
  Geo g;
  int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (!dense_top || !dense_bottom) return PISA_ERR_INVALID_ARG;
  rc = supported(g, p->dtype, PISA_PREFILL);
  if (rc != PISA_OK) return rc;
  const bool dense = route_scores_forced(g, p->dtype);  // bf16 with L >= 3
  *dense_top = dense ? g.L : 0;
  *dense_bottom = dense ? pisa::dense_bottom(g) : 0;
  return PISA_OK;
}

int pisa_select_decode(const pisa_problem* p, const void* q, const void* k_cache, const float* pyramid,
                       void* workspace, size_t workspace_bytes, int32_t* out_idx, float* out_score,
                       pisa_stream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  Geo g;
  int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (!q || !k_cache || !pyramid || !out_idx || !out_score) return PISA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(pyramid)) return PISA_ERR_INVALID_ARG;
  rc = supported(g, p->dtype, PISA_DECODE);
  if (rc != PISA_OK) return rc;
  return launch_decode(g, p->dtype, q, k_cache, pyramid, nullptr, out_idx, out_score, (hipStream_t)stream);
}

int pisa_append_keys(const pisa_problem* p, const void* k_cache, const int32_t* old_lengths,
                     const int32_t* new_lengths, int32_t max_new_keys, float* pyramid, pisa_stream_t stream) {
  Geo g;
  int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (!k_cache || !old_lengths || !new_lengths || !pyramid) return PISA_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(pyramid) || !aligned4(old_lengths) || !aligned4(new_lengths))
    return PISA_ERR_INVALID_ARG;
  if (max_new_keys < 0 || max_new_keys > p->seq_len) return PISA_ERR_INVALID_ARG;
  rc = supported(g, p->dtype, PISA_DECODE);
  if (rc != PISA_OK) return rc;
  if (max_new_keys == 0) return PISA_OK;
  return launch_append(g, p->dtype, k_cache, old_lengths, new_lengths, max_new_keys, pyramid, (hipStream_t)stream);
}

int pisa_select_decode_varlen(const pisa_problem* p, const void* q, const void* k_cache, const float* pyramid,
                              const int32_t* lengths, int32_t* out_idx, float* out_score, pisa_stream_t stream) {
  Geo g;
  int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (!q || !k_cache || !pyramid || !lengths || !out_idx || !out_score) return PISA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(pyramid) || !aligned4(lengths)) return PISA_ERR_INVALID_ARG;
  rc = supported(g, p->dtype, PISA_DECODE);
  if (rc != PISA_OK) return rc;
  return launch_decode(g, p->dtype, q, k_cache, pyramid, lengths, out_idx, out_score, (hipStream_t)stream);
}

size_t pisa_attention_workspace_bytes(const pisa_problem* p, int32_t mode) {
  Geo g;
  if (make_geo(p, &g) != PISA_OK || (mode != PISA_PREFILL && mode != PISA_DECODE)) return 0;
  return attention_key_major(g, p->dtype, mode == PISA_DECODE) ? attention_ws(g, attention_full_range(g)).total : 0;
}

size_t pisa_attention_workspace_min_bytes(const pisa_problem* p, int32_t mode) {
  Geo g;
  if (make_geo(p, &g) != PISA_OK || (mode != PISA_PREFILL && mode != PISA_DECODE)) return 0;
  if (!attention_key_major(g, p->dtype, mode == PISA_DECODE)) return 0;
  // the smallest range whose list numbering fits (at most the full range)
  for (int32_t R = kLeafQueries; R <= attention_full_range(g); R += kLeafQueries) {
    const size_t t = attention_ws(g, R).total;
    if (t != SIZE_MAX) return t;
  }
  return attention_ws(g, attention_full_range(g)).total;
}

int pisa_sparse_attention(const pisa_problem* p, int32_t mode, const void* q, const void* k, const void* v,
                          const int32_t* idx, void* workspace, size_t workspace_bytes, void* out, float* lse,
                          pisa_stream_t stream) {
  Geo g;
  int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (mode != PISA_PREFILL && mode != PISA_DECODE) return PISA_ERR_INVALID_ARG;
  if (!q || !k || !v || !idx || !out) return PISA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned4(idx) || !aligned4(lse))
    return PISA_ERR_INVALID_ARG;
  rc = supported(g, p->dtype, mode);
  if (rc != PISA_OK) return rc;
  if (attention_key_major(g, p->dtype, mode == PISA_DECODE)) {
    if (!workspace || !aligned16(workspace)) return PISA_ERR_INVALID_ARG;
    if (attention_range(g, workspace_bytes) <= 0) return PISA_ERR_WORKSPACE;
  }
  return launch_attention(g, p->dtype, q, k, v, idx, mode == PISA_DECODE, workspace, workspace_bytes, out, lse,
                          (hipStream_t)stream);
}

int pisa_bsa_select_prefill(const pisa_problem* p, const void* q, const float* pyramid, int32_t* out_idx,
                            float* out_score, pisa_stream_t stream) {
  Geo g;
  int rc = make_geo(p, &g);
  if (rc != PISA_OK) return rc;
  if (!q || !pyramid || !out_idx || !out_score) return PISA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(pyramid)) return PISA_ERR_INVALID_ARG;
  rc = supported(g, p->dtype, PISA_PREFILL);
  if (rc != PISA_OK) return rc;
  if (p->dtype != PISA_BF16) return PISA_ERR_UNSUPPORTED;
  return launch_bsa(g, q, pyramid, out_idx, out_score, (hipStream_t)stream);
}

const char* pisa_status_string(int status) {
  switch (status) {
    case PISA_OK: return "ok";
    case PISA_ERR_INVALID_ARG: return "invalid argument";
    case PISA_ERR_UNSUPPORTED: return "unsupported problem for the gfx950 kernels";
    case PISA_ERR_WORKSPACE: return "workspace too small";
    case PISA_ERR_HIP: return "HIP runtime error";
    case PISA_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

const char* pisa_version(void) { return "0.1.0"; }

}  // extern "C"
