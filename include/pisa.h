/*
 * pisa.h -- C ABI of libpisa, PISA's pyramid Top-K block selector on MI355X (gfx950).
 *
 * The method ("Block Sparse Attention with Log-Linear Complexity", as summarised on
 * agihunt.info and explained on rcap.io) picks, for each query of a block-sparse
 * attention layer, the K leaf key blocks (tiles of C consecutive keys) it will attend to:
 *
 *   - keys are mean-pooled into a pyramid: level 1 holds one mean per leaf block of C
 *     keys, each coarser level holds the mean of g adjacent nodes of the level below
 *     (agihunt.info, pyramid paragraph; rcap.io, tree paragraph);
 *   - the walk starts at the coarsest stored level, scores each candidate node by the
 *     LogSumExp over its children of the scaled dot products q.child, keeps the Top-K and
 *     expands only their children, so each level scores at most g*K candidates (rcap.io,
 *     top-down walk and scoring-rule paragraphs);
 *   - at the leaf level the LSE runs over the block's raw keys, causally masked, and the
 *     first, previous and current leaf blocks are forced in (agihunt.info, LSE and
 *     forced-block paragraph);
 *   - the query heads of one GQA group share one selection (agihunt.info, kernels
 *     paragraph).
 *
 * Readings fixed by this library where the pages are silent:
 *   - the stored pyramid stops at the first level L with at most g*K nodes (every coarser
 *     level would hold <= K nodes, all of which a walk from a root keeps);
 *   - one pyramid per (batch, KV head); the group's score of a node is the SUM over its G
 *     query heads of the per-head LSE; Top-K orders by score descending, then block index
 *     ascending (lower index wins ties);
 *   - causality above the leaves is node-granular: a node covering leaf blocks starting at
 *     f is visible to a query in leaf block b iff f <= b; its full stored mean is used;
 *   - forced blocks F = {0, b-1, b} (those that exist) count inside K: the output is
 *     F u TopK_{K-|F|}(leaf candidates \ F), so K >= 3 and |selection| = min(K, b+1);
 *   - the scale s (default 1/sqrt(d)) multiplies each dot product in fp32; inputs are
 *     read exactly and every dot product and LSE is accumulated in fp32.
 *
 * Layouts (all row-major, contiguous, 16-byte aligned device memory on the current
 * device; query head hq belongs to KV head hq / G with G = n_q_heads / n_kv_heads):
 *   q (prefill)   [B, Hq, N, d]     dtype of the problem (fp32 or bf16)
 *   q (decode)    [B, Hq, d]        the new token's query, at position N-1
 *   k / k_cache   [B, Hkv, N, d]    dtype of the problem
 *   pyramid       pisa_pyramid_bytes() bytes: first the fp32 means [B, Hkv, Tp, d]
 *                 (T = sum of level sizes, level 1 (leaves) first, see pisa_levels;
 *                 Tp = T rounded up to a multiple of 4, the nodes past T unused), then an
 *                 equally sized routing copy: each mean times s * log2(e) (fp32 product,
 *                 s as resolved from the problem) split into bf16 hi + bf16 lo (hi + lo
 *                 equals that product to 2^-18 relative).  In each (b, h) block of the copy
 *                 nodes 4Q .. 4Q+3 share a record of 8d bf16: per 16 dims 16j .. 16j+15,
 *                 a 128-byte line of hi halves [dims 16j..+8 of the four nodes | dims
 *                 16j+8..+8 of the four nodes], then the line of lo halves alike.  The
 *                 copy is tied to the problem's scale
 *   out_idx       [B, Hkv, N, K] (prefill) or [B, Hkv, K] (decode), int32: selected leaf
 *                 block ids in ascending order, padded with -1
 *   out_score     same shape, fp32: each selected block's group-summed causal leaf LSE,
 *                 padded with -inf
 *
 * Ownership and execution: the caller allocates every buffer (inputs, pyramid, workspace,
 * outputs); the library allocates nothing and keeps no pointer after a call returns.
 * Compute calls are asynchronous: they validate their arguments on the host (returning an
 * error before any HIP call), enqueue kernels on `stream` and return without
 * synchronising.  Faults inside kernels surface at the caller's next synchronisation.
 * Calls on one stream are ordered; concurrent calls must not share a workspace.  The
 * library keeps no state between calls (apart from the device scratch of
 * pisa_select_prefill_noalloc) and no C++ exception crosses this interface.
 */
#ifndef PISA_H_
#define PISA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t is `struct ihipStream_t*`; NULL means the default stream. */
struct ihipStream_t;
typedef struct ihipStream_t* pisa_stream_t;

#define PISA_MAX_LEVELS 32

enum pisa_dtype { PISA_F32 = 0, PISA_BF16 = 1 };

enum pisa_mode { PISA_PREFILL = 0, PISA_DECODE = 1 };

/*
 * Score of a routing node (levels L..2) for one head, over the scaled dots x_c of its m
 * visible children (m = 1 or 2 here).  PISA_LSE: log sum exp(x_c), the method itself.
 * PISA_PISA1 / PISA_PISA2: the ablations that truncate that LSE about the children's mean
 * at first / second order ("Block Sparse Attention with Log-Linear Complexity":
 * agihunt.info summary, LSE paragraph; rcap.io explainer, scoring-rule paragraph):
 * log m + mean(x), and that plus half the population variance of x (for two children
 * (x_0 - x_1)^2 / 8).  Leaf and forced-block scores are the exact LSE under every scorer.
 */
enum pisa_scorer { PISA_LSE = 0, PISA_PISA1 = 1, PISA_PISA2 = 2 };

enum pisa_status {
  PISA_OK = 0,
  PISA_ERR_INVALID_ARG = 1, /* bad shape, null pointer, misalignment */
  PISA_ERR_UNSUPPORTED = 2, /* valid problem outside the kernels' support matrix */
  PISA_ERR_WORKSPACE = 3,   /* workspace smaller than pisa_workspace_bytes() */
  PISA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  PISA_ERR_INTERNAL = 5
};

typedef struct {
  int32_t batch;      /* B >= 1 */
  int32_t seq_len;    /* N >= 1: prefill length; decode: key-cache length incl. the new token */
  int32_t n_q_heads;  /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;   /* d */
  int32_t block;      /* C, keys per leaf block */
  int32_t top_k;      /* K >= 3 (the three forced blocks count inside K) */
  int32_t branch;     /* g >= 2, children per pyramid node */
  float scale;        /* s; <= 0 selects 1/sqrt(d) */
  int32_t dtype;      /* enum pisa_dtype, of q and k */
  int32_t scorer;     /* enum pisa_scorer; 0 (PISA_LSE) is the method */
} pisa_problem;

/*
 * Level table.  level_nodes[l] (l = 0..L) holds n_l with n_0 = N, n_1 = ceil(N/C),
 * n_l = ceil(n_{l-1}/g), L = first level with n_L <= g*K.  level_offset[l] (l = 1..L+1) is
 * the node offset of level l inside one (batch, KV head) pyramid (level_offset[1] = 0,
 * level_offset[L+1] = T; the pyramid buffer's node stride per (batch, KV head) is T rounded
 * up to a multiple of 4).  Both arrays must hold PISA_MAX_LEVELS + 2 entries; either may
 * be NULL.  Returns PISA_OK or PISA_ERR_INVALID_ARG.
 */
int pisa_levels(const pisa_problem* p, int32_t* n_levels, int64_t* level_nodes, int64_t* level_offset);

/*
 * The same level table in the pyramid's own terms, leaf level first: nodes[i] = n_{i+1}
 * for i = 0..L-1 and node_offset[i] = offset of level i+1 inside one (batch, KV head)
 * pyramid for i = 0..L, so node_offset[L] = T, the nodes per (batch, KV head); entries
 * past those are set to 0.  nodes must hold PISA_MAX_LEVELS entries, node_offset
 * PISA_MAX_LEVELS + 1; either may be NULL.  Host only.  Returns PISA_OK or
 * PISA_ERR_INVALID_ARG.
 */
int pisa_pyramid_layout(const pisa_problem* p, int32_t* n_levels, int32_t* nodes, int64_t* node_offset);

/* PISA_OK if the kernels support this problem in this mode, else the error code. */
int pisa_supported(const pisa_problem* p, int mode);

/* Bytes of the pyramid buffer (fp32 means + routing copy, 2 * 4*B*Hkv*Tp*d with Tp = T
 * rounded up to a multiple of 4); 0 for an invalid problem. */
size_t pisa_pyramid_bytes(const pisa_problem* p);

/* Bytes of device workspace a call in `mode` needs (may be 0); 0 for an invalid problem.
 * For bf16 prefill with L >= 3 this includes room for a copy of q regrouped so that the G
 * heads of a KV head sit together per 8-dim piece, which the routing launch writes and the
 * gather and leaf launches read (their query loads then take whole cache lines); a
 * workspace of at least pisa_prefill_workspace_min_bytes runs without that copy, with the
 * same results. */
size_t pisa_workspace_bytes(const pisa_problem* p, int mode);
size_t pisa_prefill_workspace_min_bytes(const pisa_problem* p);

/*
 * Builds the pyramid of k [B, Hkv, N, d] into `pyramid` (agihunt.info, pyramid paragraph:
 * level 1 = mean of each leaf block's keys, a short last block averaging the keys it has;
 * level l = unweighted mean of the g (or fewer, at the end) level l-1 nodes below it).
 * One pass over k in HBM; writes the fp32 means and their routing copy.  The result is
 * reused by every prefill or decode call on k.
 */
int pisa_build_pyramid(const pisa_problem* p, const void* k, float* pyramid, pisa_stream_t stream);

/*
 * Prefill selection for every query position i in [0, N) of every (batch, KV head):
 * routing walk over levels L..2, leaf LSE scoring of the candidates, forced blocks and
 * Top-K as described above.  `pyramid` must hold pisa_build_pyramid's result for k.
 * Writes out_idx / out_score [B, Hkv, N, K].
 */
int pisa_select_prefill(const pisa_problem* p, const void* q, const void* k, const float* pyramid,
                        void* workspace, size_t workspace_bytes, int32_t* out_idx, float* out_score,
                        pisa_stream_t stream);

/*
 * Decode selection for one new query per sequence, at position N-1 of a key cache of
 * length N that already holds the new token's key; one fused kernel (agihunt.info,
 * kernels paragraph: single-stage decode).  Equal to row N-1 of pisa_select_prefill on
 * the same keys.  Writes out_idx / out_score [B, Hkv, K].
 */
int pisa_select_decode(const pisa_problem* p, const void* q, const void* k_cache, const float* pyramid,
                       void* workspace, size_t workspace_bytes, int32_t* out_idx, float* out_score,
                       pisa_stream_t stream);

/*
 * Same as pisa_select_prefill, and additionally records caller-created HIP events
 * (hipEvent_t handles, e.g. from hipEventCreate) on `stream` at the stage boundaries:
 * events[0] before the first kernel, events[1] after counter clearing and the routing of
 * the upper levels (bf16: the dense launch, levels of pisa_prefill_dense_levels),
 * events[2] after the routing of the levels below it down to level 2 (fp32: all levels),
 * events[3] after leaf grouping (scan + scatter), events[4] after leaf scoring,
 * events[5] after forced blocks + final Top-K.  n_events must be 6.  Stages a problem does
 * not use (L < 3; fp32 inputs walk all levels in one launch and score leaves query-major
 * in stage 4) record their boundary events back to back.  For per-kernel timing of the
 * prefill path.
 */
int pisa_select_prefill_staged(const pisa_problem* p, const void* q, const void* k, const float* pyramid,
                               void* workspace, size_t workspace_bytes, int32_t* out_idx, float* out_score,
                               void* const* events, int32_t n_events, pisa_stream_t stream);

/*
 * pisa_select_prefill for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): no workspace argument;
 * the call runs on a scratch array of PISA_NOALLOC_SCRATCH_BYTES that the library holds on
 * each device it runs on until the process ends (its address is looked up on the first
 * call on a device), and allocates nothing.  Problems whose prefill workspace
 * (pisa_prefill_workspace_min_bytes(p)) exceeds it return PISA_ERR_WORKSPACE: 64 MiB
 * covers, for example, 78K tokens with 4 KV heads at K = 8 (the regrouped query copy is
 * used when it fits as well).  Every call on a device shares
 * that device's scratch, so calls that overlap on one GPU (several streams, several host
 * threads) race: the caller orders them, e.g. on one stream.  The scratch needs no clearing
 * (each call clears its own counters with a kernel, not a memset).  Results equal
 * pisa_select_prefill's.
 */
#define PISA_NOALLOC_SCRATCH_BYTES (64u << 20)
int pisa_select_prefill_noalloc(const pisa_problem* p, const void* q, const void* k, const float* pyramid,
                                int32_t* out_idx, float* out_score, pisa_stream_t stream);

/*
 * Diagnostic, blocking: after a bf16 pisa_select_prefill on `stream` with `workspace`,
 * waits for the stream and reports how many (query group, leaf block) pairs the routing
 * walk sent to leaf scoring (forced blocks excluded).  fp32 problems report the number of
 * non-empty routed candidate slots the same way.
 */
int pisa_prefill_routed_pairs(const pisa_problem* p, const void* workspace, size_t workspace_bytes,
                              int64_t* routed_pairs, pisa_stream_t stream);

/*
 * Host only: how pisa_select_prefill splits the routing walk for p.  The bf16 path scores
 * levels *dense_top = L down to *dense_bottom densely, every visible node for all queries
 * of a leaf block at once, and walks the levels below down to level 2 by per-query gathers;
 * the dense launch covers a level while its child level has at most 1024 nodes, so with at
 * most 1024 leaf blocks every level down to 2 is dense (*dense_bottom = 2) and no gather
 * launch runs.  Both are 0 when there is no dense launch (L < 3, or fp32 inputs, which walk
 * every level by gathers).
 * The top-down walk and its result do not depend on the split.  Returns PISA_OK, or the
 * status pisa_select_prefill would return for an invalid or unsupported p.
 */
int pisa_prefill_dense_levels(const pisa_problem* p, int32_t* dense_top, int32_t* dense_bottom);

/* Static description of a status code. */
/*
 * Growing key caches (decode with per-sequence lengths).  Here p->seq_len is the cache
 * capacity: k_cache is [B, Hkv, capacity, d] and the pyramid buffer is laid out for the
 * capacity (pisa_pyramid_bytes(p), level offsets of pisa_levels(p)); sequence b holds
 * lengths[b] keys and uses, inside that layout, the level table of its own length (n_l
 * and L of a problem with seq_len = lengths[b]).
 *
 * pisa_append_keys updates the pyramid after sequence b grew from old_lengths[b] to
 * new_lengths[b] keys (the caller has written the new keys into k_cache): the leaf blocks
 * holding positions old..new-1 are recomputed from their raw keys and every ancestor of
 * those blocks from its children present at the new length, one node per level for a
 * single new key ("Block Sparse Attention with Log-Linear Complexity", agihunt.info
 * summary, pyramid paragraph: each level mean-pools the one below, so a key changes one
 * node per level).  The updated nodes hold the same bits as pisa_build_pyramid of a
 * problem with seq_len = new_lengths[b] on the same keys; levels above the sequence's own
 * top level are maintained too, for when it grows.  old_lengths = 0 builds a sequence from
 * scratch.  old_lengths / new_lengths: device int32 [B] with 0 <= old <= new <= capacity
 * and new - old <= max_new_keys (host int, 0 <= max_new_keys <= capacity); values outside
 * that contract are clamped on the device and leave the pyramid unspecified, never an
 * out-of-bounds access.  One launch on `stream` when max_new_keys == 1 (the changed path
 * carried up in registers), two otherwise; no workspace.
 *
 * pisa_select_decode_varlen is pisa_select_decode for the query of sequence b at position
 * lengths[b] - 1 (device int32 [B], 1 <= lengths[b] <= capacity, clamped on the device),
 * on the pyramid that pisa_append_keys maintains.  Equal to pisa_select_decode on a
 * problem with seq_len = lengths[b] for each sequence.  q [B, Hq, d].
 */
int pisa_append_keys(const pisa_problem* p, const void* k_cache, const int32_t* old_lengths,
                     const int32_t* new_lengths, int32_t max_new_keys, float* pyramid, pisa_stream_t stream);
int pisa_select_decode_varlen(const pisa_problem* p, const void* q, const void* k_cache, const float* pyramid,
                              const int32_t* lengths, int32_t* out_idx, float* out_score, pisa_stream_t stream);

/*
 * Block-sparse attention over a selection, the consumer the selector feeds
 * ("Block Sparse Attention with Log-Linear Complexity": agihunt.info summary, opening
 * paragraph: each query reads only its Top-K tiles of C keys; rcap.io explainer, first
 * paragraphs: attention then runs over the original keys of the picked blocks).  For every
 * query head hq of KV head h and position i (mode PISA_PREFILL: q [B, Hq, N, d], idx
 * [B, Hkv, N, K], out [B, Hq, N, d], lse [B, Hq, N]; mode PISA_DECODE: the query at N-1,
 * q [B, Hq, d], idx [B, Hkv, K], out [B, Hq, d], lse [B, Hq]):
 *   out = sum_t softmax_t(s * <q, k_t>) v_t,   lse = log sum_t exp(s * <q, k_t>),
 * over the keys t <= i of the blocks idx[b, h, i, 0..K) (shared by the G heads of the
 * group; entries < 0 or after the query's own block are skipped; entries must be distinct,
 * as pisa_select_* produce them).  k and v [B, Hkv, N, d] of q's dtype; out has q's dtype
 * (bf16 rounded to nearest even from fp32 accumulation); lse fp32, may be NULL.  A row
 * with no attended key gets out = 0, lse = -inf.  bf16 prefill attends the blocks
 * {0, b-1, b} of each leaf block b for all its queries at once (each query masked by
 * whether its selection names them), sorts the other (query group, block) pairs by block,
 * attends each block's staged key and value tiles on the matrix cores and merges the
 * partial outputs (kept in bf16 in the workspace).  The partials of one query range at a
 * time live in the workspace: with pisa_attention_workspace_bytes(p, mode) bytes (16-byte
 * aligned device memory) the whole sequence is one range; with less, but at least
 * pisa_attention_workspace_min_bytes(p, mode), the call takes as few passes over ranges of
 * consecutive queries (multiples of 2048) as the given size allows, with the same results
 * (PISA_ERR_WORKSPACE below the minimum).  fp32 inputs and decode need none (workspace may
 * be NULL; both sizes are 0).
 */
size_t pisa_attention_workspace_bytes(const pisa_problem* p, int32_t mode);
size_t pisa_attention_workspace_min_bytes(const pisa_problem* p, int32_t mode);
int pisa_sparse_attention(const pisa_problem* p, int32_t mode, const void* q, const void* k, const void* v,
                          const int32_t* idx, void* workspace, size_t workspace_bytes, void* out, float* lse,
                          pisa_stream_t stream);

/*
 * Full-scan BSA selection for every query position, the baseline the pyramid selector is
 * timed against ("Block Sparse Attention with Log-Linear Complexity": agihunt.info
 * summary, opening and baselines paragraphs; rcap.io explainer, picking-step and
 * comparison-point paragraphs: standard block-sparse attention scores every query against
 * every block's mean-pooled summary, O(N^2/C)).  Block j's score for query group
 * (b, h, i) is sum over the G heads of s * <q, mean of block j's keys> (pyramid level 1;
 * no LSE); the candidates are the blocks 0..b of the query's leaf block b; the forced
 * blocks {0, b-1, b} are kept as in pisa_select_prefill and the K - |F| best remaining
 * blocks (score descending, lower index first) join them.  Writes out_idx / out_score
 * [B, Hkv, N, K] ascending by block index; forced blocks report +inf, padding (-1, -inf).
 * `pyramid` must hold pisa_build_pyramid's result for k (only its routing copy of level 1
 * is read).  bf16 q only (PISA_ERR_UNSUPPORTED otherwise); the scorer field has no
 * effect.  No workspace; q [B, Hq, N, d] and pyramid 16-byte aligned.
 */
int pisa_bsa_select_prefill(const pisa_problem* p, const void* q, const float* pyramid, int32_t* out_idx,
                            float* out_score, pisa_stream_t stream);

const char* pisa_status_string(int status);

/* Library version, e.g. "0.1.0". */
const char* pisa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H_ */
