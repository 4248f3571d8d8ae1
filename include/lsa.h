/*
 * liblsa: content-routed block sparse attention on AMD Instinct MI355X (gfx950).
 *
 * The operation (SSA page, jonsmirl/ssa, opening paragraph and "Algorithm and
 * complexity"; LLSA page, "Minimum Usage"; Subquadratic Sparse Attention page,
 * "Architecture"): keys are mean-pooled into fixed blocks; every query (in the
 * non-causal image mode, every query block) scores the block summaries,
 * keeps its top-k blocks and, in causal mode, a local causal window; exact
 * softmax attention then runs over only the selected keys.  The dense n x n
 * score matrix is never formed.
 *
 * Tensors (all device memory, row-major, the last index fastest):
 *   q    [B, Hq,  N, D] bf16      k, v [B, Hkv, N, D] bf16
 *   kbar [B, Hkv, N/bs, D] fp32   (block means)
 *   idx  causal: [B, Hq, N, top_k] int32; image mode: [B, Hq, N/bs, top_k]
 *        (consensus routing: Hkv in place of Hq, one route per KV group)
 *   out  [B, Hq, N, D] fp32
 * Query head h reads KV head h / (Hq / Hkv) (grouped-query attention with
 * contiguous head groups).
 *
 * Conventions shared by every call:
 *   - Ownership: the caller owns every buffer.  The library never allocates
 *     or frees memory and keeps no state between calls.  Scratch space is a
 *     caller-provided workspace of lsa_workspace_bytes() bytes (256-byte
 *     aligned).
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  All
 *     work is enqueued asynchronously on it; no call synchronises the host.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; on error nothing is launched.  LSA_ERR_DEVICE reports a
 *     failed launch; a device fault surfaces at the caller's next
 *     synchronisation.
 *   - Inputs are not checked for finiteness: NaN or Inf give an unspecified
 *     result but every access stays in bounds.
 *   - Determinism: the same inputs give bitwise identical outputs.  A row
 *     whose k-th and (k+1)-th routing scores agree to within fp32 rounding
 *     may keep either block; which one can depend on the rest of the input
 *     (the fp32-accurate scores come from bf16 hi+lo MFMA products, or, when
 *     the launch's longest bf16-query row has 4096 or more candidates, from
 *     the hi product plus a bf16 dot product with the lo part; rows that
 *     overflow the router's fast path are rescored by an exact pass, one by
 *     one with fp32 FMA chains when at most 16384 rows need it, by whole
 *     tiles with the hi+lo products when more do), but never on the stream,
 *     the run or the calling thread.
 *   - Calls on distinct streams with distinct workspaces may run
 *     concurrently.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lsa_params {
    int32_t batch;     /* B >= 1 */
    int32_t q_heads;   /* Hq >= 1 */
    int32_t kv_heads;  /* Hkv >= 1, Hq % Hkv == 0 */
    int32_t seq_len;   /* N, a positive multiple of block; N/block <= 65536 */
    int32_t head_dim;  /* D; this build supports 64 */
    int32_t block;     /* bs: 16, 32, 64 or 128 (key block; in image mode also the query block) */
    int32_t top_k;     /* 1 .. 32 */
    int32_t window;    /* causal: a multiple of block, >= block; image mode: 0 */
    int32_t causal;    /* 1: per-query routing + causal window; 0: image mode */
    float scale;       /* softmax scale; <= 0 selects 1/sqrt(D) */
    int32_t consensus; /* 0: a route per query head; 1: one route per KV group,
                          shared by the group's query heads (see lsa_route_topk) */
    float beta;        /* second-cumulant weight of the routing score (see
                          lsa_route_cumulant); 0: the block-mean score.  Must be
                          finite; nonzero needs causal = 1 and consensus = 0 */
    int32_t beam;      /* two-level routing: nodes kept per query or query
                          block (see lsa_route_topk); 0: flat routing.
                          1..15, needs consensus = 0 and beta = 0 */
    int32_t chunk;     /* causal attention: query positions per chunk (see
                          lsa_sparse_attend); 0 chooses it from the geometry,
                          otherwise a power of two >= 64.  Results do not
                          depend on it; the workspace does */
} lsa_params;

typedef enum lsa_status {
    LSA_OK = 0,
    LSA_ERR_NULL = 1,        /* a required pointer is NULL */
    LSA_ERR_SHAPE = 2,       /* inconsistent sizes (N % block, Hq % Hkv, window, ...) */
    LSA_ERR_UNSUPPORTED = 3, /* valid but outside this build (D != 64, top_k > 32,
                                B*Hq*N*2^ceil(log2 top_k) >= 2^32, ...) */
    LSA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned (workspace: 256) */
    LSA_ERR_WORKSPACE = 5,   /* workspace smaller than lsa_workspace_bytes() */
    LSA_ERR_DEVICE = 6,      /* a HIP launch failed */
    LSA_ERR_SCRATCH = 7      /* needs more scratch than the static array holds
                                (lsa_decode_noalloc) */
} lsa_status;

enum {
    LSA_OP_SUMMARIZE = 0,
    LSA_OP_ROUTE = 1,
    LSA_OP_ATTEND = 2,
    LSA_OP_FORWARD = 3,
    LSA_OP_DECODE = 4     /* p->seq_len read as the cache length */
};

/* Workspace bytes needed by `op` for these parameters (0 = none needed;
 * (size_t)-1 when the parameters are invalid). */
size_t lsa_workspace_bytes(const lsa_params *p, int32_t op);

/* Block summary (SSA page, "Algorithm and complexity": the first cumulant
 * mu_c of the routing score r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q).
 * x [B, heads, N, D] bf16 -> xbar [B, heads, N/bs, D] fp32, where
 * xbar[c] = the mean of tokens [c*bs, c*bs + bs), summed in fp64 and
 * rounded once to fp32.  `heads` is Hkv for keys, Hq for pooled queries. */
lsa_status lsa_block_summarize(const lsa_params *p, const void *x, int32_t heads,
                               float *xbar, void *stream);

/* Routing: scores <q, kbar_c> (beta = 0) and top-k selection with ties
 * broken toward the lower block index.
 * Causal (causal = 1): row t of head h considers the complete blocks
 *   c < E(t) = max(0, t/bs - window/bs + 1), i.e. the blocks that end before
 *   the block-aligned local window (SSA page, "Mathematical status" and
 *   "Known limitations": a routed set is causal only once cut at the query
 *   position; Subquadratic Sparse Attention page, "Why the layer is
 *   mathematically subquadratic": completed blocks are exposed only when
 *   their last token precedes the cutoff).  idx [B, Hq, N, top_k].
 * Image mode (causal = 0): query block i (tokens [i*bs, i*bs+bs)) is pooled
 *   to its fp32 mean and scored against all N/bs key blocks (LLSA page,
 *   "Minimum Usage").  idx [B, Hq, N/bs, top_k].
 * Each idx row lists min(top_k, #candidates) block ids in ascending order,
 * then -1 padding.
 * Consensus routing (consensus = 1; SSA page, "Complete 10M transformer
 *   result": a cross-head consensus route): one route per KV group, scored
 *   by the sum of the routing scores of the group's Hq/Hkv query heads,
 *   sum_h <q_h, kbar_c> (image mode: of their pooled queries); candidates,
 *   top-k and tie-break as above.  idx [B, Hkv, N, top_k] (image mode
 *   [B, Hkv, N/bs, top_k]); every query head of the group attends through
 *   its group's route.
 * Two-level routing (beam > 0; SSA page, "Algorithm and complexity": a
 *   hierarchical router with fixed block size and budget, the measured tree
 *   at fanout 16): nodes group 16 consecutive key blocks and are summarised
 *   by the mean of their block means (fp32).  Row t scores its S =
 *   floor(E(t)/16) complete candidate nodes, keeps the best min(beam, S)
 *   (ties to the lower node), and takes its top-k among the blocks of those
 *   nodes plus the tail blocks [16 S, E(t)) of the incomplete node.  With
 *   beam >= S every candidate is scored and the result is the flat
 *   selection.  Routing work per row falls from E(t) to about
 *   E(t)/16 + 16 beam + 15 scores.  In image mode (LLSA page, "Minimum
 *   Usage": the two-level kernel for 16384 tokens and more) the rows are
 *   the pooled query blocks and every row's candidates are all N/bs key
 *   blocks: S = floor(N/bs/16) nodes and the tail [16 S, N/bs).
 * beta != 0 is LSA_ERR_UNSUPPORTED here: that score needs the keys
 * themselves (lsa_route_cumulant).
 * Diagnostic: after a call with beam = 0 has run, the workspace's first
 * 4 bytes hold (uint32) how many rows overflowed the fast path's survivor
 * lists (ties on many blocks cause this), and the next 4 bytes how many
 * 128-row tiles held such a row.  Up to 1024 such rows are redone one by
 * one; beyond that, those tiles are redone whole.  The result is the same
 * either way. */
lsa_status lsa_route_topk(const lsa_params *p, const void *q, const float *kbar,
                          int32_t *idx, void *workspace, size_t workspace_bytes,
                          void *stream);

/* Routing by the second-cumulant score (SSA page, "Algorithm and
 * complexity"):  r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q, where mu_c is
 * the mean and Sigma_c the covariance (normalised by bs) of block c's keys;
 * beta = p->beta.  Candidates (causal only), top-k, tie-break and the idx
 * layout [B, Hq, N, top_k] are those of lsa_route_topk.  q^T Sigma_c q is
 * evaluated as the variance over the block of the raw scores q . k_j, so
 * the call reads the keys k [B, Hkv, N, D] bf16 and needs no block means
 * and no workspace.  Scores are fp32 sums of exact bf16 products; each
 * block's mean and variance are formed without cancellation.  Needs
 * causal = 1 and consensus = 0 (LSA_ERR_UNSUPPORTED otherwise). */
lsa_status lsa_route_cumulant(const lsa_params *p, const void *q, const void *k,
                              int32_t *idx, void *stream);

/* Exact softmax attention over the selected keys only (SSA page, opening
 * paragraph; Subquadratic Sparse Attention page, "Architecture").
 * Causal: row t attends to the routed blocks listed in idx plus the window
 *   keys [bs*E(t), t]; logits (q . k_j) * scale.
 * Image mode: every token of query block i attends to the union of the
 *   blocks listed for i.
 * idx is normally the output of lsa_route_topk.  An entry is used only if it
 * is a candidate block (causal: 0 <= c < E(t); image mode: 0 <= c < N/bs) and
 * greater than the previously used entry of its row; anything else is
 * skipped, so every access stays in bounds for any idx contents.  With
 * consensus = 1 idx holds one route per KV group (lsa_route_topk's layout)
 * and query head h reads the route of its group h / (Hq / Hkv).
 * out [B, Hq, N, D] fp32.
 * Causal mode runs key-block-major over chunks of query positions (all
 * heads): per chunk, every (row, routed block) pair's partial softmax is
 * formed with its key block staged once for all rows that chose it, then the
 * window attention merges the row's partials.  p->chunk sets the positions
 * per chunk (0: the whole sequence, unless its partials would exceed
 * 32 GiB; chunks cost time, as each splits every key block's rows).  The
 * output does not depend on the chunk size; the workspace holds one chunk's
 * partials (B * Hq * chunk * 2^ceil(log2 top_k) rows of 128 bytes, plus
 * 4 bytes per routed pair of the chunk), 8 bytes per routed pair of the
 * whole layer, and 16 bytes per bucket: a bucket is a key block of one
 * (b, KV head) for one span of query positions, spans short enough for
 * their query rows to stay cached while the blocks that chose them run. */
lsa_status lsa_sparse_attend(const lsa_params *p, const void *q, const void *k,
                             const void *v, const int32_t *idx, float *out,
                             void *workspace, size_t workspace_bytes, void *stream);

/* The whole layer: summarize K, route, attend.  idx_out may be NULL (the
 * selection then lives in the workspace); otherwise it receives idx as
 * lsa_route_topk writes it.  With beta != 0 the routing is
 * lsa_route_cumulant's (the key summary stage is then empty). */
lsa_status lsa_forward(const lsa_params *p, const void *q, const void *k,
                       const void *v, float *out, int32_t *idx_out,
                       void *workspace, size_t workspace_bytes, void *stream);

/* One decode step: the query at position T-1 (T = p->seq_len, 1 <= T <=
 * cache_len) attends to a key/value cache with the same selection and
 * softmax as the prefill path (routing over the complete blocks before the
 * block-aligned window, top-k with the lower-index tie-break, exact softmax
 * over the routed blocks and the window [bs*E(T-1), T-1]); the SSA page
 * ("Other measured evidence") measures such steps against a growing cache
 * at a fixed selection budget.  causal must be 1.
 *   q          [B, Hq, D] bf16 (the new token's queries)
 *   k_cache,   [B, Hkv, cache_len, D] bf16, tokens [0, T) filled
 *   v_cache
 *   kbar_cache [B, Hkv, cache_len/bs, D] fp32 block means, in/out: blocks
 *              complete before the first call must be filled by the caller
 *              (lsa_block_summarize over the cache); when T is a multiple
 *              of bs this call writes the mean of block T/bs - 1, which token
 *              T-1 completes, so consecutive steps keep the cache current.
 *   out        [B, Hq, D] fp32;  idx_out [B, Hq, top_k] int32 or NULL.
 * cache_len must be a multiple of bs; workspace: lsa_workspace_bytes(p with
 * seq_len = cache_len, LSA_OP_DECODE) bytes, enough for every T <= cache_len.
 * Scores and softmax run in fp32 (no bf16 rounding of probabilities).
 * consensus, beta and beam must be 0 (LSA_ERR_UNSUPPORTED otherwise). */
lsa_status lsa_decode(const lsa_params *p, int32_t cache_len, const void *q,
                      const void *k_cache, const void *v_cache, float *kbar_cache,
                      float *out, int32_t *idx_out, void *workspace,
                      size_t workspace_bytes, void *stream);

/* lsa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments, layouts, results and errors are those of lsa_decode, without
 * the workspace: its scratch (the same layout, lsa_workspace_bytes(p with
 * seq_len = cache_len, LSA_OP_DECODE) bytes) lives in a static device array of
 * LSA_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  A geometry that needs more returns
 * LSA_ERR_SCRATCH before anything is enqueued.  The call allocates and frees
 * nothing; the first call on a device looks the array's address up once.
 * The array keeps the last call's contents and everything that must start at
 * zero is cleared by the call's own kernels, but it is shared by every call
 * on that GPU: calls that overlap on one GPU (concurrent streams or host
 * threads) race and must be serialised by the caller. */
#define LSA_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
lsa_status lsa_decode_noalloc(const lsa_params *p, int32_t cache_len, const void *q,
                              const void *k_cache, const void *v_cache, float *kbar_cache,
                              float *out, int32_t *idx_out, void *stream);

/* lsa_forward with stage timing, for profiling tools.  `events` holds
 * LSA_PROFILE_EVENTS hipEvent_t handles created by the caller; event i is
 * recorded on `stream` at the i-th stage boundary:
 *   0 start, 1 key summary, 2 routing, 3 routing fallback, 4 V transpose and
 *   bucket count, 5 bucket scan, 6 bucket scatter, 7 routed-block partials,
 *   8 window and merge (image mode: 1 includes the query pooling, 4-7 are
 *   empty and 8 is the image-mode attention).
 * Elapsed time between events i-1 and i is the duration of stage i.  No
 * synchronisation happens inside; otherwise identical to lsa_forward. */
#define LSA_PROFILE_EVENTS 9
lsa_status lsa_forward_profiled(const lsa_params *p, const void *q, const void *k,
                                const void *v, float *out, int32_t *idx_out,
                                void *workspace, size_t workspace_bytes, void *stream,
                                void *const *events);

/* Static description of a status code. */
const char *lsa_status_str(lsa_status s);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
