/*
 * sa.h -- C ABI of the query-dependent sparse-attention library (libsa.so),
 * written for AMD Instinct MI355X (gfx950).
 *
 * The library computes one hot path:
 *   1. an indexer scores every cached key cheaply -- either a low-rank (r = 16)
 *      projection of pre-RoPE queries and keys ("Full Attention Strikes Back",
 *      method section 2; one head-collapsed channel per key/value group,
 *      "Oracle-Guided Sparse Prefill", section 2.2), or a second-order Taylor
 *      score of 64-token pages from their mean and diagonal variance ("SPLA",
 *      section 2.1);
 *   2. a support set is chosen by dynamic top-p attention mass with a
 *      sort-free histogram threshold, or by top-k ("Full Attention Strikes
 *      Back", method sections 3 and 5);
 *   3. exact softmax attention runs over the selected keys/values only, one
 *      support per key/value group shared by its query heads, per query in
 *      decode and per block of b_sel queries in causal prefill
 *      ("Oracle-Guided Sparse Prefill", section 2.1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless marked "host".  The caller owns every
 *    buffer; the library never allocates or frees memory.  Scratch memory is
 *    passed in as a workspace whose size comes from sa_workspace_size().
 *  - A workspace must be zero-filled once before its first use; every call
 *    leaves the parts it relies on zero again, so one workspace serves any
 *    number of calls of the same entry point and shape (its layout depends
 *    on both; other parts may be left holding intermediate values).  Calls
 *    that share a workspace must be ordered (same stream, or synchronised).
 *  - Every call is asynchronous on the given HIP stream (NULL = default
 *    stream) and never synchronises the host.
 *  - Few-row problems may run as one persistent launch (one workgroup per
 *    compute unit, the workgroups of a row meeting at in-memory barriers):
 *    sa_decode_step and sa_decode_step_pages with batch * n_kv_heads <= 16,
 *    and sa_select_topp / sa_select_topk on up to 16 long rows.  The library
 *    takes that path only when the runtime reports that a workgroup of the
 *    kernel fits a compute unit; the launch still needs the compute units to
 *    itself while it runs (no kernel of another stream resident beside it).
 *    A barrier that waits about a second gives up so the launch ends: every
 *    row whose barrier gave up then reports count[row] = -1 (its list and
 *    outputs are invalid), and the next call on the workspace starts clean.
 *    Whenever count[row] >= 0 the row's results are complete.
 *  - Arguments are checked on the host before anything is launched; a failed
 *    check returns an error code, launches nothing and writes nothing.
 *    sa_last_error() then gives a message (per calling thread).  A failed
 *    launch returns SA_ERR_HIP.
 *  - Layouts are row-major, rightmost index fastest.  Grouped-query attention:
 *    with G = n_q_heads / n_kv_heads, query head h uses key/value group h / G.
 *  - Paged caches: a pool holds n_pool_pages pages, each [n_kv_heads][page][w]
 *    for a row width w (head_dim for keys/values, idx_rank for indexer keys,
 *    2 * head_dim for page statistics: mean then variance).  Token t of
 *    sequence b lives in pool page page_table[b][t / page], slot t % page.
 *    seq_lens[b] must lie in [0, max_len] and every page id a sequence uses in
 *    [0, n_pool_pages); kernels clamp both into range rather than fault, so a
 *    violation gives wrong values, never an out-of-bounds access.
 *  - Support lists: idx[row][cap] int32, ascending token indices padded with -1,
 *    count[row] the number of valid entries; row = b * n_kv_heads + g for decode
 *    and blk * n_kv_heads + g for prefill.
 *  - Results are deterministic: identical inputs give bit-identical outputs.
 *  - Supported shapes: head_dim 64 or 128, idx_rank 16, page 64,
 *    G in {1, 2, 4, 8, 16}.
 */
#ifndef SA_H_
#define SA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size or parameter        */
  SA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (shape, dtype)   */
  SA_ERR_CAPACITY = 3,         /* cap below the worst-case support size      */
  SA_ERR_WORKSPACE = 4,        /* workspace missing or smaller than required */
  SA_ERR_HIP = 5               /* a HIP launch failed                        */
} sa_status;

typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

/* Host-side problem description. */
typedef struct {
  int32_t batch;        /* B sequences (1 for prefill)                          */
  int32_t n_q_heads;    /* H_q                                                  */
  int32_t n_kv_heads;   /* H_kv, divides H_q                                    */
  int32_t head_dim;     /* d                                                    */
  int32_t idx_rank;     /* r of the indexer projection                          */
  int32_t page_size;    /* tokens per page                                      */
  int32_t max_pages;    /* columns of page_table                                */
  int32_t max_len;      /* host bound on seq_lens[b]; <= max_pages * page_size  */
  int64_t n_pool_pages; /* pages in every pool                                  */
} sa_shape;

/* Device-side paging of the caches. */
typedef struct {
  const int32_t* page_table; /* [batch][max_pages] */
  const int32_t* seq_lens;   /* [batch]; unused by the prefill calls */
} sa_pages;

/* Operation ids for sa_workspace_size(). */
typedef enum {
  SA_OP_INDEX_SCORES = 0,
  SA_OP_SELECT = 1,          /* param = max candidates per row (tokens or pages) */
  SA_OP_SPARSE_DECODE = 2,   /* param = cap of the support lists                 */
  SA_OP_PREFILL_SELECT = 3,  /* param = n_tokens of the prefill                  */
  SA_OP_DECODE_STEP = 4,     /* param = cap                                      */
  SA_OP_SPARSE_DECODE_RLA = 5, /* param = cap                                    */
  SA_OP_ATTENTION_MASS = 6,    /* param unused                                   */
  SA_OP_PREFILL_QUERY = 7,     /* param = cap                                    */
  SA_OP_PBS_IMPORTANCE = 8,    /* param = n_rows                                 */
  SA_OP_PBS_SELECT = 9,        /* param = k_blocks                               */
  SA_OP_PREFILL_ORACLE = 10,   /* param unused                                   */
  SA_OP_DECODE_STEP_PAGES = 11, /* param = cap                                   */
  SA_OP_DECODE_STEP_RLA = 12    /* param = cap                                   */
} sa_op;

/* Bytes of workspace the operation needs for this shape (0 if none).  A
 * workspace sized for the maximum over the operations a caller uses may be
 * shared by them (calls ordered on one stream). */
size_t sa_workspace_size(sa_op op, const sa_shape* shape, int64_t param);

/* ---------------------------------------------------------------------------
 * Cache maintenance (off the per-step path)
 * ------------------------------------------------------------------------- */

/* Indexer keys of newly appended tokens ("Full Attention Strikes Back",
 * method section 2: the low-rank projector acts on keys before RoPE):
 *   kidx_pool[slot[t] / page][g][slot[t] % page][:] = W_k[g]^T k_pre[t][g][:]
 * k_pre [T][n_kv_heads][head_dim], w_k [n_kv_heads][head_dim][idx_rank],
 * kidx_pool [n_pool_pages][n_kv_heads][page][idx_rank], all of dtype;
 * slot [T] int64 pool token rows (page id * page_size + slot in page).
 * fp32 accumulation, one rounding to dtype on store. */
sa_status sa_index_append(const sa_shape* shape, const void* k_pre, const void* w_k,
                          sa_dtype dtype, const int64_t* slot, int32_t T,
                          void* kidx_pool, hipStream_t stream);

/* Page statistics for the Taylor page score ("SPLA", section 2.1, diagonal
 * covariance): for each listed pool page and group, the mean and the
 * population variance (divide by n) over the first n_valid[i] tokens:
 *   stats_pool[pages[i]][g][0][:] = mean,  stats_pool[pages[i]][g][1][:] = var
 * k_pool [n_pool_pages][n_kv_heads][page][head_dim]; pages, n_valid [n] int32
 * (n_valid in [1, page]); stats_pool [n_pool_pages][n_kv_heads][2][head_dim];
 * k_pool and stats_pool of dtype.  fp32 accumulation (two passes). */
sa_status sa_page_stats(const sa_shape* shape, const void* k_pool, sa_dtype dtype,
                        const int32_t* pages, const int32_t* n_valid, int32_t n,
                        void* stats_pool, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Decode: indexer scores
 * ------------------------------------------------------------------------- */

/* Token indexer scores ("Full Attention Strikes Back", method section 2;
 * head-collapsed channel, "Oracle-Guided Sparse Prefill", section 2.2):
 *   q_c[b][g] = s_idx * mean_{h in g} W_q[h]^T q[b][h]
 *   x[(b * n_kv_heads + g) * ldx + j] = q_c[b][g] . Kidx[b][g][j],  j < seq_lens[b]
 * q [batch][n_q_heads][head_dim], w_q [n_q_heads][head_dim][idx_rank],
 * kidx_pool [n_pool_pages][n_kv_heads][page][idx_rank], all of dtype;
 * x fp32 with row stride ldx >= max_len (entries j >= seq_lens[b] untouched).
 * fp32 arithmetic. */
sa_status sa_index_scores(const sa_shape* shape, const sa_pages* pages, const void* q,
                          const void* w_q, const void* kidx_pool, sa_dtype dtype,
                          float s_idx, float* x, int64_t ldx, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Taylor page scores ("SPLA", section 2.1): for page p of sequence b with
 * n = min(page, seq_lens[b] - p * page) valid tokens, q'_h = s_att * q[b][h]:
 *   x[(b * n_kv_heads + g) * ldx + p] =
 *       mean_{h in g} [ q'_h . mean_p + log(1 + 0.5 * sum_i q'_{h,i}^2 var_{p,i}) ]
 *       + log(n / page)
 * (the log of exp(q.kbar)(1 + q^T diag(var) q / 2), averaged over the group's
 * heads; the last term keeps a partial page's estimate of its total mass).
 * q [batch][n_q_heads][head_dim] and stats_pool of dtype; x fp32, ldx >=
 * max_pages. */
sa_status sa_page_scores(const sa_shape* shape, const sa_pages* pages, const void* q,
                         const void* stats_pool, sa_dtype dtype, float s_att, float* x,
                         int64_t ldx, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Support selection (sort-free histogram threshold)
 * ------------------------------------------------------------------------- */

/* Dynamic top-p support ("Full Attention Strikes Back", method sections 3 and
 * 5) over the token scores x (rows b * n_kv_heads + g, stride ldx, n = seq_lens[b]
 * candidates): with masses P_j = exp(x_j - max x) / sum exp(x - max x), rank
 * the candidates by (x descending, index ascending) and keep the shortest
 * prefix whose mass reaches p (>= p); p >= 1 keeps all.  The sink tokens
 * [0, n_sink) and the window [n - n_window, n) are then added (attention sink
 * and sliding window, method section 1).  Output: idx[row][cap] ascending,
 * -1 padded; count[row].  cap >= max_len.  The threshold is found by a radix
 * histogram over order-preserving keys of the fp32 scores, with masses summed
 * in 2^-40 fixed point, so the result does not depend on scheduling. */
sa_status sa_select_topp(const sa_shape* shape, const sa_pages* pages, const float* x,
                         int64_t ldx, float p, int32_t n_sink, int32_t n_window,
                         int32_t* idx, int32_t* count, int32_t cap, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* Static top-k support ("Full Attention Strikes Back", method section 3;
 * "Oracle-Guided Sparse Prefill", section 2.2): the first min(k, n) candidates
 * of the same ranking.  unit = 1: candidates are tokens (n = seq_lens[b]), and
 * the sink/window tokens are added as for top-p; cap >= min(k, max_len) +
 * n_sink + n_window (or max_len if smaller).  unit = page_size: candidates are
 * pages (n = ceil(seq_lens[b] / page)), each selected page expands to its
 * tokens; n_sink and n_window must be 0; cap >= k * page_size (or max_len if
 * smaller). */
sa_status sa_select_topk(const sa_shape* shape, const sa_pages* pages, const float* x,
                         int64_t ldx, int32_t k, int32_t unit, int32_t n_sink,
                         int32_t n_window, int32_t* idx, int32_t* count, int32_t cap,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Decode: exact attention over the support
 * ------------------------------------------------------------------------- */

/* Split-KV sparse decode ("Oracle-Guided Sparse Prefill", section 2.1:
 * attention recomputed with the original q, k, v restricted to the support):
 * for every query head h of group g of sequence b, over the listed tokens
 * S = idx[b * n_kv_heads + g][0 .. count)
 *   out[b][h] = sum_{j in S} softmax_S(s_att * q[b][h] . k_j) v_j
 *   lse[b][h] = log sum_{j in S} exp(s_att * q[b][h] . k_j)   (lse may be NULL)
 * An empty support gives out = 0 and lse = -inf.  batch * n_kv_heads <= 4096.
 * q, k_pool, v_pool of dtype;
 * out [batch][n_q_heads][head_dim] of out_dtype; lse fp32.  List entries must
 * be in [0, seq_lens[b]).  fp32 accumulation. */
sa_status sa_sparse_decode(const sa_shape* shape, const sa_pages* pages, const void* q,
                           const void* k_pool, const void* v_pool, sa_dtype dtype,
                           const int32_t* idx, const int32_t* count, int32_t cap,
                           float s_att, void* out, sa_dtype out_dtype, float* lse,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Residual linear attention state ("SPLA", section 2.2: the tokens left out
 * of the support are condensed into a linear-attention state; feature map
 * phi(x) = exp(x) elementwise, applied to the raw key rows): for each sequence
 * b and group g, over tokens j in [first_token, seq_lens[b]),
 *   state[b][g][i][c] += sum_j exp(k_j[i]) v_j[c]   (i, c < head_dim)
 *   state[b][g][head_dim][i] += sum_j exp(k_j[i])
 * state [batch][n_kv_heads][head_dim + 1][head_dim] fp32, accumulated in
 * place (the caller zero-fills it for a fresh build and passes the first new
 * token to extend it); k_pool, v_pool of dtype.  Cache maintenance, off the
 * per-step path.  Deterministic (one owner per state element, fixed order). */
sa_status sa_rla_state(const sa_shape* shape, const sa_pages* pages, const void* k_pool,
                       const void* v_pool, sa_dtype dtype, int32_t first_token, float* state,
                       hipStream_t stream);

/* sa_sparse_decode plus the residual linear attention over the tokens NOT in
 * the support ("SPLA", section 2.2, subtraction form: the global state's term
 * minus the listed tokens' terms, computed from the K/V rows the exact
 * attention already loads, so unlisted rows are never read):
 *   rla_num[b][h][:] = phi(q)^T S[b][g] - sum_{j in S} (phi(q) . phi(k_j)) v_j
 *   rla_den[b][h]    = phi(q) . z[b][g] - sum_{j in S}  phi(q) . phi(k_j)
 * with phi = exp elementwise on the raw q and k rows and (S, z) from
 * sa_rla_state over the whole sequence.  rla_num / rla_den is the linear
 * attention over the unlisted tokens (the learned gate and RMS norm the page
 * applies on top stay with the caller).  rla_state as written by
 * sa_rla_state; rla_num [batch][n_q_heads][head_dim] fp32, rla_den
 * [batch][n_q_heads] fp32.  Other arguments, outputs and limits as
 * sa_sparse_decode; workspace from SA_OP_SPARSE_DECODE_RLA. */
sa_status sa_sparse_decode_rla(const sa_shape* shape, const sa_pages* pages, const void* q,
                               const void* k_pool, const void* v_pool, sa_dtype dtype,
                               const int32_t* idx, const int32_t* count, int32_t cap,
                               float s_att, void* out, sa_dtype out_dtype, float* lse,
                               const float* rla_state, float* rla_num, float* rla_den,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* One whole decode step ("Full Attention Strikes Back", method sections 2, 3
 * and 5: low-rank indexer scores of every cached key, a dynamic top-p support
 * by a sort-free histogram threshold, sparse decode over it; "Oracle-Guided
 * Sparse Prefill", section 2.1: exact attention recomputed over the support):
 * sa_index_scores, then sa_select_topp (p in (0, 1]) or, if top_k > 0,
 * sa_select_topk with unit 1, then sa_sparse_decode.  The scores x
 * ([batch * n_kv_heads][ldx] fp32), idx and count are outputs too.  With few
 * rows (batch * n_kv_heads <= 16, group size >= 4) the step runs as one
 * persistent launch with the same scores, lists and counts as the three
 * calls and outputs equal within rounding (count[row] = -1 marks a row whose
 * barrier gave up, see the conventions above).  Workspace from
 * SA_OP_DECODE_STEP (param = cap); it holds the separate calls' regions and
 * the persistent launch's region side by side, so one workspace serves calls
 * that take either path. */
sa_status sa_decode_step(const sa_shape* shape, const sa_pages* pages, const void* q,
                         const void* w_q, const void* kidx_pool, const void* k_pool,
                         const void* v_pool, sa_dtype dtype, float s_idx, float s_att,
                         float p, int32_t top_k, int32_t n_sink, int32_t n_window,
                         float* x, int64_t ldx, int32_t* idx, int32_t* count, int32_t cap,
                         void* out, sa_dtype out_dtype, float* lse, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* sa_decode_step for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, results and kernels, minus the workspace.  Its scratch is
 * a 64 MiB array the library holds on each device it runs on until the
 * process ends (set up, and its zero-state part cleared by a fill kernel on
 * the given stream, by the first call on a device).  Shapes whose workspace
 * (SA_OP_DECODE_STEP) plus that zero-state part exceed it are rejected with
 * SA_ERR_WORKSPACE before anything is launched.  The call allocates nothing.
 * Every call on a device shares that device's scratch and leaves it as the
 * previous call's state: calls that overlap on one device (different
 * streams without ordering, or different host threads) race, so they must
 * be ordered like calls sharing a workspace. */
sa_status sa_decode_step_noalloc(const sa_shape* shape, const sa_pages* pages, const void* q,
                                 const void* w_q, const void* kidx_pool, const void* k_pool,
                                 const void* v_pool, sa_dtype dtype, float s_idx, float s_att,
                                 float p, int32_t top_k, int32_t n_sink, int32_t n_window,
                                 float* x, int64_t ldx, int32_t* idx, int32_t* count, int32_t cap,
                                 void* out, sa_dtype out_dtype, float* lse, hipStream_t stream);

/* sa_decode_step plus the residual linear attention over the tokens left out
 * of the support ("SPLA", section 2.2, subtraction form), as
 * sa_sparse_decode_rla computes it: the same scores, lists and counts as
 * sa_decode_step and outputs equal within rounding (the attention may be
 * split over a different number of workgroups), and rla_num
 * [batch][n_q_heads][head_dim],
 * rla_den [batch][n_q_heads] (fp32) from rla_state as written by
 * sa_rla_state over the whole sequence.  The persistent launch (few rows,
 * bf16) forms the listed tokens' terms from the K/V tiles its attention
 * already holds in LDS; otherwise the step ends with sa_sparse_decode_rla.
 * Workspace from SA_OP_DECODE_STEP_RLA (param = cap): the SA_OP_DECODE_STEP
 * layout followed by the residual terms' partial sums, so one workspace of
 * this size also serves sa_decode_step calls. */
sa_status sa_decode_step_rla(const sa_shape* shape, const sa_pages* pages, const void* q,
                             const void* w_q, const void* kidx_pool, const void* k_pool,
                             const void* v_pool, sa_dtype dtype, float s_idx, float s_att,
                             float p, int32_t top_k, int32_t n_sink, int32_t n_window,
                             float* x, int64_t ldx, int32_t* idx, int32_t* count, int32_t cap,
                             void* out, sa_dtype out_dtype, float* lse, const float* rla_state,
                             float* rla_num, float* rla_den, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* One whole page-level decode step ("SPLA", section 2.1: pages ranked by the
 * Taylor score, the top_k pages attended exactly): sa_page_scores, then
 * sa_select_topk with unit = page_size (n_sink = n_window = 0), then
 * sa_sparse_decode, with the same results as those three calls.  The page
 * scores x ([batch * n_kv_heads][ldx] fp32, ldx >= max_pages), idx and count
 * are outputs too; cap >= min(top_k * page_size, max_len).  stats_pool as
 * written by sa_page_stats; q, stats_pool, k_pool, v_pool of dtype.  With few
 * rows (batch * n_kv_heads <= 16, group size >= 4, top_k <= 32, bf16) the step
 * runs as one persistent launch whose workgroups meet at bounded in-memory
 * barriers; otherwise as the three launches.  Workspace from
 * SA_OP_DECODE_STEP_PAGES (param = cap). */
sa_status sa_decode_step_pages(const sa_shape* shape, const sa_pages* pages, const void* q,
                               const void* stats_pool, const void* k_pool, const void* v_pool,
                               sa_dtype dtype, float s_att, int32_t top_k, float* x, int64_t ldx,
                               int32_t* idx, int32_t* count, int32_t cap, void* out,
                               sa_dtype out_dtype, float* lse, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Attention-mass oracle support and coverage
 * ------------------------------------------------------------------------- */

/* Dense head-averaged attention mass ("Oracle-Guided Sparse Prefill",
 * section 2.1: the oracle takes the full attention distribution of each query
 * head and averages it over the heads into one token-importance distribution
 * P): for each sequence b and group g, row = b * n_kv_heads + g, and every
 * token j < seq_lens[b],
 *   x[row][j] = ln( (1/G) sum_{h in g} softmax_j(s_att * q[b][h] . k_j) )
 * (natural log, fp32; entries j >= seq_lens[b] are not written).  Since the
 * softmax of x is P itself and x orders tokens as P does, sa_select_topk on x
 * returns the attention-mass top-k oracle support and sa_select_topp on x the
 * shortest prefix by mass that reaches p.  q [batch][n_q_heads][head_dim],
 * k_pool of dtype; x [batch * n_kv_heads][ldx], ldx >= max_len;
 * batch * n_kv_heads <= 4096; workspace from SA_OP_ATTENTION_MASS, which
 * needs no zero-fill but is left holding the logits (an exception to the
 * zeroing convention: do not share it with the other calls' workspaces).
 * Reads every cached key: an instrument and reference policy, not a
 * sparse step.  fp32 logits and accumulation; deterministic. */
sa_status sa_attention_mass(const sa_shape* shape, const sa_pages* pages, const void* q,
                            const void* k_pool, sa_dtype dtype, float s_att, float* x,
                            int64_t ldx, void* ws, size_t ws_bytes, hipStream_t stream);

/* Coverage of a support under the attention mass ("Oracle-Guided Sparse
 * Prefill", section 2.1, and "Full Attention Strikes Back", results: the
 * attention mass a sparse support keeps): for each row,
 *   mass[row]    = sum_{j in S} exp(x[row][j])     S = idx[row][0 .. count)
 *   overlap[row] = | S  intersect  R |             R = ref_idx[row][0 .. ref_count)
 * with x as written by sa_attention_mass.  List entries outside
 * [0, seq_lens[b]) are skipped; lists as the selection calls write them
 * (strictly ascending).  ref_idx may be NULL (then ref_count, overlap are
 * ignored and may be NULL).  mass [batch * n_kv_heads] fp32, overlap int32.
 * fp32 sums in a fixed order (deterministic). */
sa_status sa_support_coverage(const sa_shape* shape, const sa_pages* pages, const float* x,
                              int64_t ldx, const int32_t* idx, const int32_t* count, int32_t cap,
                              const int32_t* ref_idx, const int32_t* ref_count, int32_t ref_cap,
                              float* mass, int32_t* overlap, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Causal prefill with supports shared by blocks of b_sel queries
 * ------------------------------------------------------------------------- */

/* Prefill supports ("Oracle-Guided Sparse Prefill", sections 2.1 and 2.2:
 * one support per selection block of b_sel queries, b_sel = 64, or per query,
 * b_sel = 1).  b_sel = 64: for query block blk = rows
 * [blk * b_sel, min(n_tokens, (blk + 1) * b_sel)) and group g,
 *   q_c = s_idx * mean_{i in blk, h in g} W_q[h]^T q[i][h]
 * scores x_j = q_c . Kidx[g][j] over the keys of earlier blocks,
 * j < blk * b_sel, and keeps the top k of them (all when there are at most k)
 * ranked as in sa_select_topk.  Output idx[blk * n_kv_heads + g][cap]
 * ascending, -1 padded, count likewise; cap >= min(k, n_tokens).  The block's
 * own keys are not listed: sa_sparse_prefill always attends to them causally.
 * b_sel = 1 (per query, the rule of a decode step on the prefix): row
 * i * n_kv_heads + g keeps the top k of x_j = q_c(i) . Kidx[g][j] over
 * j <= i, q_c(i) = s_idx * mean_{h in g} W_q[h]^T q[i][h], plus the query's
 * own token i, which is always listed; cap >= min(k + 1, n_tokens); the lists
 * feed sa_sparse_prefill_query.
 * q [n_tokens][n_q_heads][head_dim], w_q, kidx_pool of dtype; page_table row 0
 * of pages maps the single sequence; workspace from SA_OP_PREFILL_SELECT
 * (param = n_tokens): for 64-query blocks it holds fp32 score rows for up to
 * 2048 blocks at once (one slab for a 128K prefill, about 8.6 GB with 8
 * key/value heads), so that each selection kernel runs as one launch. */
sa_status sa_select_prefill_topk(const sa_shape* shape, const sa_pages* pages,
                                 int32_t n_tokens, const void* q, const void* w_q,
                                 const void* kidx_pool, sa_dtype dtype, float s_idx,
                                 int32_t b_sel, int32_t k, int32_t* idx, int32_t* count,
                                 int32_t cap, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Per-query supports ranked by the mean of the heads' probabilities (the
 * aggregation the oracle of "Oracle-Guided Sparse Prefill", section 2.1,
 * uses, applied to the low-rank channels instead of the head-collapsed one):
 * b_sel must be 1; for query i and group g, each head h in g scores
 * x_hj = s_idx * (W_q[h]^T q[i][h]) . Kidx[g][j] over j <= i, and the
 * candidates are ranked by P_j = mean_h softmax_j(x_hj) (ties lower index
 * first); the top k plus the own token are listed as for
 * sa_select_prefill_topk with b_sel = 1.  Same arguments, outputs and
 * workspace. */
sa_status sa_select_prefill_topk_probs(const sa_shape* shape, const sa_pages* pages,
                                       int32_t n_tokens, const void* q, const void* w_q,
                                       const void* kidx_pool, sa_dtype dtype, float s_idx,
                                       int32_t b_sel, int32_t k, int32_t* idx, int32_t* count,
                                       int32_t cap, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* Per-query sparse prefill attention ("Oracle-Guided Sparse Prefill",
 * section 2.1, per-query granularity): query i, head h of group g attends to
 * the listed keys S = idx[i * n_kv_heads + g][0 .. count) only (lists from
 * sa_select_prefill_topk with b_sel = 1 hold the query's own token):
 *   out[i][h] = sum_{j in S} softmax_S(s_att * q[i][h] . k_j) v_j,  lse likewise.
 * List entries must be in [0, i].  The group's heads share every gathered
 * K/V row (split-KV kernels of sa_sparse_decode, each query a sequence of
 * length i + 1 on page-table row 0).  q [n_tokens][n_q_heads][head_dim],
 * k_pool, v_pool of dtype; out of out_dtype; lse fp32 or NULL; workspace from
 * SA_OP_PREFILL_QUERY (param = cap, sized for n_tokens = max_len). */
sa_status sa_sparse_prefill_query(const sa_shape* shape, const sa_pages* pages,
                                  int32_t n_tokens, const void* q, const void* k_pool,
                                  const void* v_pool, sa_dtype dtype, const int32_t* idx,
                                  const int32_t* count, int32_t cap, float s_att, void* out,
                                  sa_dtype out_dtype, float* lse, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* Attention-mass oracle supports for prefill ("Oracle-Guided Sparse Prefill",
 * section 2.1: the full causal attention distribution of each query,
 * averaged over the group's heads, and its top k, per query or shared by a
 * selection block).  b_sel = 1: row i * n_kv_heads + g lists the top k of
 * P_i(j) = mean_{h in g} softmax_{j' <= i}(s_att * q[i][h] . k_j')[j] over
 * j <= i plus the query's own token (cap >= min(k + 1, n_tokens); lists for
 * sa_sparse_prefill_query).  b_sel = 64: row blk * n_kv_heads + g lists the
 * top k over the keys of earlier blocks j < 64 blk of the mean of P_i over
 * the block's queries i (cap >= min(k, n_tokens); lists for
 * sa_sparse_prefill, which adds the block's own keys causally).  Ties lower
 * index first; lists ascending, -1 padded.  Reads every causal key for every
 * query: an instrument and reference, not a sparse step.  q, k_pool of
 * dtype; n_kv_heads <= 64; workspace from SA_OP_PREFILL_ORACLE (sized for
 * n_tokens = max_len; needs no zero-fill, left holding intermediate values,
 * so not shared with the zeroed workspaces of other calls). */
sa_status sa_select_prefill_oracle(const sa_shape* shape, const sa_pages* pages,
                                  int32_t n_tokens, const void* q, const void* k_pool,
                                  sa_dtype dtype, float s_att, int32_t b_sel, int32_t k,
                                  int32_t* idx, int32_t* count, int32_t cap, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* Segment-permuted block selection ("Sparser Block-Sparse Attention via Token
 * Permutation", sections 2 to 4), three calls whose lists feed
 * sa_sparse_prefill.
 *
 * Key importance (section 3: estimated from the last query block): with
 * first = n_tokens - n_rows, for every group g and key j,
 *   importance[g][j] = mean over rows i < n_rows and heads h in g of
 *                      softmax_{j' <= first + i}(s_att * q[first + i][h] . k_j')[j]
 * (zero where j > first + i).  importance [n_kv_heads][n_tokens] fp32;
 * n_rows * n_kv_heads <= 4096; workspace from SA_OP_PBS_IMPORTANCE
 * (param = n_rows, sized for n_tokens = max_len; it needs no zero-fill and is
 * left holding intermediate values, so it is not shared with the zeroed
 * workspaces of the other calls).  q, k_pool of dtype. */
sa_status sa_pbs_importance(const sa_shape* shape, const sa_pages* pages, int32_t n_tokens,
                            const void* q, const void* k_pool, sa_dtype dtype, float s_att,
                            int32_t n_rows, float* importance, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Segment permutation (sections 2 and 3): inside every segment
 * [s * seg, (s + 1) * seg) of every group the positions are ordered by
 * importance, largest first (equal values: lower position first):
 * perm[g][p] = position of the key placed at p; no key leaves its segment.
 * seg a multiple of 64 in [64, 4096]; perm [n_kv_heads][n_tokens] int32.
 * No workspace. */
sa_status sa_pbs_permutation(const sa_shape* shape, const float* importance, int32_t n_tokens,
                             int32_t seg, int32_t* perm, hipStream_t stream);

/* Block selection on the permuted keys (section 4: mean pooling): query
 * block blk (rows [64 blk, 64 blk + 64)) and group g score each earlier key
 * block c < blk by qbar . kbar_c, qbar = mean of q over the block's rows and
 * the group's heads, kbar_c = mean of the 64 keys of block c, where block c
 * of a segment before the query block's own segment is taken in the
 * permuted order (keys perm[g][64 c .. 64 c + 63]) and a block of the own
 * segment in natural order; the top k_blocks blocks (ties lower block first)
 * are expanded to key lists idx[blk * n_kv_heads + g][cap] (block order,
 * the permuted order inside a block; not sorted), count = 64 * blocks,
 * cap >= 64 * min(k_blocks, blk); the own block is attended causally by
 * sa_sparse_prefill on top.  b_sel must be 64; perm as written by
 * sa_pbs_permutation (or any per-segment permutation); workspace from
 * SA_OP_PBS_SELECT (param = k_blocks, sized for n_tokens = max_len). */
sa_status sa_pbs_select(const sa_shape* shape, const sa_pages* pages, int32_t n_tokens,
                        const void* q, const void* k_pool, sa_dtype dtype, const int32_t* perm,
                        int32_t seg, int32_t b_sel, int32_t k_blocks, int32_t* idx,
                        int32_t* count, int32_t cap, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Block-sparse causal prefill attention ("Oracle-Guided Sparse Prefill",
 * section 2.1): row i of block blk, head h of group g attends to the listed
 * keys S = idx[blk * n_kv_heads + g][0 .. count) plus the block's own keys
 * j in [blk * b_sel, i]:
 *   out[i][h] = sum_j softmax(s_att * q[i][h] . k_j) v_j,  lse[i][h] likewise.
 * Listed keys must precede the block.  q [n_tokens][n_q_heads][head_dim],
 * k_pool, v_pool of dtype (SA_BF16 only); out [n_tokens][n_q_heads][head_dim]
 * of out_dtype; lse [n_tokens][n_q_heads] fp32 or NULL.  b_sel must be 64,
 * head_dim 128, cap <= 2048.
 * bf16 matrix-core products with fp32 accumulation and fp32 softmax. */
sa_status sa_sparse_prefill(const sa_shape* shape, const sa_pages* pages, int32_t n_tokens,
                            const void* q, const void* k_pool, const void* v_pool,
                            sa_dtype dtype, const int32_t* idx, const int32_t* count,
                            int32_t cap, int32_t b_sel, float s_att, void* out,
                            sa_dtype out_dtype, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Diagnostics
 * ------------------------------------------------------------------------- */

/* Static name of a status code. */
const char* sa_status_string(sa_status status);

/* Message of the last non-OK return on the calling thread ("" if none). */
const char* sa_last_error(void);

/* Library version string. */
const char* sa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SA_H_ */
