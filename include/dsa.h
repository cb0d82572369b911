/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek Sparse Attention forward path.
 *
 * The method (sources cited by page title, then section/equation):
 *  [P1] "DeepSeek-V3.2" release thread with a technical-report walk-through
 *       (freezhihu.org question 1978819912970555965)
 *       §2.1.1 Lightning Indexer: index score
 *              I_{t,s} = sum_j w^I_{t,j} ReLU(q^I_{t,j} . k^I_s), few heads, FP8;
 *       §2.1.2 Fine-grained token selection: keep the top-k scored KV entries
 *              per query token and attend over them only (O(L^2) -> O(Lk));
 *       §2.2   DSA instantiated in MLA, MQA mode: every latent KV entry is
 *              shared by all query heads of the token;
 *       §2.3.2 k = 2048 selected KV tokens per query token.
 *  [P2] "DeepSeek v3.2" analysis article (2048ai.net) §1.2: the indexer key is
 *       one 128-dim vector per token, evaluated in FP8, ReLU for throughput.
 *
 * Conventions shared by every call
 *  - Pointers are DEVICE pointers unless stated otherwise.  The caller owns
 *    and allocates every buffer; the library never allocates device memory
 *    at run time and keeps no per-call state (the one exception is the
 *    static scratch of dsa_forward_decode_paged_noalloc, below).  `stream` is
 *    a hipStream_t (NULL = default).
 *  - Calls are asynchronous and ordered on `stream`.  Inputs are read only;
 *    outputs are fully overwritten (including -1 / -inf padding).
 *  - Arguments are validated on the host before any launch.  On failure the
 *    call returns a status != DSA_OK, launches nothing and touches no output;
 *    dsa_last_error_message() then describes the problem (thread-local).
 *  - Launch failures map to DSA_ERR_HIP.  Faults inside kernels surface at
 *    the caller's next synchronisation.
 *  - Element types: FP8 = OCP E4M3FN bytes (unit scale); bf16 = raw 16-bit
 *    patterns in uint16_t; scores, weights, outputs are IEEE fp32.
 *  - Supported shapes: d_I = 128, 1 <= H_I <= 64, 1 <= H <= 128,
 *    D_qk = 576, D_v = 512, 1 <= k <= 4096, page_size = 64.  Every pointer
 *    must be 16-byte aligned.
 *  - Positions: query row t of a prefill call sits at position q_pos0 + t and
 *    its candidates are the keys s <= q_pos0 + t (itself included), capped at
 *    N.  A decode query of sequence b sits at position ctx_len[b] - 1 and its
 *    candidates are s = 0 .. ctx_len[b] - 1 (its own key is already cached).
 *  - Selected indices are token positions (logical positions in paged
 *    layouts), ascending, padded with -1 when fewer than k candidates exist.
 *    Equal scores are broken toward the lower position.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,         /* null pointer, bad shape, misalignment */
  DSA_ERR_UNSUPPORTED = 2,         /* valid but outside the supported shapes */
  DSA_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes below the *_workspace_bytes query */
  DSA_ERR_HIP = 4                  /* a HIP runtime call or launch failed */
} dsa_status;

typedef void* dsa_stream_t; /* hipStream_t */

/* Version of this ABI (bumped on any signature change). */
int32_t dsa_abi_version(void);
/* Static description of a status code: any integer is accepted, codes that
 * are not a dsa_status give "unknown status". */
const char* dsa_status_string(int32_t status);
/* Detail of the last failure on the calling thread ("" if none). */
const char* dsa_last_error_message(void);

/* Launch timing (a measurement aid; off by default).  After
 * dsa_timing_begin(), every call below made on the same host thread brackets
 * each of its kernel stages with two HIP events recorded on the stream the
 * stage is launched on; dsa_timing_end() stops recording, waits for the
 * recorded events and writes, for each stage kind i < n_kinds, the summed
 * durations ms[i] (milliseconds) and the number of launches[i].  A stage is
 * one kernel, except that the attention stage includes the split combine and
 * the multi-workgroup decode top-k is its three kernels.  The events add a
 * few microseconds per launch.  n_kinds may be 0 (just stop); otherwise ms
 * and launches are host arrays of n_kinds entries.  dsa_timing_begin() drops
 * any record still pending on the thread.  Errors: DSA_ERR_INVALID_ARG for a
 * bad n_kinds or NULL array, DSA_ERR_HIP when an event failed (the other
 * records are still summed). */
enum {
  DSA_KERNEL_INDEXER = 0,    /* lightning-indexer scores (prefill and decode) */
  DSA_KERNEL_TOPK = 1,       /* per-row top-k */
  DSA_KERNEL_ATTENTION = 2,  /* sparse MLA-MQA attention (+ split combine) */
  DSA_KERNEL_INDEXER_KL = 3, /* indexer KL loss (sparse training stage) */
  DSA_KERNEL_DENSE_KL = 4,   /* indexer KL loss (dense warm-up stage) */
  DSA_KERNEL_MLA_BWD_DQ = 5, /* attention backward: dq, P and dS */
  DSA_KERNEL_MLA_BWD_DKV = 6,/* attention backward: per-entry dkv addends */
  DSA_KERNEL_MLA_BWD_REDUCE = 7, /* attention backward: addends summed per cache row */
  DSA_KERNEL_KINDS = 8
};
dsa_status dsa_timing_begin(void);
dsa_status dsa_timing_end(double* ms, int64_t* launches, int32_t n_kinds);

/* ---------------------------------------------------------------------------
 * Lightning-indexer scores, [P1] §2.1.1 (index-score equation).
 *   q_idx  [T, H_I, d_I] FP8   query-side indexer vectors q^I_{t,j}
 *   w      [T, H_I]      fp32  per-head weights w^I_{t,j} (any sign)
 *   k_idx  [N, d_I]      FP8   indexer key of each token s
 *   scores [T, ld]       fp32  out: scores[t*ld + s] = I_{t,s} for candidate s
 *                              (s <= q_pos0 + t, s < N); -inf for 0 <= s < N
 *                              that are not candidates.  ld >= N.
 * Products are exact; sums are fp32 (relative error ~1e-6).
 */
dsa_status dsa_indexer_scores(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t T,
                              int64_t N, int32_t H_I, int32_t d_I, int64_t q_pos0, float* scores, int64_t ld,
                              dsa_stream_t stream);

/* Indexer scores of B decode queries over paged indexer keys (same equation).
 *   q_idx [B, H_I, d_I], w [B, H_I]
 *   k_pool     [n_pages, page_size, d_I] FP8 pool of indexer keys
 *   page_table [B, max_pages] int32: physical page of logical page p of seq b
 *   ctx_len    [B] int32 (device), 1 <= ctx_len[b] <= max_ctx <= max_pages*page_size
 *   scores     [B, ld] fp32 out, ld >= max_ctx: scores[b*ld + s] for s < ctx_len[b],
 *              -inf for ctx_len[b] <= s < max_ctx.
 * Token s of sequence b is row page_table[b][s / page_size]*page_size + s % page_size
 * of the pool; a page id outside [0, n_pages) reads as a non-candidate (-inf).
 */
dsa_status dsa_indexer_scores_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_pool,
                                    int64_t n_pages, const int32_t* page_table, int32_t max_pages,
                                    const int32_t* ctx_len, int32_t page_size, int64_t B, int32_t H_I,
                                    int32_t d_I, int64_t max_ctx, float* scores, int64_t ld,
                                    dsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Per-row top-k selection, [P1] §2.1.2.
 *   scores [T, ld] fp32 (finite values and -inf; NaN is undefined)
 *   n_valid: NULL -> row t has candidates s < min(q_pos0 + t + 1, N);
 *            else device int32 [T]: row t has candidates s < min(n_valid[t], N).
 *   idx [T, k] int32 out: the min(k, n_t) positions with the largest scores,
 *            ties to the lower position, ascending, then -1.  -0 equals +0.
 * Deterministic: the output is a function of the score values only.
 */
dsa_status dsa_topk(const float* scores, int64_t ld, int64_t T, int64_t N, int64_t q_pos0,
                    const int32_t* n_valid, int32_t k, int32_t* idx, dsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Sparse MLA attention in MQA mode, [P1] §2.1.2 (attention over the selected
 * entries) with §2.2 (one latent KV row shared by all heads).
 *   q   [T, H, D_qk] bf16  per-head query in the latent space (512 + 64 rope)
 *   kv  [N, D_qk]    bf16  latent KV rows; keys use all D_qk dims, values
 *                          the first D_v dims
 *   idx [T, k] int32       selected rows per query; entries < 0 or >= N skip
 *   out [T, H, D_v] fp32   out = sum_s softmax_s(scale * q.kv_s) kv_s[:D_v]
 *   lse [T, H] fp32        natural-log log-sum-exp of the scaled logits
 * A row with no valid entry yields out = 0 and lse = -inf.  Products are
 * bf16 x bf16 with fp32 accumulation; probabilities enter the value product
 * as bf16 (relative error ~2e-3).
 * ws: scratch for split-key partials when T is small; size from
 * dsa_sparse_mla_fwd_workspace_bytes (0 is valid when that returns 0).
 */
size_t dsa_sparse_mla_fwd_workspace_bytes(int64_t T, int32_t H, int32_t D_v, int32_t k);
dsa_status dsa_sparse_mla_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int64_t T,
                              int64_t N, int32_t H, int32_t D_qk, int32_t D_v, int32_t k, float scale,
                              float* out, float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream);

/* Same attention for B decode queries over a paged latent pool
 *   q [B, H, D_qk]; kv_pool [n_pages, page_size, D_qk]; page_table/ctx_len as above;
 *   idx [B, k] logical positions; entries < 0 or >= ctx_len[b] skip.
 */
size_t dsa_sparse_mla_fwd_paged_workspace_bytes(int64_t B, int32_t H, int32_t D_v, int32_t k);
dsa_status dsa_sparse_mla_fwd_paged(const uint16_t* q, const uint16_t* kv_pool, int64_t n_pages,
                                    const int32_t* page_table, int32_t max_pages, const int32_t* ctx_len,
                                    int32_t page_size, const int32_t* idx, int64_t B, int32_t H,
                                    int32_t D_qk, int32_t D_v, int32_t k, float scale, float* out,
                                    float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Backward of dsa_sparse_mla_fwd, for the sparse training stage of [P1]
 * §2.3.2 (the main model is trained through the sparse attention of §2.1.2 in
 * the MQA form of §2.2).  For each query t, head h and valid entry s of idx:
 *   P  = exp(scale * q[t,h] . kv[s] - lse[t,h]),   dP = dout[t,h] . kv[s][:D_v]
 *   dS = scale * P * (dP - dout[t,h] . out[t,h])
 *   dq[t,h] = sum_s dS kv[s]
 *   dkv[s]  = sum over (t, h) selecting s of  dS q[t,h] + P dout[t,h] (dims < D_v)
 *   q [T, H, D_qk] bf16, kv [N, D_qk] bf16, idx [T, k] int32 (entries < 0 or
 *   >= N skip; an index listed twice counts twice, as in the forward), out [T, H, D_v] fp32 and
 *   lse [T, H] fp32 as dsa_sparse_mla_fwd wrote them for the same inputs,
 *   dout [T, H, D_v] bf16 the upstream gradient.
 *   dq [T, H, D_qk] fp32 out (overwritten); dkv [N, D_qk] fp32 out (zeroed,
 *   then accumulated; rows no query selects are 0).
 * P and dS enter the gradient products as bf16 (relative error ~2^-9 per
 * term); products are bf16 x bf16 with fp32 accumulation.  Each (query,
 * entry) contribution to dkv is formed in fp32 and stored as a bf16 row
 * (rounded to nearest, 2^-9 relative); the rows of one cache row are summed
 * in fp32 in an order that may vary from call to call.
 * ws: P, dS and the contribution rows of a tile of up to 2048 queries plus
 * their grouping by cache row; size from
 * dsa_sparse_mla_bwd_workspace_bytes(T, N, H, k) (about 7 GB at k = 2048,
 * H = 128; DSA_ERR_WORKSPACE_TOO_SMALL below it).  N <= 2^30.  All pointers
 * are device memory owned by the caller.
 */
size_t dsa_sparse_mla_bwd_workspace_bytes(int64_t T, int64_t N, int32_t H, int32_t k);
dsa_status dsa_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* out,
                              const float* lse, const uint16_t* dout, int64_t T, int64_t N, int32_t H,
                              int32_t D_qk, int32_t D_v, int32_t k, float scale, float* dq, float* dkv,
                              void* ws, size_t ws_bytes, dsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Indexer KL loss of the sparse training stage, [P1] §2.3.2 (target built as
 * in §2.3.1: the attention scores of all heads summed, then L1-normalised
 * along the selected tokens).  For each query t, with S_t its valid entries
 * of idx:
 *   P_h(s) = exp(scale * q[t,h] . kv[s] - lse[t,h])   (head h's attention)
 *   p(s)   = (1/H) sum_h P_h(s),   r(s) = softmax over S_t of scores[t, s]
 *   kl[t]  = sum_{s in S_t} p(s) * (ln p(s) - ln r(s))
 * The loss is sum_t kl[t].
 *   q [T, H, D_qk] bf16, kv [N, D_qk] bf16, idx [T, k] int32 (entries < 0 or
 *   >= N skip), lse [T, H] fp32 as written by dsa_sparse_mla_fwd for the same
 *   q, kv and idx, scores [T, ld] fp32 with row t holding I[t, s] at column s
 *   (as dsa_indexer_scores writes it; only the selected columns are read),
 *   kl [T] fp32 out.  A row with no valid entry gives 0.
 * Logit products are bf16 x bf16 with fp32 accumulation; the rest is fp32.
 * No workspace; errors as for the other calls.
 */
dsa_status dsa_indexer_kl_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const float* lse,
                              const float* scores, int64_t ld, int64_t T, int64_t N, int32_t H, int32_t D_qk,
                              int32_t k, float scale, float* kl, dsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Indexer KL loss of the dense warm-up stage, [P1] §2.3.1: for each query t
 * at position q_pos0 + t, over every key s < n_t = min(q_pos0 + t + 1, N),
 *   z_h(s) = scale * q[t,h] . kv[s]   (all D_qk dims),
 *   lse_h  = ln sum_s exp(z_h(s))      (the dense attention's normaliser),
 *   p(s)   = (1/H) sum_h exp(z_h(s) - lse_h),   r(s) = softmax over the n_t keys of scores[t, s],
 *   kl[t]  = sum_s p(s) * (ln p(s) - ln r(s)).
 *   q [T, H, D_qk] bf16, kv [N, D_qk] bf16, scores [T, ld] fp32 (row t holds
 *   I[t, s] for s < n_t, as dsa_indexer_scores writes it; ld >= N), kl [T]
 *   fp32 out, lse [T, H] fp32 out (the dense lse_h; may be NULL).
 * Logit products are bf16 x bf16 with fp32 accumulation; the rest is fp32.
 * Cost: two passes of dense logits over all n_t keys per query (O(L^2)).
 */
dsa_status dsa_indexer_dense_kl_fwd(const uint16_t* q, const uint16_t* kv, const float* scores, int64_t ld,
                                    int64_t T, int64_t N, int64_t q_pos0, int32_t H, int32_t D_qk, float scale,
                                    float* kl, float* lse, dsa_stream_t stream);

/* The dense warm-up loss of one sequence fused: indexer scores over row tiles
 * (as dsa_forward_prefill tiles them, in a workspace score tile) and
 * dsa_indexer_dense_kl_fwd on each tile.  Inputs as in dsa_forward_prefill;
 * kl [T] and lse [T, H] (may be NULL) out.  The loss is sum_t kl[t]. */
size_t dsa_dense_warmup_loss_workspace_bytes(int64_t T, int64_t N);
dsa_status dsa_dense_warmup_loss(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const uint16_t* q,
                                 const uint16_t* kv, int64_t T, int64_t N, int32_t H_I, int32_t d_I, int32_t H,
                                 int32_t D_qk, int64_t q_pos0, float scale, float* kl, float* lse, void* ws,
                                 size_t ws_bytes, dsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Fused prefill of one sequence: the whole DSA chain of [P1] -- index scores
 * (§2.1.1 index-score equation), fine-grained top-k token selection and
 * attention over the selected latent entries (§2.1.2), MLA in MQA mode (§2.2)
 * -- for the T queries at positions q_pos0 .. q_pos0+T-1 over keys 0 .. N-1
 * (N >= q_pos0+T is not required; candidates are capped at N).  The L x L
 * score matrix is never formed: scores live in a row-tiled part of the
 * workspace.  The selection equals dsa_indexer_scores followed by dsa_topk
 * bit for bit: every causal pair is first scored on the FP8 matrix cores, and
 * every key whose place relative to its row's threshold that approximate
 * score leaves open (a bound on its error holds by construction) is rescored
 * with the exact arithmetic of dsa_indexer_scores.  The outputs are those of
 * dsa_sparse_mla_fwd over that selection.
 *   idx may be NULL (then kept in the workspace); otherwise [T, k] out.
 */
size_t dsa_forward_prefill_workspace_bytes(int64_t T, int64_t N, int32_t H, int32_t D_v, int32_t k);
dsa_status dsa_forward_prefill(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const uint16_t* q,
                               const uint16_t* kv, int64_t T, int64_t N, int32_t H_I, int32_t d_I, int32_t H,
                               int32_t D_qk, int32_t D_v, int32_t k, int64_t q_pos0, float scale,
                               int32_t* idx, float* out, float* lse, void* ws, size_t ws_bytes,
                               dsa_stream_t stream);

/* Row-tile plan of dsa_forward_prefill: the fused call runs the indexer and
 * top-k over consecutive row tiles of *tile_rows rows, using a score scratch of
 * row stride *score_ld (fp32) at the start of ws, then one sparse-attention
 * launch over all T rows.  Lets a caller replay the fused call stage by stage
 * with dsa_indexer_scores / dsa_topk / dsa_sparse_mla_fwd (e.g. to time each
 * kernel).  Host pointers; returns DSA_ERR_INVALID_ARG for T < 1 or N < 1. */
dsa_status dsa_forward_prefill_plan(int64_t T, int64_t N, int64_t* tile_rows, int64_t* score_ld);

/* Fused chunked prefill of B sequences over paged caches (64-token pages),
 * several sequences per call.  Sequence b holds ctx_len[b] tokens in the
 * pools (its new chunk already written there) and contributes the
 * n_b = q_start[b+1] - q_start[b] query rows q_start[b] .. q_start[b+1]-1,
 * which are its last n_b tokens: row q_start[b] + i is the query at position
 * p = ctx_len[b] - n_b + i.  Each query is the one of dsa_forward_prefill at
 * position p: the indexer scores keys 0..p of its own sequence, the top-k
 * keeps k of them (ties to the lower position, ascending, -1 padded) and the
 * attention runs over them.  A chunk with n_b == ctx_len[b] is a whole prompt;
 * n_b == 1 is a decode step.
 *   q_idx [total_q, H_I, d_I] FP8, w [total_q, H_I] fp32, q [total_q, H, D_qk]
 *   bf16, with total_q = q_start[B];
 *   k_pool [n_pages, page_size, d_I], kv_pool [n_pages, page_size, D_qk];
 *   page_table [B, max_pages] int32 (device): page j of sequence b, which must
 *   be a valid page for every j < ceil(ctx_len[b] / page_size);
 *   q_start [B+1] int64 and ctx_len [B] int64 are HOST arrays (they size the
 *   launches): q_start[0] == 0, non-decreasing, and
 *   n_b <= ctx_len[b] <= min(max_pages * page_size, 262144);
 *   idx [total_q, k] out (logical positions; may be NULL), out
 *   [total_q, H, D_v] fp32, lse [total_q, H] fp32.
 * The workspace query takes total_q and the largest ctx_len.  Sequences run
 * one after another on `stream`, each in row tiles as in dsa_forward_prefill.
 */
size_t dsa_forward_prefill_paged_workspace_bytes(int64_t total_q, int64_t max_ctx, int32_t H, int32_t D_v,
                                                 int32_t k);
dsa_status dsa_forward_prefill_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_pool,
                                     const uint16_t* q, const uint16_t* kv_pool, int64_t n_pages,
                                     const int32_t* page_table, int32_t max_pages, int32_t page_size,
                                     const int64_t* q_start, const int64_t* ctx_len, int64_t B, int32_t H_I,
                                     int32_t d_I, int32_t H, int32_t D_qk, int32_t D_v, int32_t k, float scale,
                                     int32_t* idx, float* out, float* lse, void* ws, size_t ws_bytes,
                                     dsa_stream_t stream);

/* Fused decode of B sequences with contiguous caches, one query each: the DSA
 * chain of [P1] §2.1.1 (index scores), §2.1.2 (top-k selection and attention
 * over the selected entries) and §2.2 (MQA mode) for the newest token of each
 * sequence, whose key is already in the cache:
 *   k_idx [B, N, d_I], kv [B, N, D_qk]; ctx_len [B] (device) with
 *   1 <= ctx_len[b] <= N.  Other arguments as in the calls above.  Scores are
 *   exact (the arithmetic of dsa_indexer_scores_paged); each query's entries
 *   may be split over several workgroups and merged exactly (same out/lse).
 */
size_t dsa_forward_decode_workspace_bytes(int64_t B, int64_t N, int32_t H, int32_t D_v, int32_t k);
dsa_status dsa_forward_decode(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, const uint16_t* q,
                              const uint16_t* kv, const int32_t* ctx_len, int64_t B, int64_t N, int32_t H_I,
                              int32_t d_I, int32_t H, int32_t D_qk, int32_t D_v, int32_t k, float scale,
                              int32_t* idx, float* out, float* lse, void* ws, size_t ws_bytes,
                              dsa_stream_t stream);

/* Fused decode of B sequences over paged caches (64-token pages): the chain
 * of dsa_forward_decode ([P1] §2.1.1, §2.1.2, §2.2) with every key and latent
 * row read through the page table (a serving layout; the pages do not fix
 * one):
 *   k_pool [n_pages, page_size, d_I], kv_pool [n_pages, page_size, D_qk],
 *   page_table [B, max_pages], ctx_len [B] with ctx_len[b] <= max_ctx <=
 *   max_pages * page_size.  Returned indices are logical positions.
 */
size_t dsa_forward_decode_paged_workspace_bytes(int64_t B, int64_t max_ctx, int32_t H, int32_t D_v,
                                                int32_t k);
dsa_status dsa_forward_decode_paged(const uint8_t* q_idx, const float* w, const uint8_t* k_pool,
                                    const uint16_t* q, const uint16_t* kv_pool, int64_t n_pages,
                                    const int32_t* page_table, int32_t max_pages, const int32_t* ctx_len,
                                    int32_t page_size, int64_t B, int64_t max_ctx, int32_t H_I, int32_t d_I,
                                    int32_t H, int32_t D_qk, int32_t D_v, int32_t k, float scale,
                                    int32_t* idx, float* out, float* lse, void* ws, size_t ws_bytes,
                                    dsa_stream_t stream);

/* dsa_forward_decode_paged without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments (less ws and
 * ws_bytes), validation and results, bit for bit.  Its scratch is one
 * 96 MiB array per GPU inside the library, held by each GPU the library runs
 * on until the process ends: a call needing more
 * (dsa_forward_decode_paged_workspace_bytes above 100663296 bytes; 32
 * sequences of up to 131072 tokens with H = 128 and k = 2048 need about
 * 52 MB) returns DSA_ERR_UNSUPPORTED before any launch.  The call allocates
 * nothing (no hipMalloc, no allocating library routine).  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams
 * or threads) race and give undefined results; calls ordered on one stream
 * are safe, and no part of the array needs clearing between them.
 */
dsa_status dsa_forward_decode_paged_noalloc(const uint8_t* q_idx, const float* w, const uint8_t* k_pool,
                                            const uint16_t* q, const uint16_t* kv_pool, int64_t n_pages,
                                            const int32_t* page_table, int32_t max_pages, const int32_t* ctx_len,
                                            int32_t page_size, int64_t B, int64_t max_ctx, int32_t H_I,
                                            int32_t d_I, int32_t H, int32_t D_qk, int32_t D_v, int32_t k,
                                            float scale, int32_t* idx, float* out, float* lse,
                                            dsa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
