/*
 * s3r.h - C ABI of the S3R (self-sparse speculative rollouts) attention and
 * sampling step on AMD Instinct MI355X (gfx950).
 *
 * One round of the method for a batch of sequences is four calls on one
 * stream:
 *   s3r_select              keep the newest window plus the positions the last
 *                           verification attended to most (budget s * L);
 *   s3r_sparse_decode_attn  one draft step: single-query attention over the
 *                           kept positions plus this round's positions
 *                           (called k times per round);
 *   s3r_verify_attn         dense attention of the k + 1 block queries over
 *                           the complete paged cache, causal inside the block;
 *                           also emits the next round's selector scores
 *                           (or s3r_verify_attn_deferred now and
 *                           s3r_verify_scores on another stream);
 *   s3r_spec_sample         exact speculative sampling: accept each draft with
 *                           probability min(1, p/q), else draw the correction
 *                           from the normalised residual max(0, p - q); a fully
 *                           accepted round adds a bonus token drawn from p.
 * Rounds are joined on the device by s3r_kv_append (new K/V rows into the
 * cache) and s3r_commit (lengths and pending token for the next round);
 * s3r_length_order gives the draft steps a dispatch order for batches of
 * mixed lengths.
 *
 * Sources (web pages about the method, cited by title and section):
 *   [news]      "Long-context RL training stops waiting on autoregressive
 *               rollouts: sparse self-drafting plus full-attention verification
 *               lifts throughput 1.39x" (ai4snews), Interpretation;
 *   [listing]   "S^3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative
 *               Decoding" (thelatestinai paper page), Abstract, Tables 4-7;
 *   [explainer] "S3R - Self-sparse speculative rollouts for RL - What does it
 *               mean?" (learnaivisually), Jargon and the mechanism paragraphs.
 *
 * Conventions shared by all calls
 *   - Every pointer argument is DEVICE memory owned by the caller, except the
 *     s3r_paged_kv descriptor itself, which is a HOST struct read during the
 *     call (its pointer members are device pointers). The library never
 *     allocates or frees memory and keeps no state between calls.
 *   - Calls are asynchronous on `stream`; a call returns after enqueuing its
 *     kernels. Outputs are valid once the stream reaches that point.
 *   - Per-sequence values live in device arrays; host scalars give the shape
 *     bounds (max_*, *_cap) used for validation, grid and workspace sizing.
 *     Device values beyond the host bounds are undefined behaviour.
 *   - The workspace of a call is caller memory of at least the size the
 *     matching *_workspace_bytes() returns; its content on entry does not
 *     matter and on exit is unspecified, except that s3r_verify_attn_deferred
 *     leaves in it what the following s3r_verify_scores reads. Concurrent
 *     calls must not share one.
 *   - Identical inputs give bit-identical outputs (no float atomics; fixed
 *     reduction orders).
 *   - Status codes: S3R_ERR_INVALID_ARG for null required pointers,
 *     non-positive sizes, Hq not a multiple of Hkv, k outside [0, 15],
 *     capacities smaller than the host bounds require, or an invalid budget
 *     ratio; S3R_ERR_UNSUPPORTED for page_size != 16, head_dim not 64 or 128,
 *     or shapes a kernel does not cover (listed per call); S3R_ERR_WORKSPACE
 *     for a workspace smaller than required; S3R_ERR_HIP when a kernel launch
 *     fails. On any error nothing is enqueued.
 *
 * Paged KV cache layout: k_pages and v_pages are
 * [num_pages][num_kv_heads][page_size][head_dim] in `dtype`; position j of
 * sequence b is slot j % page_size of physical page
 * block_table[b * max_pages_per_seq + j / page_size]. Query head h reads KV
 * head h / (Hq / Hkv) (grouped-query attention).
 */
#ifndef S3R_H
#define S3R_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  S3R_OK = 0,
  S3R_ERR_INVALID_ARG = 1,
  S3R_ERR_UNSUPPORTED = 2,
  S3R_ERR_WORKSPACE = 3,
  S3R_ERR_HIP = 4
} s3r_status;

typedef enum { S3R_F32 = 0, S3R_BF16 = 1 } s3r_dtype;

typedef struct {
  const void* k_pages;          /* device, [num_pages][num_kv_heads][page_size][head_dim] */
  const void* v_pages;          /* device, same layout as k_pages */
  const int32_t* block_table;   /* device, [B][max_pages_per_seq] physical page ids */
  int32_t num_pages;
  int32_t max_pages_per_seq;
  int32_t num_kv_heads;
  int32_t head_dim;             /* 64 or 128 */
  int32_t page_size;            /* 16 */
  int32_t dtype;                /* s3r_dtype of K, V and the queries */
} s3r_paged_kv;

/* Human-readable name of a status code (static string). */
const char* s3r_status_string(s3r_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t s3r_version(void);

/*
 * Selection budget for a context of L committed positions (host helper):
 * min(L, max(min(window, L), ceil(s_num * L / s_den))). [explainer], Jargon,
 * "Sparse attention budget": a fraction s of the cached positions (0.05 by
 * default) made of the newest positions plus the most attended ones; the
 * ratio is exact integers and the newest window counts inside the budget.
 * Returns -1 on invalid arguments (L < 0, s_den <= 0, s_num < 0,
 * s_num > s_den, window < 0). Use it to size nsel_cap from a host bound.
 */
int32_t s3r_budget(int32_t L, int32_t s_num, int32_t s_den, int32_t window);

/*
 * s3r_select - newest window plus top-scoring older positions, per (sequence,
 * KV head). [explainer], mechanism paragraph: the set the drafter reads is the
 * most recent positions together with those the previous verification pass
 * weighted most, chosen again at every round; [news], Interpretation: the
 * draft attends to a small subset of the cached entries, picked by score.
 *
 *   scores    device f32 [B][Hkv][score_stride]: score of position j of each
 *             (sequence, KV head); only j < ctx_len[b] is read. NaN scores are
 *             undefined behaviour; +inf ranks highest; -0.0 equals +0.0.
 *   ctx_len   device i32 [B]: committed context L_b, 1 <= L_b <= max_ctx_len.
 *   s_num/s_den, window: budget as in s3r_budget (0 <= s_num <= s_den).
 *   idx       device i32 [B][Hkv][nsel_cap] output: the n_sel[b] kept positions
 *             in ascending order (window [L_b - min(window, L_b), L_b) plus the
 *             top n_sel - window older positions by score, ties to the lower
 *             position). Entries at and beyond n_sel[b] are not written.
 *   n_sel     device i32 [B] output: s3r_budget(L_b, s_num, s_den, window).
 *   order     device i32 [B] output or NULL: the draft steps' dispatch order,
 *             as s3r_length_order(ctx_len) writes it (formed by the same launch).
 *   nsel_cap  >= s3r_budget(max_ctx_len, ...) (INVALID_ARG otherwise);
 *   score_stride >= max_ctx_len.
 * No workspace. UNSUPPORTED: none.
 */
s3r_status s3r_select(const float* scores, int32_t score_stride, const int32_t* ctx_len,
                      int32_t B, int32_t Hkv, int32_t max_ctx_len, int32_t s_num, int32_t s_den,
                      int32_t window, int32_t* idx, int32_t nsel_cap, int32_t* n_sel, int32_t* order,
                      hipStream_t stream);

/*
 * s3r_select_grouped - selection variants. [explainer], mechanism paragraph:
 * the kept set is described there as whole pages (recent ones plus those the
 * previous verification weighted most); [news], Perspective: choosing the
 * context adaptively is named as further work.
 *
 * Arguments as for s3r_select, plus:
 *   unit      1: single positions (the s3r_select rule);
 *             16: whole pages. The newest min(window, L) positions are kept as
 *             whole pages from page f = floor((L - min(window, L)) / 16) on
 *             (wc = L - 16 f positions); of the f full older pages, the
 *             min(f, ceil(max(0, n - wc) / 16)) with the largest float32 sum of
 *             their 16 scores (slot order) are kept, ties to the lower page,
 *             where n = s3r_budget(L, ...). Every KV head keeps
 *             n_sel[b] = wc + 16 x (pages kept) positions, ascending.
 *   all_heads 0: one kept set per KV head; 1: one kept set per sequence,
 *             chosen on the float32 sum of the KV heads' scores (heads in
 *             ascending order, before the page sum), written for every KV head.
 *   nsel_cap  >= s3r_select_grouped_capacity(max_ctx_len, s_num, s_den,
 *             window, unit) (INVALID_ARG otherwise).
 *   ws        workspace of s3r_select_grouped_workspace_bytes(...) bytes (none
 *             for unit 1 with all_heads 0, which is s3r_select).
 *   order     as for s3r_select (NULL: not written).
 * INVALID_ARG also for unit not in {1, 16}.
 */
int32_t s3r_select_grouped_capacity(int32_t max_ctx_len, int32_t s_num, int32_t s_den, int32_t window,
                                    int32_t unit);
size_t s3r_select_grouped_workspace_bytes(int32_t B, int32_t Hkv, int32_t max_ctx_len, int32_t s_num,
                                          int32_t s_den, int32_t window, int32_t unit, int32_t all_heads);
s3r_status s3r_select_grouped(const float* scores, int32_t score_stride, const int32_t* ctx_len, int32_t B,
                              int32_t Hkv, int32_t max_ctx_len, int32_t s_num, int32_t s_den, int32_t window,
                              int32_t unit, int32_t all_heads, int32_t* idx, int32_t nsel_cap, int32_t* n_sel,
                              int32_t* order, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * s3r_select_pages - the whole-page selection of s3r_select_grouped (unit 16)
 * from scores given per page, as s3r_verify_attn_pages writes them: the key of
 * candidate page p is page_scores[b][kv][p] (all_heads: the float32 sum over
 * the KV heads in ascending order) instead of the float32 sum of its 16
 * position scores. The window pages, the count of kept pages, the tie rule
 * and the output are those of s3r_select_grouped with unit 16.
 *
 *   page_scores device f32 [B][Hkv][page_stride]: only the candidate pages
 *             p < floor((L_b - min(window, L_b)) / 16) are read;
 *   page_stride >= ceil(max_ctx_len / 16);
 *   nsel_cap  >= s3r_select_grouped_capacity(max_ctx_len, s_num, s_den, window, 16);
 *   ws        s3r_select_grouped_workspace_bytes(B, Hkv, max_ctx_len, s_num,
 *             s_den, window, 16, all_heads) bytes.
 * Other arguments as for s3r_select_grouped.
 */
s3r_status s3r_select_pages(const float* page_scores, int32_t page_stride, const int32_t* ctx_len, int32_t B,
                            int32_t Hkv, int32_t max_ctx_len, int32_t s_num, int32_t s_den, int32_t window,
                            int32_t all_heads, int32_t* idx, int32_t nsel_cap, int32_t* n_sel, int32_t* order,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * s3r_sparse_decode_attn - one sparse draft step. [news], Interpretation:
 * drafting uses the policy's own weights and attends to the selected KV
 * entries; [explainer], mechanism paragraph: k quick draft steps over the
 * kept subset of the cache.
 *
 * For sequence b and query head h (KV head kv = h / (Hq / Hkv)) the attended
 * set is S = idx[b][kv][0 .. n_sel[b]) united with [sel_len[b], cur_len[b])
 * (this round's positions, the querying token's own included), and
 *   out[b][h] = softmax(scale * q[b][h] . K_S) V_S,
 *   lse[b][h] = log sum_S exp(scale * q[b][h] . K_j)  (natural log).
 * An empty S gives out = 0 and lse = -inf.
 *
 *   q         device [B][Hq][head_dim] in kv->dtype.
 *   idx, nsel_cap, n_sel: as written by s3r_select (positions < sel_len[b]).
 *   sel_len   device i32 [B]: L_b, the context length the selection used.
 *   cur_len   device i32 [B]: L_b + j at draft step j (1..k); K/V of positions
 *             [L_b, cur_len) must already be in the cache.
 *   order     device i32 [B] or NULL: a permutation of 0..B-1, the order in
 *             which workgroups take the sequences (NULL: 0..B-1). It changes
 *             when each sequence is computed, never a result. Entries outside
 *             [0, B) are skipped (their sequence is not computed); a repeated
 *             entry computes that sequence twice, identically. s3r_length_order
 *             writes the order that takes long contexts first, which keeps
 *             workgroups of similar length together on batches of mixed
 *             lengths.
 *   max_attend host bound on n_sel[b] + cur_len[b] - sel_len[b] (>= 1).
 *   out       device f32 [B][Hq][head_dim]; lse device f32 [B][Hq] or NULL.
 *   ws        workspace of s3r_sparse_decode_workspace_bytes(B, Hq, head_dim,
 *             max_attend) bytes.
 * UNSUPPORTED: Hq / Hkv > 16 (bf16, head_dim 128) or Hq / Hkv not in {1, 2, 4, 8}
 * (other dtype / head_dim combinations).
 */
size_t s3r_sparse_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t head_dim, int32_t max_attend);
s3r_status s3r_sparse_decode_attn(const void* q, const s3r_paged_kv* kv, const int32_t* idx,
                                  int32_t nsel_cap, const int32_t* n_sel, const int32_t* sel_len,
                                  const int32_t* cur_len, const int32_t* order, int32_t B, int32_t Hq,
                                  float scale, int32_t max_attend, float* out, float* lse, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/*
 * s3r_length_order - the dispatch order for s3r_sparse_decode_attn: order[r]
 * is the sequence of rank r when the sequences are sorted by descending
 * len[b], ties by ascending b (a stable sort). Not part of the method's
 * arithmetic: it only arranges when each sequence's workgroups run.
 * s3r_select, s3r_select_grouped and s3r_select_pages form the same order in
 * their own launches when given an order array.
 *
 *   len    device i32 [B] (e.g. the context lengths L_b of the round);
 *   order  device i32 [B], written.
 * INVALID_ARG: null pointers, B < 1 or B > 65535. One kernel; O(B^2) compares
 * spread over ceil(B / 256) workgroups.
 */
s3r_status s3r_length_order(const int32_t* len, int32_t B, int32_t* order, hipStream_t stream);

/*
 * s3r_verify_attn - dense block verification. [news], Interpretation:
 * verification recomputes the proposed block against the complete historical
 * KV cache; [listing], Abstract: responses are generated through
 * full-attention verification.
 *
 * The block is the last k + 1 positions of each sequence's cache: row i
 * (0..k) sits at position P_i = seq_len[b] - (k + 1) + i and attends to
 * [0, P_i]:
 *   out[b][i][h] = softmax(scale * q[b][i][h] . K_[0,P_i]) V_[0,P_i],
 *   lse[b][i][h] = the natural-log normaliser of that row.
 * Scores for the next selection (reading adopted: a sum over the G query
 * heads of the KV head and over all k + 1 rows of each row's normalised
 * probability):
 *   scores[b][kv][j] = sum_{h in group(kv)} sum_{i : j <= P_i} prob_{b,i,h}(j)
 * for j < seq_len[b]; entries at and beyond seq_len[b] are not written. The
 * scores of one (b, kv) sum to G (k + 1). Precision: with bf16 K/V and
 * head_dim 128 each probability enters the scores as the bf16 value that also
 * weights V (relative step 2^-8; probabilities under 2^-22 of the row's running
 * maximum may come out anywhere below that fraction); otherwise float32.
 *
 *   q         device [B][k+1][Hq][head_dim] in kv->dtype.
 *   seq_len   device i32 [B]: cache length including the block,
 *             k + 1 <= seq_len[b] <= max_seq_len.
 *   out       device f32 [B][k+1][Hq][head_dim]; lse device f32 [B][k+1][Hq]
 *             or NULL; scores device f32 [B][Hkv][score_stride] or NULL
 *             (score_stride >= max_seq_len when scores is not NULL).
 *   ws        workspace of s3r_verify_workspace_bytes(...) bytes.
 * UNSUPPORTED: (k + 1) * Hq / Hkv > 64 rows per KV head.
 */
size_t s3r_verify_workspace_bytes(int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                  int32_t dtype, int32_t max_seq_len);
s3r_status s3r_verify_attn(const void* q, const s3r_paged_kv* kv, const int32_t* seq_len,
                           int32_t B, int32_t k, int32_t Hq, float scale, int32_t max_seq_len,
                           float* out, float* lse, float* scores, int32_t score_stride, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/*
 * s3r_verify_attn_pages - the verification with scores per page instead of
 * per position, for selection in whole pages (s3r_select_pages). [explainer],
 * mechanism paragraph: the drafter's set is described as the recent pages
 * plus the pages the previous verification weighted most.
 *
 * out and lse exactly as s3r_verify_attn (the same arithmetic). The score of
 * page p (positions [16 p, 16 p + 16) that lie below seq_len[b]) is the sum of
 * the position scores of s3r_verify_attn over those positions:
 *   page_scores[b][kv][p] = sum_{j in page p, j < seq_len[b]} scores[b][kv][j],
 * for p < ceil(seq_len[b] / 16); later entries are not written. The split
 * pass keeps one value per (page, query row) instead of one per (position,
 * query row), so the pass writes 16x fewer partial bytes. Precision: with
 * bf16 K/V, head_dim 128 and at most 32 query rows per KV head the page
 * masses are kept as bf16 relative to the split's row maxima (relative step
 * 2^-8); otherwise float32.
 *
 *   page_scores device f32 [B][Hkv][page_stride], required;
 *   page_stride >= ceil(max_seq_len / 16);
 *   ws        workspace of s3r_verify_pages_workspace_bytes(...) bytes (same
 *             arguments as s3r_verify_workspace_bytes).
 * Other arguments, statuses and UNSUPPORTED cases as for s3r_verify_attn.
 */
size_t s3r_verify_pages_workspace_bytes(int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t head_dim,
                                        int32_t dtype, int32_t max_seq_len);
s3r_status s3r_verify_attn_pages(const void* q, const s3r_paged_kv* kv, const int32_t* seq_len, int32_t B,
                                 int32_t k, int32_t Hq, float scale, int32_t max_seq_len, float* out, float* lse,
                                 float* page_scores, int32_t page_stride, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * The same verification in two calls, so that the scores, which only the
 * next round's selection reads, can be formed on another stream while the
 * output rows go on to sampling. [explainer], mechanism paragraph: the
 * selector ranks positions by the attention of the previous verification
 * pass, and the ranking is renewed at each round.
 *
 * s3r_verify_attn_deferred writes out and lse exactly as s3r_verify_attn and
 * leaves the score partials in ws. s3r_verify_scores then writes scores
 * exactly as s3r_verify_attn would (bit for bit) from those partials; call it
 * with the same kv description, seq_len, B, k, Hq, max_seq_len and ws, on
 * any stream ordered after the deferred call (e.g. through an event), and
 * before ws is used again. Arguments as for s3r_verify_attn; scores is
 * required by s3r_verify_scores, which reads only the metadata of kv
 * (num_kv_heads, head_dim, dtype, page_size, max_pages_per_seq).
 */
s3r_status s3r_verify_attn_deferred(const void* q, const s3r_paged_kv* kv, const int32_t* seq_len,
                                    int32_t B, int32_t k, int32_t Hq, float scale, int32_t max_seq_len,
                                    float* out, float* lse, void* ws, size_t ws_bytes,
                                    hipStream_t stream);
s3r_status s3r_verify_scores(const s3r_paged_kv* kv, const int32_t* seq_len, int32_t B, int32_t k,
                             int32_t Hq, int32_t max_seq_len, float* scores, int32_t score_stride,
                             const void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * s3r_spec_sample - exact speculative sampling with caller-supplied uniforms.
 * [explainer], Jargon "Exact speculative sampling" and the draft/verify
 * illustration (first mismatch replaced, the rest discarded); [news],
 * Interpretation (accept candidates or draw from the residual); [listing],
 * Table 7 caption (a fully accepted round yields k + 1 tokens).
 *
 * For each sequence b, in float64 from the float32 logits:
 *   p_i = softmax(target_logits[b][i] / T), i = 0..k;
 *   q_i = softmax(draft_logits[b][i] / T), i = 0..k-1;
 *   draft i (x = draft_tokens[b][i]) is accepted iff p_i(x) >= q_i(x) or
 *   uniforms[b][i] * q_i(x) < p_i(x); at the first reject i* the correction
 *   is drawn from max(0, p_i* - q_i*) (from p_i* if that residual is all zero);
 *   if every draft is accepted the bonus is drawn from p_k. Draws use the
 *   inverse CDF in token order with the single uniform uniforms[b][k]:
 *   y = min{y : sum_{y' <= y} w(y') > u * sum(w)} (the last y with w > 0 if
 *   rounding leaves none). T = 0 is greedy: accept iff x is the first argmax
 *   of target row i; correction and bonus are that argmax.
 *
 *   target_logits device f32 [B][k+1][V]; draft_logits device f32 [B][k][V]
 *   (may be NULL when k = 0); a logit of -inf is a token of probability 0 (a
 *   masked or padded vocabulary entry); NaN or +inf logits, or a row with no
 *   finite logit, are undefined behaviour; draft_tokens device i32 [B][k] in [0, V);
 *   uniforms device f32 [B][k+1] in [0, 1); temperature >= 0 (host).
 *   tokens    device i32 [B][k+1] output: the n_out[b] emitted tokens, then -1.
 *   n_out     device i32 [B] output: accepted drafts + 1.
 *   accepted  device i8 [B][k] output or NULL: 1 accepted, 0 the first
 *             reject, -1 not reached.
 *   ws        workspace of s3r_spec_sample_workspace_bytes(B, k, V) bytes.
 */
size_t s3r_spec_sample_workspace_bytes(int32_t B, int32_t k, int32_t V);
s3r_status s3r_spec_sample(const float* target_logits, const float* draft_logits,
                           const int32_t* draft_tokens, const float* uniforms, int32_t B,
                           int32_t k, int32_t V, float temperature, int32_t* tokens,
                           int32_t* n_out, int8_t* accepted, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * s3r_spec_sample_noalloc - s3r_spec_sample for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): no workspace argument, and no allocation in the
 * call. Same arguments, kernels and results (bit for bit) as s3r_spec_sample.
 *
 * Its scratch is a fixed array of S3R_SAMPLE_SCRATCH_BYTES in the library's
 * own device memory: each GPU the library runs on holds one copy until the
 * process ends; its device address is looked up on the first call on that
 * GPU (the GPU that runs `stream`). Every call on one GPU uses that GPU's
 * copy: calls that overlap in time on one GPU (different streams, or host
 * threads without ordering between them) race and give undefined results;
 * calls ordered on one stream are safe. Nothing in it needs clearing between
 * calls.
 * S3R_ERR_WORKSPACE when s3r_spec_sample_workspace_bytes(B, k, V) exceeds
 * S3R_SAMPLE_SCRATCH_BYTES (about 6700 sequences at k = 6, 5400 at k = 15);
 * S3R_ERR_HIP also when the array's device address cannot be obtained;
 * otherwise the statuses of s3r_spec_sample.
 */
#define S3R_SAMPLE_SCRATCH_BYTES ((size_t)8 << 20)
s3r_status s3r_spec_sample_noalloc(const float* target_logits, const float* draft_logits,
                                   const int32_t* draft_tokens, const float* uniforms, int32_t B, int32_t k,
                                   int32_t V, float temperature, int32_t* tokens, int32_t* n_out,
                                   int8_t* accepted, hipStream_t stream);

/*
 * Multi-round driving: the two calls that join rounds on the device, so that
 * rounds follow each other without a host synchronisation (and can be
 * captured in a HIP graph together with the four calls above).
 *
 * s3r_kv_append - write new K/V rows into the paged cache. [explainer],
 * mechanism paragraph: each draft step reads this round's own positions, so
 * a draft token's K/V row is cached before the step that reads it; [news],
 * Interpretation: verification recomputes the block against the complete
 * cache, so the block's K/V rows replace the draft rows at those positions.
 *
 *   k_rows, v_rows device [B][n][num_kv_heads][head_dim] in kv->dtype: row t
 *             of sequence b is written at position pos[b] + t (all KV heads),
 *             byte for byte.
 *   kv        the cache: its k_pages and v_pages are WRITTEN (the descriptor's
 *             const qualifiers describe the reading calls); block_table must
 *             map every written position of a sequence to a page no other
 *             sequence writes in the same call (pages shared by several
 *             sequences, such as a common prompt prefix, must not be written).
 *   pos       device i32 [B]: first position of each sequence's rows.
 *   n         rows per sequence (host, >= 1).
 *   max_pos   host bound: pos[b] + n <= max_pos <= max_pages_per_seq * 16.
 *             Rows whose position falls outside [0, max_pages_per_seq * 16)
 *             are skipped; other device values beyond the bounds are
 *             undefined behaviour.
 * No workspace. UNSUPPORTED: page_size != 16, head_dim not 64 or 128.
 */
s3r_status s3r_kv_append(const void* k_rows, const void* v_rows, const s3r_paged_kv* kv,
                         const int32_t* pos, int32_t B, int32_t n, int32_t max_pos, hipStream_t stream);

/*
 * s3r_commit - close a round on the device. [explainer], Jargon "Block
 * efficiency (tau)" and the draft/verify illustration: a round outputs the
 * accepted drafts plus one corrected (or bonus) token, the pending token and
 * the accepted drafts join the cache, and the last output token is the next
 * round's pending token. Rows of rejected drafts at and beyond the new length
 * stay in the cache until the next round overwrites them; nothing reads them
 * before (the rollback is implicit).
 *
 * For each sequence b with 1 <= n_out[b] <= k + 1 (others are left as they
 * are):
 *   ctx_len[b] (in/out)  L_b -> L'_b = L_b + n_out[b];
 *   pending[b]           tokens[b][n_out[b] - 1]                 (or NULL);
 *   cur_len[(j-1)*B + b] L'_b + j, j = 1..k: the next round's draft steps
 *                        (one [B] array per step, as s3r_sparse_decode_attn
 *                        takes them)                             (or NULL);
 *   seq_len[b]           L'_b + k + 1, the next verification     (or NULL);
 *   verified[0] (in/out) += sum of n_out over the updated sequences (or NULL).
 *
 *   n_out, tokens: as written by s3r_spec_sample (device i32 [B], [B][k+1]).
 * No workspace; one workgroup.
 */
s3r_status s3r_commit(const int32_t* n_out, const int32_t* tokens, int32_t B, int32_t k, int32_t* ctx_len,
                      int32_t* pending, int32_t* cur_len, int32_t* seq_len, int64_t* verified,
                      hipStream_t stream);

/*
 * Measurement helpers (not part of the method): the HBM read patterns of the
 * verification and of one draft step, for the read ceiling the attention
 * kernels are measured against. Each reads exactly the K and V bytes the
 * bf16 / head_dim 128 kernel of that call reads (whole 32-position subtiles
 * of every sequence's cache; the kept rows plus [sel_len, cur_len)), in the
 * same launch shape, performs no arithmetic on them, and writes one 32-bit
 * checksum (an xor of the loaded words) per workgroup to sink so no load is
 * dropped. The checksums carry no meaning beyond that.
 *
 *   s3r_read_verify_pattern: kv and seq_len as for s3r_verify_attn;
 *   s3r_read_draft_pattern: kv, idx, nsel_cap, n_sel, sel_len, cur_len, B and
 *             max_attend as for s3r_sparse_decode_attn (no order);
 *   sink      device u32 of at least s3r_read_pattern_sink_words(B, Hkv,
 *             max_seq_len or max_attend, draft = 0 or 1) words.
 * UNSUPPORTED unless bf16, head_dim 128, page_size 16.
 */
size_t s3r_read_pattern_sink_words(int32_t B, int32_t Hkv, int32_t max_len, int32_t draft);
s3r_status s3r_read_verify_pattern(const s3r_paged_kv* kv, const int32_t* seq_len, int32_t B, int32_t max_seq_len,
                                   uint32_t* sink, size_t sink_words, hipStream_t stream);
s3r_status s3r_read_draft_pattern(const s3r_paged_kv* kv, const int32_t* idx, int32_t nsel_cap,
                                  const int32_t* n_sel, const int32_t* sel_len, const int32_t* cur_len, int32_t B,
                                  int32_t max_attend, uint32_t* sink, size_t sink_words, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* S3R_H */
