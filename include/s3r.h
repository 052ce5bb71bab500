/*
 * libs3r: the data-parallel hot path of Self-Sparse Speculative Rollouts on one
 * MI355X (gfx950).
 *
 * "S3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative Decoding",
 * Abstract: in one rollout round the policy proposes tokens while attending to
 * only part of its KV cache; a dense pass over every cached key and value then
 * checks them, and speculative sampling accepts or resamples so that the output
 * keeps the dense policy's distribution. Drafter and verifier are one model, so
 * they share one cache. The calls below are that round's per-step operations.
 *
 * Conventions for every call
 * --------------------------
 * - Pointers are device pointers (hipMalloc'd or torch CUDA tensors) unless a
 *   comment says "host". The caller owns every buffer and keeps it alive until
 *   the work queued on `stream` has completed. The library allocates and frees
 *   no device memory; scratch is the caller's `workspace`, sized by the
 *   matching *_workspace() query (host-only, no HIP call). The one exception,
 *   s3r_spec_sample_noalloc, uses a scratch array the library keeps in device
 *   memory instead (see there).
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls
 *   only enqueue work: no call synchronises the device or the host (except
 *   under S3R_DEBUG).
 * - Host-side validation of scalars, pointers and shapes happens before any HIP
 *   call; a failed check returns its status and enqueues nothing. Device data
 *   (page ids, seq_lens, token ids) is trusted unless S3R_DEBUG is set (see
 *   "Device data checks" below). No C++ exception crosses the
 *   ABI. The library keeps no state between calls; calls on different streams
 *   are safe if their outputs and workspaces are disjoint (calls of
 *   s3r_spec_sample_noalloc on one GPU share that GPU's scratch).
 * - k_pool, v_pool, bounds, q, attention outputs, new K/V rows and every
 *   workspace must be 16-byte aligned (torch allocations are): the kernels
 *   move them as 16-byte vectors. A misaligned one is INVALID_ARGUMENT.
 *   Logits rows, page tables, lengths, selections and tokens need only their
 *   element alignment.
 * - Supported: head_dim 64 or 128, page_size 16, num_q_heads a multiple of
 *   num_kv_heads with G = num_q_heads/num_kv_heads <= 8, kv dtype f32 or bf16,
 *   G * n_queries <= 64 attention rows per kv head, 1 <= gamma <= 16.
 *
 * Data layout in HBM
 * ------------------
 *   k_pool     [num_phys_pages][Hkv][P][D]  key of token t at slot t % P
 *   v_pool     [num_phys_pages][Hkv][D][P]  value, transposed inside each page
 *   page_table [B][max_pages_per_seq] int32 logical page -> physical page
 *   seq_lens   [B] int32                    KV positions visible to the last query
 *   bounds     [num_phys_pages][Hkv][2][D]  kv dtype; [0] elementwise key min,
 *                                           [1] elementwise key max of the page
 * Every physical page belongs to one sequence. The entries of a sequence's
 * pages below seq_len must be valid physical pages (0 <= entry < num_phys_pages):
 * attention, bounds and selection read them unchecked. Only the KV commit
 * accepts a negative entry, as an unallocated page. A sequence with seq_len <= 0,
 * and a causal verify row that sees no position, get an all-zero output.
 *
 * Device data checks (S3R_DEBUG)
 * ------------------------------
 * The kernels trust three kinds of device data, which sit on the device and are
 * not checked by default:
 *   - seq_lens: ceil(seq_len / P) must not exceed max_pages_per_seq;
 *   - page_table entries of the pages a call reads: each must lie in
 *     [0, num_phys_pages), or be >= 0 when num_phys_pages is 0;
 *   - draft_tokens of s3r_spec_sample: each must lie in [0, vocab).
 * Selection lists, first_pos and refresh_from need no check: the kernels mask
 * or clamp every value.
 * When the environment variable S3R_DEBUG is set to anything but "" or "0" at
 * call time, every call that reads such data first waits for its stream,
 * copies that data to the host and checks it. On a bad value it prints the
 * call, the index and the value to stderr and returns INVALID_ARGUMENT without
 * launching anything. Such a call synchronises its stream, so it cannot be
 * captured into a graph: under capture it returns UNSUPPORTED. A failed copy
 * returns HIP.
 */
#ifndef S3R_H
#define S3R_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t s3r_status;
#define S3R_OK 0
#define S3R_ERR_INVALID_ARGUMENT 1
#define S3R_ERR_UNSUPPORTED 2
#define S3R_ERR_WORKSPACE_TOO_SMALL 3
#define S3R_ERR_HIP 4

typedef enum { S3R_F32 = 0, S3R_BF16 = 1 } s3r_dtype;

/* Host struct describing caller-owned device buffers of one paged KV cache.
   Every call that takes one returns INVALID_ARGUMENT for non-positive sizes,
   Hq not a multiple of Hkv, NULL or non-16-byte-aligned pools, or NULL
   page_table/seq_lens; UNSUPPORTED for another dtype, D or P, Hq/Hkv > 8, or
   num_seqs * num_q_heads > 2^24 (the kernels index (sequence, head) pairs and
   their grids in 32 bits). */
typedef struct {
  int32_t num_seqs;          /* B */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv; q head g reads kv head g / (Hq/Hkv) */
  int32_t head_dim;          /* D: 64 or 128 */
  int32_t page_size;         /* P: 16 */
  int32_t max_pages_per_seq; /* row length of page_table */
  int32_t total_pages_hint;  /* host: sum over sequences of their page count,
                                or 0 if unknown (then B * max_pages_per_seq is
                                assumed). It sizes the split-KV partitioning and,
                                when below half of B * max_pages_per_seq (a
                                ragged batch), has the attention calls take the
                                sequences longest first, which adds B int32 of
                                scheduling order to their workspace. Results do
                                not depend on it beyond rounding. */
  s3r_dtype kv_dtype;        /* dtype of k_pool, v_pool, bounds and q */
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int32_t num_phys_pages;    /* pages in k_pool, v_pool and bounds, or 0 if not
                                given. Only the S3R_DEBUG checks read it. */
} s3r_paged_kv;

/* Workspace sizes in bytes (host computation only; 0 means none needed). */
size_t s3r_page_select_workspace(const s3r_paged_kv* kv, int32_t budget_tokens);
/* n_queries: 1 for the draft, gamma+1 for verify. max_pages_attended: k
   (= budget/P) for the draft, max_pages_per_seq for verify. */
size_t s3r_attn_workspace(const s3r_paged_kv* kv, int32_t n_queries, int32_t max_pages_attended);
size_t s3r_spec_sample_workspace(int32_t num_seqs, int32_t gamma, int32_t vocab);

/*
 * s3r_page_bounds_update: recompute the exact elementwise min and max of the
 * keys of every page touched since the last call, over the page's valid
 * tokens j*P <= t < min((j+1)*P, seq_len). This keeps the per-page key bounds
 * that s3r_page_select scores against in step with the KV cache after a KV
 * append or rollback (support for the query-aware selection rule). S3R
 * Abstract: drafter and verifier are one model over one cache, so the pages
 * the sparse draft ranks are the same pages verification later reads; their
 * bounds must describe exactly the keys they hold at each draft step.
 *   bounds     out, [num_phys_pages][Hkv][2][D] in kv dtype.
 *   first_pos  [B] int32: for sequence b, pages from first_pos[b] / P to the
 *              last page of seq_lens[b] are recomputed. NULL = every page.
 *   max_pages_touched  host: an upper bound on the pages any sequence has
 *              touched when first_pos is given (ignored when NULL).
 * Errors: INVALID_ARGUMENT for NULL kv/pools/page_table/seq_lens/bounds or a
 * non-positive max_pages_touched with first_pos given.
 */
s3r_status s3r_page_bounds_update(const s3r_paged_kv* kv, void* bounds, const int32_t* first_pos,
                                  int32_t max_pages_touched, void* stream);

/*
 * s3r_page_select: query-aware page selection for the sparse draft. The S3R
 * abstract states only that drafting uses sparse attention; this library fixes
 * the rule, after the Quest work the S3R reference list cites: per (sequence
 * b, kv head h) with n = ceil(seq_len/P) pages and k = budget_tokens / P,
 *   score_j = max over the G q heads of h of
 *             softmax_scale * sum_d max(q_d * kmin_{j,d}, q_d * kmax_{j,d}),
 * an upper bound on each head's logit for any token of page j. If k >= n all
 * pages 0..n-1 are taken; otherwise the k best by (score desc, page asc).
 *   q            [B][Hq][D] kv dtype, the draft query.
 *   selected     out [B][Hkv][k] int32 logical page ids, ascending, -1 padded.
 *   num_selected out [B] int32 = min(k, n).
 * Errors: INVALID_ARGUMENT for NULL pointers or budget_tokens < P;
 * UNSUPPORTED if max_pages_per_seq > 32768 (the block top-k holds at most
 * 32768 page keys per row, 524288 tokens); WORKSPACE_TOO_SMALL if workspace_bytes <
 * s3r_page_select_workspace().
 * Scores are fp32; ties closer than fp32 rounding may order differently from an
 * exact computation.
 */
s3r_status s3r_page_select(const s3r_paged_kv* kv, const void* bounds, const void* q,
                           int32_t budget_tokens, float softmax_scale, int32_t* selected,
                           int32_t* num_selected, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * s3r_sparse_draft_attn: one draft step's attention, over the selected pages
 * only (S3R Abstract: the drafter is the policy itself, attending sparsely). Query head g
 * of sequence b attends, with softmax(softmax_scale * q K^T) V, to the tokens
 * t < seq_len of the pages in selected[b][g / G]. The G heads of a kv head
 * share each K/V tile they read.
 *   q         [B][Hq][D] kv dtype.
 *   selected  [B][Hkv][k] int32 logical page ids in s3r_page_select's format:
 *             entries equal to -1 are skipped; only the first
 *             min(k, ceil(seq_len/P)) entries of each row are read.
 *   out       [B][Hq][D] in out_dtype (f32 or bf16), written, never read.
 * Errors: INVALID_ARGUMENT / UNSUPPORTED / WORKSPACE_TOO_SMALL as above.
 */
s3r_status s3r_sparse_draft_attn(const s3r_paged_kv* kv, const void* q, const int32_t* selected,
                                 int32_t k, float softmax_scale, s3r_dtype out_dtype, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_sparse_draft_step: one whole draft step (S3R Abstract: the policy
 * drafts with sparse attention over its own KV cache, reading only part of
 * it), the fused form of
 *   s3r_page_bounds_update(refresh_from)  (when refresh_from is not NULL)
 *   s3r_page_select(q, budget_tokens)     -> selected, num_selected
 *   s3r_sparse_draft_attn(q, selected)    -> out
 * The bounds written and the selection are identical to those calls'; the
 * attention output equals theirs up to the order in which split partials are
 * merged. bf16 KV runs one kernel when one workgroup per (sequence, kv head)
 * fills the device (it refreshes, scores, ranks in LDS and attends), else two
 * (scores with the refresh, then rank-and-attend); fp32 KV and very long page
 * tables run the three calls' kernels.
 *   bounds        in/out, [num_phys_pages][Hkv][2][D] kv dtype.
 *   refresh_from  [B] int32 or NULL: pages from refresh_from[b] / P to the
 *                 tail get their bounds recomputed from K first.
 *   selected, num_selected: out, as s3r_page_select.   out: as s3r_sparse_draft_attn.
 * Errors: as the three calls; WORKSPACE_TOO_SMALL if workspace_bytes <
 * s3r_sparse_draft_step_workspace().
 */
size_t s3r_sparse_draft_step_workspace(const s3r_paged_kv* kv, int32_t budget_tokens);
s3r_status s3r_sparse_draft_step(const s3r_paged_kv* kv, void* bounds, const int32_t* refresh_from,
                                 const void* q, int32_t budget_tokens, float softmax_scale,
                                 int32_t* selected, int32_t* num_selected, s3r_dtype out_dtype,
                                 void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_sparse_draft_round: draft step 0 of a round whose selection is made
 * once and reused by the round's later steps (a selection-frequency variant of
 * re-selecting at every step; the S3R abstract leaves the frequency open).
 * As s3r_sparse_draft_step, except the selection: with seq_len the step-0
 * length, the logical pages holding positions seq_len - 1 .. seq_len + gamma - 2
 * (where the round's gamma draft queries sit; one or two pages, clipped to
 * max_pages_per_seq) are always kept, including one that does not exist yet,
 * and the other k - |forced| slots go to the best-scoring remaining pages (all
 * of them if they fit). Rows are ascending and -1 padded; num_selected[b]
 * counts the kept pages. Draft step j > 0 then calls s3r_sparse_draft_attn
 * with the same `selected` and its own seq_lens (pages past the sequence are
 * masked until they fill).
 *   gamma  1..16, the round's draft length.
 * Errors: INVALID_ARGUMENT if gamma is out of range or budget_tokens < 2 * P;
 * otherwise as s3r_sparse_draft_step, whose workspace query applies.
 */
s3r_status s3r_sparse_draft_round(const s3r_paged_kv* kv, void* bounds, const int32_t* refresh_from,
                                  const void* q, int32_t budget_tokens, int32_t gamma,
                                  float softmax_scale, int32_t* selected, int32_t* num_selected,
                                  s3r_dtype out_dtype, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * s3r_kv_commit: the KV step either side of a round. It writes new K/V rows
 * (what a draft or verify forward pass produced) into their pages and keeps
 * the page bounds exact for the committed lengths; a length below rows already
 * written rolls them back. S3R Abstract: drafter and verifier are one model
 * over one KV cache, so these rows are the ones the sparse draft later ranks.
 *   kv          seq_lens holds the committed lengths AFTER the call. The call
 *               writes the pools kv->k_pool and kv->v_pool point at.
 *   k_new, v_new  [B][count][Hkv][D] kv dtype, 16-byte aligned: row i of
 *               sequence b goes to position first_pos[b] + i (logical page
 *               pos / P via page_table, slot pos % P; V transposed inside the
 *               page). Rows past max_pages_per_seq pages, or in a page
 *               whose page_table entry is negative (unallocated), are dropped.
 *   first_pos   [B] int32, >= 0.
 *   count       rows per sequence, >= 0 (0: a pure rollback).
 *   bounds      in/out [num_phys_pages][Hkv][2][D] kv dtype, or NULL for no
 *               bounds upkeep. Every logical page from
 *               min(first_pos[b], seq_len - 1) / P through the last written
 *               page or the tail page of seq_len is recomputed over its tokens
 *               < seq_len, if it has any; other pages are left alone.
 * Errors: INVALID_ARGUMENT for count < 0, NULL first_pos, NULL or misaligned
 * rows when count > 0; otherwise as check of kv. No workspace.
 */
s3r_status s3r_kv_commit(const s3r_paged_kv* kv, const void* k_new, const void* v_new,
                         const int32_t* first_pos, int32_t count, void* bounds, void* stream);

/*
 * s3r_dense_verify_attn: full-attention verification of the draft (S3R
 * Abstract: verifying reads every cached key and value of the sequence).
 * Query i = 0..n_q-1 of sequence b sits at position seq_len - n_q + i and
 * attends causally to every position <= its own, over
 * all pages of the sequence. n_q = gamma + 1 (the last committed token plus
 * the gamma drafts) gives the gamma + 1 target distributions of one round.
 *   q    [B][n_q][Hq][D] kv dtype.
 *   out  [B][n_q][Hq][D] in out_dtype.
 * Errors: INVALID_ARGUMENT for NULL pointers or n_q < 1; UNSUPPORTED if
 * G * n_q > 64; WORKSPACE_TOO_SMALL as above.
 */
s3r_status s3r_dense_verify_attn(const s3r_paged_kv* kv, const void* q, int32_t n_q,
                                 float softmax_scale, s3r_dtype out_dtype, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_spec_sample: exact speculative sampling of one round ("exact speculative
 * sampling", S3R Abstract; the rule of the speculative decoding/sampling works
 * its reference list cites). Per sequence b, with p_i = softmax(target_i / T)
 * and q_i = softmax(draft_i / T):
 *   for i = 0..gamma-1, x = draft_tokens[b][i], u = U(b, i, 0):
 *     accept iff (q_i(x) > 0 and u < p_i(x)/q_i(x)) or (q_i(x) = 0 and p_i(x) > 0);
 *     at the first reject emit ICDF(max(0, p_i - q_i), U(b, i, 1)) (p_i if that
 *     residual has no mass) and stop;
 *   if all accept, emit the bonus ICDF(p_gamma, U(b, gamma, 1)).
 * ICDF(w, u) is the smallest token t with sum_{s<=t} w_s > u * sum(w).
 * U(b, slot, stream) = (w0 >> 11) * 2^-53 with w0 word 0 of Philox4x64-10
 * (Salmon et al., SC'11) at key (seed, 0), counter (offset, b, slot, stream).
 *   draft_logits  [B][gamma][V] fp32;  target_logits [B][gamma+1][V] fp32.
 *                 -inf masks a token (probability 0). Every row needs at least
 *                 one finite logit; NaN, +inf or a fully masked row give
 *                 unspecified tokens (the writes stay inside out_tokens).
 *   draft_tokens  [B][gamma] int32 in [0, V).
 *   out_tokens    out [B][gamma+1] int32: accepted drafts, then the drawn token,
 *                 then -1.
 *   num_accepted  out [B] int32: accepted drafts n (n + 1 tokens committed).
 * Errors: INVALID_ARGUMENT for NULL pointers, num_seqs < 1, vocab < 1, gamma
 * outside 1..16, temperature not finite and > 0; UNSUPPORTED when
 * num_seqs * (2 * gamma + 1) * ceil(vocab / 4096) >= 2^31; WORKSPACE_TOO_SMALL.
 * Deterministic: no floating-point atomics; reductions run in a fixed order.
 */
s3r_status s3r_spec_sample(int32_t num_seqs, int32_t gamma, int32_t vocab,
                           const float* draft_logits, const float* target_logits,
                           const int32_t* draft_tokens, float temperature, uint64_t seed,
                           uint64_t offset, int32_t* out_tokens, int32_t* num_accepted,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_spec_sample_noalloc: s3r_spec_sample for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same results from the same kernels, with the
 * workspace taken from a scratch array the library holds in device memory
 * (one per GPU it runs on, kept until the process ends) instead of a caller
 * buffer. The call allocates nothing. Arguments and errors as
 * s3r_spec_sample, except WORKSPACE_TOO_SMALL when
 * s3r_spec_sample_workspace(num_seqs, gamma, vocab) exceeds
 * s3r_spec_sample_noalloc_max_workspace() (4 MiB: for example B = 256,
 * gamma = 16 at a 152K vocabulary), and HIP if the scratch's device address
 * cannot be looked up. Every value the call reads from the scratch it first
 * writes itself, so nothing is cleared between calls. All calls on one GPU
 * share its scratch: two calls that may overlap on that GPU (other streams,
 * other host threads) race and give undefined tokens; serialise them.
 */
size_t s3r_spec_sample_noalloc_max_workspace(void);
s3r_status s3r_spec_sample_noalloc(int32_t num_seqs, int32_t gamma, int32_t vocab,
                                   const float* draft_logits, const float* target_logits,
                                   const int32_t* draft_tokens, float temperature, uint64_t seed,
                                   uint64_t offset, int32_t* out_tokens, int32_t* num_accepted,
                                   void* stream);

/*
 * s3r_draft_sample: the drafter's own draws, sampling directly from the
 * sparse policy (S3R Abstract: sparse attention proposes the tokens; sampling
 * from that policy with no dense check is the direct-sparse-sampling
 * comparator the abstract finds unstable). Row r of sequence b draws
 *   tokens[b][r] = ICDF(softmax(logits[b][r] / T), U(b, first_slot + r, 2)),
 * ICDF and U as in s3r_spec_sample; stream 2 is the drafter's, so these draws
 * are independent of the sampler's accept (0) and residual (1) uniforms. With
 * first_slot = 0 and n_rows = gamma the tokens are the draft_tokens input of
 * s3r_spec_sample; a drafter that samples one position at a time passes
 * n_rows = 1 and first_slot = that position's draft index.
 *   logits      [B][n_rows][V] fp32; -inf masks a token. Every row needs a
 *               finite logit (a fully masked row gives an unspecified token
 *               in [-1, V)).
 *   first_slot  >= 0.
 *   tokens      out [B][n_rows] int32 in [0, V).
 * Errors: INVALID_ARGUMENT for NULL pointers, num_seqs, n_rows or vocab < 1,
 * first_slot < 0, temperature not finite and > 0; UNSUPPORTED when
 * num_seqs * n_rows * ceil(vocab / 4096) >= 2^31; WORKSPACE_TOO_SMALL.
 * Deterministic; two launches (chunk statistics, then one draw per row).
 */
size_t s3r_draft_sample_workspace(int32_t num_seqs, int32_t n_rows, int32_t vocab);
s3r_status s3r_draft_sample(int32_t num_seqs, int32_t n_rows, int32_t vocab, const float* logits,
                            float temperature, uint64_t seed, uint64_t offset, int64_t first_slot,
                            int32_t* tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * s3r_acceptance_rate: per draft position, the probability that exact
 * speculative sampling accepts a draft drawn from q_i,
 *   alpha[b][i] = sum_x min(p_i(x), q_i(x)),  i = 0..gamma-1,
 * with p_i = softmax(target_logits[b][i] / T), q_i = softmax(draft_logits[b][i] / T).
 * 1 - alpha is the total-variation distance TV(p_i, q_i): how far a token
 * sampled directly from the sparse policy is from the dense policy's law,
 * the gap that S3R turns into a lower acceptance rate instead (S3R Abstract).
 *   draft_logits [B][gamma][V], target_logits [B][gamma+1][V] fp32 (the
 *                layouts of s3r_spec_sample; the bonus row is not read).
 *   alpha        out [B][gamma] double, 8-byte aligned.
 * Errors: INVALID_ARGUMENT for NULL or misaligned pointers, num_seqs, gamma
 * or vocab < 1, temperature not finite and > 0; UNSUPPORTED when
 * num_seqs * 2 * gamma * ceil(vocab / 4096) >= 2^31; WORKSPACE_TOO_SMALL.
 * Deterministic: fp64 sums in a fixed order.
 */
size_t s3r_acceptance_rate_workspace(int32_t num_seqs, int32_t gamma, int32_t vocab);
s3r_status s3r_acceptance_rate(int32_t num_seqs, int32_t gamma, int32_t vocab,
                               const float* draft_logits, const float* target_logits,
                               float temperature, double* alpha, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Static description of a status code (host, never NULL). */
const char* s3r_status_string(s3r_status status);
/* Library version: major * 10000 + minor * 100 + patch. */
int32_t s3r_version(void);

#ifdef __cplusplus
}
#endif

#endif /* S3R_H */
