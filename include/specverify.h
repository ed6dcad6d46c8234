/*
 * specverify.h - C ABI of the MI355X (gfx950) batched speculative-sampling
 * verifier, the verify half of one speculative-decoding round.
 *
 * What it computes (sources cited by page title and section):
 *  - bloss0m.com, "Speculative Decoding：用小模型打草稿、大模型一次驗…",
 *    section "技術機制 / Technical mechanism": speculative sampling (paper
 *    §2.3) and Algorithm 1 - each drafted token x_i is kept when
 *    r_i <= p_i(x_i) / q_i(x_i); the scan stops at the first rejection; a
 *    replacement is drawn from norm(max(0, p - q)) at that position, or a bonus
 *    token from p_{gamma+1} when every draft was kept.
 *  - blog.vllbc.top, "Speculative Decoding：draft 先猜，target 一次验证":
 *    the same Algorithm 1 steps; the vLLM verification path, which scans a
 *    flattened batch through cu_num_draft_tokens and returns accepted +
 *    recovered + bonus tokens; the note on paper §2.2 (temperature folds into
 *    p and q, a greedy draft is a one-hot q).
 *  - timinsight.com, "Speculative Decoding 實作指南：基準、驗證與取捨",
 *    section "Step 2": target probabilities are a softmax of the target
 *    logits; when the residual mass is not above 1e-8 the replacement is drawn
 *    from p instead.
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller. The library
 *    never allocates and never synchronises, and keeps no state apart from the
 *    fixed scratch of spec_verify_probs_noalloc (and the host-side benchmark
 *    diagnostics); work is enqueued on `stream` (a hipStream_t passed as
 *    void*, NULL = the null stream) and the outputs are valid once that
 *    stream has completed the work.
 *  - Target temperature: p = softmax(logits / T) for T > 0; T == 0 means
 *    argmax decoding (p one-hot at the argmax, lowest index on ties).
 *  - Accept test, in product form: x is kept iff p(x) > 0 and u * q(x) <= p(x).
 *  - Uniforms: a request with g drafts owns g + 1 uniforms in (0, 1]: entries
 *    0..g-1 are the accept uniforms, entry g is the single sample uniform,
 *    used for the emitted replacement or bonus token.
 *  - Sampling is by inverse CDF in ascending token order: the emitted token is
 *    the smallest k with C[k] >= u * C[V-1], C the running sum of the
 *    (unnormalised) weights.
 *  - Results equal exact-arithmetic results. Every decision taken in fp32 is
 *    checked against a rigorous error bound; rows where a decision is within
 *    the bound are recomputed in fp64 before anything is written.
 *  - Device-side preconditions (not checked, cannot be reported without a
 *    sync; violating them never makes a kernel read or write out of bounds):
 *    draft tokens in [0, V) (an out-of-range token is rejected with p(x) = 0);
 *    uniforms in (0, 1]; logits finite or -inf with at least one finite value
 *    per row (no NaN); q finite and >= 0; cu_num_draft_tokens non-decreasing
 *    from 0 to num_draft_tokens.
 *  - Errors found on the host return a negative status and launch nothing.
 */
#ifndef SPECVERIFY_H_
#define SPECVERIFY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the target logits. Draft probabilities are always fp32. */
enum sv_dtype { SV_DTYPE_F32 = 0, SV_DTYPE_BF16 = 1 };

/* Status codes. */
enum sv_status {
  SV_OK = 0,
  SV_ERR_INVALID_ARGUMENT = -1, /* null pointer, negative size, bad temperature or flags */
  SV_ERR_UNSUPPORTED = -2,      /* unknown dtype, vocab_size above SV_MAX_VOCAB */
  SV_ERR_LAUNCH = -3,           /* a kernel launch failed (hipGetLastError) */
  SV_ERR_WORKSPACE = -4         /* workspace missing or smaller than required */
};

/* Largest supported vocabulary. */
#define SV_MAX_VOCAB (1 << 21)

/* flags for spec_verify_probs / spec_verify_ragged. The three ways of drawing
 * replacements give identical results; they differ in the bytes they read:
 *  default (lazy): pass 1 over the logits decides the accept tests, positions
 *    in order across the batch; a row after a position already known to be
 *    a certain rejection is not read (rows whose earlier positions are still
 *    undecided are read speculatively); the residual max(0, p - q) is then
 *    drawn only at each request's first rejection (the logits and q of that
 *    one row are read again; with one-hot drafts only its logits: the
 *    residual is then p without the draft token). Row statistics imply
 *    SV_FLAG_ALL_RESIDUALS.
 *  SV_FLAG_EAGER: every draft row whose own accept test fails draws its
 *    replacement in the same launch (speculatively; most are unused).
 *  SV_FLAG_ALL_RESIDUALS: every draft row draws its replacement. */
#define SV_FLAG_EXACT 0x1u         /* take every row through the fp64 path (reference / testing) */
#define SV_FLAG_ALL_RESIDUALS 0x2u /* draw the replacement token of every draft row, accepted or not */
#define SV_FLAG_EAGER 0x4u         /* draw the replacement of every locally rejected draft row */

/* Workspace: device memory of spec_verify_workspace_size() bytes, 256-byte
 * aligned, ZERO-FILLED BEFORE ITS FIRST USE; every call that completes
 * leaves it ready for the next one, of any kind, row count or vocabulary
 * size (the counters sit at a fixed offset and return to zero; per-request
 * state is cleared by the call that uses it). One workspace per call in
 * flight (calls that share one on different streams race); a call that was
 * never run to completion leaves the workspace to be zero-filled again. It
 * starts with a 256-byte block of counters, then one 8-byte record per target
 * row, {int32 token, uint32 row_flags} (documented for diagnostics), then the
 * list and fp64 tile sums of the rows recomputed in fp64 and the lazy mode's
 * state. row_flags bits: */
#define SV_ROW_ACCEPTED 0x1u  /* the row's own accept test passed */
#define SV_ROW_EXACT 0x2u     /* the row was recomputed on the fp64 path */
#define SV_ROW_RESIDUAL 0x4u  /* the row's replacement token was drawn (q read in full) */
#define SV_ROW_FALLBACK 0x8u  /* residual mass <= 1e-8: the replacement was drawn from p */
/* why a row went to the fp64 path (set together with SV_ROW_EXACT): */
#define SV_ROW_WHY_ACCEPT 0x10u    /* accept test within the fp32 error bound, or p(x) < 1e-30 */
#define SV_ROW_WHY_FALLBACK 0x20u  /* residual mass within the bound of the 1e-8 threshold */
#define SV_ROW_WHY_SEARCH 0x40u    /* inverse-CDF search inconclusive in fp32 */
#define SV_ROW_WHY_MARGIN 0x80u    /* sample uniform within the bound of a CDF boundary */
#define SV_ROW_WHY_FORCED 0x100u   /* SV_FLAG_EXACT, or a degenerate row */
#define SV_ROW_DEFERRED 0x400u     /* lazy mode: rejected (or bonus) row whose token was not needed (not drawn) */
#define SV_ROW_UNDECIDED 0x800u    /* lazy mode: accept test left to the per-request fp64 pass, which did not
                                      need this row (an earlier row was rejected) */
#define SV_ROW_UNREAD 0x1000u      /* lazy mode: row after a position known to be a certain rejection: not
                                      needed, its logits not read (or not read to the end: a row of the
                                      second per-row launch stops once that becomes known) */
/* top-k / top-p (the *_filtered entry points): how the row's threshold was
 * found when the head gathered during the first pass over the row (its
 * largest logits) could not decide it: */
#define SV_ROW_HEAD2 0x2000u       /* from a second, larger or smaller, gathered head */
#define SV_ROW_ROW_SELECT 0x4000u  /* from a radix select over the whole row */
/* lazy mode, one-hot drafts (no q rows) with bf16 logits: */
#define SV_ROW_TILE_SUMS 0x8000u   /* rejected (or bonus) row whose fp64 tile sums the per-row pass kept (the
                                      per-request stage does not read its logits again) */

/* Bytes of workspace needed for `num_target_rows` target rows (dense:
 * num_requests * (gamma + 1); ragged: num_draft_tokens + num_requests) of
 * `vocab_size` tokens: 104 bytes per row for the records, list, counters and
 * lazy-mode statistics, marks and task list, plus 28 * ceil(vocab_size / 2048) bytes
 * per row for fp64 tile sums, each part rounded up to 256 bytes. The greedy
 * entry point needs only the counters and the records (256 bytes, then 8
 * bytes per row rounded up to 256).
 * Returns 0 for a negative row count or a vocab_size outside [1, SV_MAX_VOCAB]. */
size_t spec_verify_workspace_size(int64_t num_target_rows, int32_t vocab_size);

/* Static, human-readable text for a status code. */
const char* spec_verify_status_string(int status);

/* Library ABI version (currently 3: 2 added the *_filtered entry points, 3
 * spec_verify_probs_noalloc). */
int spec_verify_version(void);

/* Self-check of the one hardware property the certified fast path relies on:
 * writes to *max_rel_err (device pointer to one double) the largest relative
 * error of the GPU's fp32 exp2 over every fp32 input in [-126, 0], measured
 * against fp64 exp2. spec_verify_exp2_error_bound() returns the bound the
 * error analysis assumes; a measured value above it means results are no
 * longer certified on that device. Asynchronous on `stream`. */
int spec_verify_selftest_exp2(double* max_rel_err, void* stream);
double spec_verify_exp2_error_bound(void);

/* Benchmark context: a read-only stream of known size. Reads `bytes` of
 * device memory at `src` once, with 16-byte loads, and writes the sum of its
 * 32-bit words (as unsigned, modulo 2^64) to *word_sum (device pointer to
 * one 64-bit integer); its rate is the practical HBM read ceiling the
 * verifier's streaming kernels are measured against. Requires `src` 16-byte
 * aligned, `bytes` a multiple of 16 (0 allowed), `word_sum` not NULL;
 * otherwise SV_ERR_INVALID_ARGUMENT, and nothing is launched. Asynchronous on
 * `stream`; allocates nothing. */
int spec_verify_stream_read(const void* src, size_t bytes, unsigned long long* word_sum, void* stream);

/* Benchmark diagnostics: time kernels of the probabilistic entry points with
 * HIP events that the library records on the launch stream right before and
 * right after each launch of a selected kernel.
 *   kernel_mask  bit SV_PROFILE_ROWS: the per-row pass (softmax statistics
 *                and accept test, every mode; both launches of the default
 *                mode); bit SV_PROFILE_REQUEST: the per-request stage of the
 *                default (lazy) mode; bit SV_PROFILE_ROWS_FIRST: the first
 *                per-row launch of the default mode alone
 *   capacity     launches recorded per kernel, 1 .. 2^20; later ones are not
 * spec_verify_profile_start drops any earlier recording, creates the events
 * and starts recording (SV_ERR_INVALID_ARGUMENT for a bad mask or capacity,
 * SV_ERR_LAUNCH if events cannot be created). spec_verify_profile_stop waits
 * for the recorded events, writes per kernel id (arrays of 3) the summed
 * duration in milliseconds and the number of launches recorded, releases the
 * events and stops recording (either pointer may be NULL). Library-wide host
 * state: not for concurrent callers.
 * spec_verify_profile_every (after start) records only every `every`-th call
 * (the first, then each `every` calls later), so that a timed loop carries
 * few events: an event recorded between two kernels delays the second by
 * a few microseconds. SV_ERR_INVALID_ARGUMENT for every < 1. */
#define SV_PROFILE_ROWS 0
#define SV_PROFILE_REQUEST 1
#define SV_PROFILE_ROWS_FIRST 2
int spec_verify_profile_start(uint32_t kernel_mask, int32_t capacity);
int spec_verify_profile_every(int32_t every);
int spec_verify_profile_stop(double* total_ms, int32_t* launches);

/*
 * spec_verify_probs - dense batch, rejection-sampling verification.
 *
 *  target_logits  [B, gamma+1, V] contiguous, dtype `logits_dtype`; row
 *                 gamma of each request is its bonus row.
 *  draft_probs    [B, gamma, V] fp32 contiguous, or NULL for one-hot drafts
 *                 (q = onehot(x): accept with probability p(x), residual = p
 *                 without x).
 *  draft_tokens   [B, gamma] int64.
 *  uniforms       [B, gamma+1] fp32 (see the uniform convention above).
 *  num_requests B >= 0, gamma >= 0, 1 <= vocab_size V <= SV_MAX_VOCAB.
 *  temperature    T >= 0 and finite (double, so that callers, kernels and
 *                 references agree on the exact value); T == 0 runs the
 *                 greedy kernel (draft_probs and uniforms are then not read).
 *  flags          SV_FLAG_* bits.
 *  out_tokens     [B, gamma+1] int64: x_1..x_n, then the drawn token, then -1.
 *  num_accepted   [B] int32: n, the number of accepted drafts.
 *  row_stats      [B, gamma+1, 4] fp32 or NULL: per target row
 *                 {max(l/T), ln sum exp(l/T - max), p(x), R}; R = sum
 *                 max(0, p - q) for draft rows; p(x) = NaN and R = 1 for bonus
 *                 rows. Requires T > 0. Implies SV_FLAG_ALL_RESIDUALS.
 *                 Statistics come at the cost of reading every q row.
 *  workspace      device scratch of at least
 *                 spec_verify_workspace_size(B * (gamma + 1), V) bytes, see
 *                 the workspace note above.
 */
int spec_verify_probs(const void* target_logits, int logits_dtype, const float* draft_probs,
                      const int64_t* draft_tokens, const float* uniforms, int32_t num_requests,
                      int32_t gamma, int32_t vocab_size, double temperature, uint32_t flags,
                      int64_t* out_tokens, int32_t* num_accepted, float* row_stats,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_probs_noalloc - spec_verify_probs for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The same verification and arguments as
 * spec_verify_probs, minus the workspace: the library's own fixed device
 * array of SV_NOALLOC_SCRATCH_BYTES takes its place (one per device, held
 * until the process ends).
 *  - Allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *  - A batch that needs more (spec_verify_workspace_size(B * (gamma + 1), V)
 *    above SV_NOALLOC_SCRATCH_BYTES) returns SV_ERR_WORKSPACE and launches
 *    nothing.
 *  - Every call on a device shares that device's array: calls that overlap
 *    in time on one device (several streams or host threads) race and must
 *    be ordered by the caller (one stream, or events).
 *  - The first call on a device looks up the array's address and enqueues a
 *    zero-fill of it on `stream`, ahead of its own kernels; every completed
 *    call leaves the array ready for the next call of any shape.
 */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)
int spec_verify_probs_noalloc(const void* target_logits, int logits_dtype, const float* draft_probs,
                              const int64_t* draft_tokens, const float* uniforms, int32_t num_requests,
                              int32_t gamma, int32_t vocab_size, double temperature, uint32_t flags,
                              int64_t* out_tokens, int32_t* num_accepted, float* row_stats, void* stream);

/*
 * spec_verify_greedy - dense batch, argmax verification (temperature 0; the
 * pages' temp=0 decoding, bloss0m.com Table 2). A draft is kept while it
 * equals the argmax of its target row (lowest index on ties); the emitted
 * token is the argmax of the first mismatching row, or of the bonus row.
 * Shapes and outputs as in spec_verify_probs; no q, no uniforms.
 */
int spec_verify_greedy(const void* target_logits, int logits_dtype, const int64_t* draft_tokens,
                       int32_t num_requests, int32_t gamma, int32_t vocab_size,
                       int64_t* out_tokens, int32_t* num_accepted, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * spec_verify_ragged - flattened batch with per-request draft counts (the
 * vLLM verification path on blog.vllbc.top scans requests through
 * cu_num_draft_tokens; the layout below is this library's own).
 *
 *  cu_num_draft_tokens [B+1] int32 device: cu[0] = 0, request b owns draft
 *                 rows cu[b]..cu[b+1]-1 and target rows cu[b]+b..cu[b+1]+b
 *                 (the last is its bonus row); g_b = cu[b+1]-cu[b] >= 0.
 *  target_logits  [num_draft_tokens + B, V].
 *  draft_probs    [num_draft_tokens, V] fp32, or NULL (one-hot drafts).
 *  draft_tokens   [num_draft_tokens] int64.
 *  uniforms       [num_draft_tokens + B] fp32 in target-row layout.
 *  out_tokens     [num_draft_tokens + B] int64, target-row layout, -1 padded.
 *  num_accepted   [B] int32.  row_stats [num_draft_tokens + B, 4] or NULL.
 *  Temperature 0 runs the greedy kernel on the same layout.
 */
int spec_verify_ragged(const void* target_logits, int logits_dtype, const float* draft_probs,
                       const int64_t* draft_tokens, const int32_t* cu_num_draft_tokens,
                       const float* uniforms, int32_t num_requests, int32_t num_draft_tokens,
                       int32_t vocab_size, double temperature, uint32_t flags,
                       int64_t* out_tokens, int32_t* num_accepted, float* row_stats,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_probs_filtered / spec_verify_ragged_filtered - the same
 * verification on a target adjusted by top-k and top-p (blog.vllbc.top, the
 * note on paper §2.2: like the temperature, top-k and top-p fold into the
 * adjusted p, and the rejection sampling then runs on it; the draft
 * probabilities must arrive already adjusted by the drafter's own settings).
 * The pages give no further detail; this library's reading:
 *  - the filters act on the temperature-scaled target, top-k first, then
 *    top-p on the renormalised top-k distribution;
 *  - both are thresholds on the logit value, ties kept: top-k keeps every
 *    token whose logit is >= the top_k-th largest logit (counted with
 *    multiplicity); top-p then keeps every token whose logit is >= t, t the
 *    largest logit value whose tokens at or above it carry at least top_p of
 *    the top-k mass (the boundary inclusive);
 *  - p = the softmax renormalised over the kept tokens and 0 elsewhere, for
 *    every target row (draft positions and the bonus row); a draft token
 *    outside the kept set has p(x) = 0 and is rejected.
 *  top_k          <= 0 or >= vocab_size: no top-k.
 *  top_p          in (0, 1]; 1: no top-p. Anything else (or NaN) is
 *                 SV_ERR_INVALID_ARGUMENT.
 *  temperature    > 0 and finite (greedy verification has no use for
 *                 the filters: the argmax is always kept).
 *  draft_probs    required (not NULL).
 * Every other argument as in spec_verify_probs / spec_verify_ragged (no
 * flags, no row statistics: the default lazy mode). Results equal
 * exact-arithmetic results; the top-p comparison is certified in fp32 and
 * settled in fp64 when within the bound, so only a top-p mass within about
 * 1e-12 relative of the target can come out either way. Same workspace
 * size. With both filters off the results are those of spec_verify_probs /
 * spec_verify_ragged.
 */
int spec_verify_probs_filtered(const void* target_logits, int logits_dtype, const float* draft_probs,
                               const int64_t* draft_tokens, const float* uniforms, int32_t num_requests,
                               int32_t gamma, int32_t vocab_size, double temperature, int32_t top_k, double top_p,
                               int64_t* out_tokens, int32_t* num_accepted, void* workspace, size_t workspace_bytes,
                               void* stream);
int spec_verify_ragged_filtered(const void* target_logits, int logits_dtype, const float* draft_probs,
                                const int64_t* draft_tokens, const int32_t* cu_num_draft_tokens,
                                const float* uniforms, int32_t num_requests, int32_t num_draft_tokens,
                                int32_t vocab_size, double temperature, int32_t top_k, double top_p,
                                int64_t* out_tokens, int32_t* num_accepted, void* workspace,
                                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H_ */
