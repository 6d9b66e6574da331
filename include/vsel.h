/* vsel.h -- vocab-row selection on one MI355X (gfx950) GPU.
 *
 * A C ABI over hand-written HIP kernels that reduce batches of
 * vocabulary-sized logit rows to token choices, so that only the few values a
 * sampler needs leave the device:
 *
 *   vsel_argmax       first-maximum argmax per row
 *   vsel_argmax_excluding
 *                     the greedy serving argmax: excluded ids masked inside
 *                     the reduction, a status word per row
 *   vsel_topk         exact top-k (value, token id) per row, fused with the
 *                     row's argmax and log-sum-exp in one pass over the row
 *   vsel_topk_noalloc vsel_topk with its scratch in a fixed device array, for
 *                     callers that cannot allocate
 *   vsel_sample       temperature sampling with top-k then top-p, one caller
 *                     uniform per row
 *   vsel_sample_chain the ordered sampler chain: top-n-sigma, top-k,
 *                     typical-p, top-p, min-p, then the temperature
 *   vsel_spec_match   speculative-decoding acceptance by sampler-match and
 *                     the per-position sum p*q
 *   vsel_spec_accept  speculative-decoding acceptance: modified rejection
 *                     sampling and argmax-against-argmax, with the per-position
 *                     coupling sum of min(p, q)
 *   vsel_spec_accept_filtered, vsel_spec_match_filtered
 *                     the same rules with p and q filtered by top-k, top-p
 *                     and min-p before the temperature
 *
 * Common conventions
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     where marked "host".  The library never allocates, frees or
 *     synchronises; every call is asynchronous on `stream` (a hipStream_t; NULL
 *     is the default stream).  Inputs are never written.
 *   - A row is `vocab` valid elements at a stride of `ld` elements (ld >= vocab);
 *     elements in [vocab, ld) are never read.  Rows are float32 (VSEL_F32) or
 *     bfloat16 (VSEL_BF16), which widens exactly to float32.  The element
 *     pointer must be aligned to its element size; rows whose start is 16-byte
 *     aligned take the vector-load path.
 *   - Token ids are uint32 in [0, vocab); vocab must be below 2^31.
 *   - Order between elements: a before b iff x_a > x_b, or x_a == x_b and
 *     a < b.  Comparisons are float comparisons, so -0.0 and +0.0 tie and the
 *     lower index wins.
 *   - Fail closed: a row holding a NaN or +inf has VSEL_NONFINITE in its index
 *     or token output and its other outputs are undefined (NaN where floating
 *     point).  -inf is a legal mask value; a row with no element above -inf
 *     has no argmax (VSEL_NONFINITE) but still has a well-defined top-k.
 *   - Workspace: device scratch of at least vsel_workspace_bytes(...) bytes,
 *     zero-filled ONCE by the caller after allocation.  Calls leave the
 *     counters they use at zero again, so a workspace can be reused by later
 *     calls of the same operation with the same rows, vocab and k (the
 *     arguments it was sized for) on the same stream (calls that share a
 *     workspace must be ordered on one stream).  Before using it for other
 *     arguments, or after a call that failed on the device, zero it again.
 *   - Errors are returned synchronously, before anything is launched:
 *     VSEL_EINVAL for a bad argument, VSEL_EWORKSPACE for a workspace that is
 *     too small or misaligned (256 bytes), VSEL_EDEVICE when a launch fails.
 */
#ifndef VSEL_H
#define VSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VSEL_OK = 0,
  VSEL_EINVAL = 1,
  VSEL_EWORKSPACE = 2,
  VSEL_EDEVICE = 3
} vsel_status;

typedef enum { VSEL_F32 = 0, VSEL_BF16 = 1 } vsel_dtype;

typedef enum {
  VSEL_OP_ARGMAX = 0,
  VSEL_OP_TOPK = 1,
  VSEL_OP_SAMPLE = 2,
  VSEL_OP_SPEC_ACCEPT = 3,
  VSEL_OP_SAMPLE_CHAIN = 4,
  VSEL_OP_SPEC_FILTERED = 5
} vsel_op;

/* Index/token written for a fail-closed row: the high-bit latch of the greedy
 * serving kernel, whose 0xffffffff result the caller turns into a hard error
 * ("Chapter 21 - Sampling, argmax, and grammar", sections 21.4 and 21.6). */
#define VSEL_NONFINITE 0xFFFFFFFFu

/* Largest k accepted by vsel_topk and vsel_sample. */
#define VSEL_K_MAX 1024

/* Library version, (major << 16) | minor. */
int vsel_version(void);

/* Short text for a vsel_status value (static storage). */
const char* vsel_status_string(int status);

/* Workspace bytes an operation needs.
 *   VSEL_OP_ARGMAX:      rows, vocab; k ignored.
 *   VSEL_OP_TOPK:        rows, vocab, k.
 *   VSEL_OP_SAMPLE:      rows, vocab, k = top_k (the same as VSEL_OP_SAMPLE_CHAIN).
 *   VSEL_OP_SPEC_ACCEPT: rows = batch, vocab, k = gamma.
 *   VSEL_OP_SAMPLE_CHAIN: rows, vocab, k = top_k.
 *   VSEL_OP_SPEC_FILTERED: rows = batch, vocab, k = gamma (any filters).
 * Returns 0 for arguments the operation would reject. */
size_t vsel_workspace_bytes(int op, int dtype, int64_t rows, int64_t vocab, int32_t k);

/* First-maximum argmax of each row.
 * The reduction of one row to the (value, index) pair of its maximum with a
 * strictly-greater comparison, so ties keep the lower index -- the scalar
 * first-maximum convention ("Chapter 21", section 21.3 and Figure 21.1; the
 * fail-closed greedy variant of section 21.4).
 *   logits  [rows, ld] elements of `dtype`
 *   out_idx [rows] uint32: the argmax, or VSEL_NONFINITE
 *   out_val [rows] float32 or NULL: the maximum (the row's own bits)
 */
vsel_status vsel_argmax(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                        uint32_t* out_idx, float* out_val, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Largest excluded-id set accepted by vsel_argmax_excluding. */
#define VSEL_EXCLUDED_MAX 256

/* Greedy serving argmax with an excluded-id set and a status word per row.
 * The production greedy kernel of "Chapter 21", section 21.4: the request's
 * end-of-generation ids are masked inside the reduction (taken as -inf; the
 * logits are not modified) and the fail-closed latch is reported per row.
 *   excluded   [n_excluded] uint32 device ids, any order; duplicates and ids
 *              >= vocab are allowed and exclude nothing more.  One set for
 *              every row of the call.  NULL when n_excluded == 0.
 *   n_excluded 0 <= n_excluded <= VSEL_EXCLUDED_MAX
 *   out_idx    [rows] uint32: the first maximum of the non-excluded elements,
 *              VSEL_NONFINITE whenever out_status is not 0
 *   out_status [rows] uint32: 0 ok; 1 the row holds a NaN or +inf, at an
 *              excluded id or not; 2 no non-excluded element above -inf
 *   workspace  as for VSEL_OP_ARGMAX with the same rows and vocab
 */
vsel_status vsel_argmax_excluding(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                                  const uint32_t* excluded, int32_t n_excluded, uint32_t* out_idx,
                                  uint32_t* out_status, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Exact top-k of each row, fused with its argmax and log-sum-exp.
 * After decode, the k largest logits of each row are selected on the device
 * and gathered with their token ids, so that only k candidates per row are
 * copied off the device (llama.cpp PR #49, "Change": top_k + get_rows per
 * device share; the candidates hold the k largest logits with tokens and
 * values).  Candidates are ordered by value descending, then id ascending;
 * with that order the result is unique.
 *   k          1 <= k <= min(vocab, VSEL_K_MAX)
 *   out_vals   [rows, k] float32: the selected elements' own values
 *   out_ids    [rows, k] uint32 token ids (out_ids[r*k] is VSEL_NONFINITE for
 *              a fail-closed row)
 *   out_argmax [rows] uint32 or NULL: first-maximum argmax (= out_ids[r*k] for
 *              a row with an element above -inf)
 *   out_lse    [rows] float32 or NULL: log sum_i exp(x_i) (temperature 1);
 *              -inf for an all -inf row
 */
vsel_status vsel_topk(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, int32_t k,
                      float* out_vals, uint32_t* out_ids, uint32_t* out_argmax, float* out_lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/* vsel_topk for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments and outputs as vsel_topk, with no workspace
 * argument.  Its scratch is a fixed device array of
 * VSEL_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; the call itself allocates nothing.  Every call on a GPU shares
 * that GPU's array, so calls that overlap on one GPU (on two streams, or beside
 * a replay of a graph that captured a call) race; calls ordered on one stream
 * do not.  A device's first call also launches a small kernel, on `stream`,
 * that zeroes the array's counters.
 *   rows        1 <= rows <= VSEL_NOALLOC_MAX_ROWS, else VSEL_EINVAL
 *   Shapes whose scratch (for the call's own segment plan) exceeds the array
 *   return VSEL_EWORKSPACE before any launch; the large decode batch
 *   (1,024 x 202,048, k <= 128) needs about 82 KiB.  VSEL_EDEVICE: no current
 *   device, or a launch failed.
 */
#define VSEL_NOALLOC_MAX_ROWS 16384
#define VSEL_NOALLOC_SCRATCH_BYTES (8u << 20)
vsel_status vsel_topk_noalloc(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld, int32_t k,
                              float* out_vals, uint32_t* out_ids, uint32_t* out_argmax, float* out_lse,
                              void* stream);

/* Temperature sampling with top-k then top-p and one caller uniform per row.
 * Filtering acts on the untempered distribution and the temperature is applied
 * last ("speculative-acceptance.md", "The rules": p is the target
 * distribution after top-k / top-p filtering on the untempered distribution and
 * the final temperature scaling; the ordered chain top_k then top_p of
 * "Chapter 21", section 21.7).  Per row, with candidates c_0.. in (value desc,
 * id asc) order:
 *   1. temperature == 0 or top_k == 1: the argmax token, logprob 0 (greedy
 *      draws nothing, "speculative-acceptance.md", "RNG dependency").
 *   2. candidates: the top min(top_k, vocab) elements; top_k == 0 means the
 *      whole row: in id order when top_p == 1, else in (value desc, id asc)
 *      order for the cut and the draw (vsel_sample_chain with top_p alone).
 *   3. p0_j = exp(z_j - z_0) / sum over candidates (untempered).
 *   4. keep the first n >= 1 candidates, n the smallest with
 *      p0_0 + ... + p0_{n-1} >= top_p (all of them when top_p == 1).
 *   5. w_j = exp((z_j - z_0) / temperature) over the kept set, W = sum w_j.
 *   6. token = c_j for the first j with u*W < w_0 + ... + w_j (float64), else
 *      the last kept candidate with w_j > 0.
 *   out_logprob = log(w_j / W), the log-probability under the distribution
 *   actually drawn from.
 *   temperature >= 0, 0 <= top_k <= VSEL_K_MAX, 0 < top_p <= 1; with
 *   top_k == 0, vocab <= 67,108,864 (256 segments of 1,024 chunks of 256).
 *   The workspace (VSEL_OP_SAMPLE) has the layout of VSEL_OP_SAMPLE_CHAIN.
 *   u           [rows] float32 in [0, 1)
 *   out_token   [rows] uint32 (VSEL_NONFINITE for a fail-closed row)
 *   out_logprob [rows] float32 or NULL
 */
vsel_status vsel_sample(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                        float temperature, int32_t top_k, float top_p, const float* u,
                        uint32_t* out_token, float* out_logprob, void* workspace,
                        size_t workspace_bytes, void* stream);

/* The ordered sampler chain with one caller uniform per row ("Chapter 21",
 * section 21.7: top_n_sigma masking against the maximum, top_k, typical_p,
 * then the top_p nucleus; min_p a filter on the untempered distribution too,
 * and the temperature applied last, "speculative-acceptance.md", "The rules").
 * Per row, starting from the whole row in id order; each filter keeps at
 * least one candidate:
 *   1. top_n_sigma > 0: keep z >= z_max - top_n_sigma * sigma, sigma the
 *      population standard deviation of the row's elements above -inf
 *      (order unchanged);
 *   2. top_k > 0: the top min(top_k, candidates) in (value desc, id asc) order;
 *   3. typical_p < 1: p = softmax of the candidates, H = -sum p log p; reorder
 *      by |-log p - H| ascending (ties keep value order) and keep the
 *      shortest prefix with sum p >= typical_p;
 *   4. top_p < 1: back to (value desc, id asc) order, keep the shortest prefix
 *      with sum p >= top_p (p the softmax of the candidates left);
 *   5. min_p > 0: keep z >= max z + log(min_p), i.e. p >= min_p * max p
 *      (order unchanged);
 *   6. w = exp((z - z_max) / temperature) over the kept candidates, the
 *      inverse-CDF draw with u in their current order (float64), and
 *      out_logprob = log(w_j / W).
 * temperature == 0 or top_k == 1: the argmax token, logprob 0.  With all
 * filters off except top_k / top_p this is vsel_sample.
 *   temperature >= 0 and finite; top_n_sigma >= 0 and finite;
 *   0 <= top_k <= VSEL_K_MAX; 0 < typical_p <= 1; 0 < top_p <= 1;
 *   0 <= min_p <= 1.  With top_k == 0,
 *   vocab <= 67,108,864, and the filters act on the whole row: typical_p < 1
 *   orders it by |z - c| (c = the p-weighted mean of z, since -log p - H =
 *   c - z), then id; top_p < 1 orders it (or the typical set) by value, and
 *   the draw follows the last order (with neither, id order, as in
 *   vsel_sample).  The typical order compares the float64 distances with
 *   their mantissas cut to 30 bits (distances within 2^-30 relative of each
 *   other tie and fall to the lower id).
 *   u, out_token, out_logprob as vsel_sample; workspace VSEL_OP_SAMPLE_CHAIN
 *   with k = top_k.
 */
vsel_status vsel_sample_chain(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                              float temperature, float top_n_sigma, int32_t top_k, float typical_p,
                              float top_p, float min_p, const float* u, uint32_t* out_token,
                              float* out_logprob, void* workspace, size_t workspace_bytes, void* stream);

/* Speculative-decoding acceptance for `batch` sequences of `gamma` drafts.
 * p_i = softmax(target row i / T), q_i = softmax(draft row i / T).
 * Modified rejection sampling ("speculative-acceptance.md", "Modified
 * rejection sampling"; the exact acceptance of "Chapter 21", section 21.9):
 * accept draft t_i iff u_accept[i] * q_i(t_i) <= p_i(t_i) (q = 0 accepts);
 * at the first rejection L emit one token drawn from normalize(max(p_L - q_L,
 * 0)) with u_resid[L] (from p_L if that residual sums to 0) and stop; if all
 * gamma drafts are accepted emit a bonus token drawn from p_gamma (the last
 * target row) with u_bonus.  Draws take tokens in id order: the first x with
 * u*W < w_0 + ... + w_x.  Argmax-against-argmax ("speculative-acceptance.md",
 * "Argmax-against-argmax"): accept iff t_i == argmax of target row i and emit
 * that argmax at the first mismatch.  summin_i = sum_x min(p_i(x), q_i(x)), the
 * acceptance ceiling of any distribution-preserving rule ("The acceptance
 * ceiling"), for every position.  temperature == 0 is greedy: both rules are
 * argmax-against-argmax and summin_i is 1 where the two argmaxes agree, else 0.
 *   1 <= gamma <= 256; temperature >= 0 and finite; vocab <= 67,108,864
 *   target_logits [batch*(gamma+1), ld_t] float32; row b*(gamma+1)+i is verify
 *                 position i of sequence b (row b*(gamma+1)+gamma: bonus row)
 *   draft_logits  [batch*gamma, ld_d] float32
 *   draft_tokens  [batch*gamma] uint32
 *   u_accept, u_resid [batch*gamma] float32 in [0, 1); u_bonus [batch]
 *   out_len_mrs   [batch] int32: accepted drafts L in [0, gamma], or -1 for a
 *                 fail-closed sequence (a nonfinite row, or a draft id >= vocab)
 *   out_tok_mrs   [batch*(gamma+1)] uint32: t_0..t_{L-1} then the drawn token;
 *                 the remaining slots VSEL_NONFINITE
 *   out_len_aa, out_tok_aa: the same for argmax-against-argmax (may be NULL)
 *   out_summin    [batch*gamma] float32 or NULL
 *   out_sumprod   [batch*gamma] float32 or NULL: sum_x p_i(x) q_i(x), the
 *                 sampler-match rule's acceptance probability, from the same
 *                 pass ("Verifying the gain before trusting a throughput
 *                 number" reads both closed forms for one run)
 */
vsel_status vsel_spec_accept(const float* target_logits, int64_t ld_t, const float* draft_logits,
                             int64_t ld_d, int64_t batch, int32_t gamma, int64_t vocab,
                             float temperature, const uint32_t* draft_tokens, const float* u_accept,
                             const float* u_resid, const float* u_bonus, int32_t* out_len_mrs,
                             uint32_t* out_tok_mrs, int32_t* out_len_aa, uint32_t* out_tok_aa,
                             float* out_summin, float* out_sumprod, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Speculative-decoding acceptance by sampler-match ("speculative-acceptance.md",
 * "The rules": sampler-match, the default rule at temperature > 0): at verify
 * position i a fresh token x_i is drawn from p_i with u_match[i] (id order,
 * the first x with u*W < w_0 + ... + w_x over W = sum of p_i), and draft t_i
 * is accepted iff x_i == t_i.  The chain stops at the first mismatch L (or at
 * gamma, where x_gamma is drawn from the bonus row) and emits t_0 .. t_{L-1},
 * x_L: the draw is emitted on both branches, so the stream is a target-only
 * sample.  sumprod_i = sum_x p_i(x) q_i(x), the rule's acceptance probability
 * for a proposal drawn from q ("The acceptance ceiling"; the diagnostic of
 * "Verifying the gain before trusting a throughput number"), for every
 * position.  temperature == 0 is greedy: the sampler is argmax, so the rule is
 * argmax-against-argmax and sumprod_i is 1 where the two argmaxes agree.
 *   Shapes, limits and fail-closed sequences as vsel_spec_accept; workspace as
 *   VSEL_OP_SPEC_ACCEPT with the same batch, vocab and gamma.
 *   u_match     [batch*(gamma+1)] float32 in [0, 1): position i of sequence b
 *               at b*(gamma+1) + i, the bonus draw at b*(gamma+1) + gamma
 *   out_len     [batch] int32: accepted drafts L in [0, gamma], or -1
 *   out_tok     [batch*(gamma+1)] uint32: t_0..t_{L-1} then x_L; the rest
 *               VSEL_NONFINITE
 *   out_sumprod [batch*gamma] float32 or NULL
 */
vsel_status vsel_spec_match(const float* target_logits, int64_t ld_t, const float* draft_logits,
                            int64_t ld_d, int64_t batch, int32_t gamma, int64_t vocab,
                            float temperature, const uint32_t* draft_tokens, const float* u_match,
                            int32_t* out_len, uint32_t* out_tok, float* out_sumprod,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Speculative-decoding acceptance with filtered distributions
 * ("speculative-acceptance.md", "The rules": p is the target's distribution
 * after top-k / top-p / min-p filtering on the untempered distribution and the
 * final temperature scaling; q the distribution the drafter drew from, here
 * under the same sampler settings).  For every target and draft row:
 *   1. top_k > 0: the top min(top_k, vocab) elements, (value desc, id asc);
 *      top_k == 0: the whole row, in that order when top_p < 1;
 *   2. top_p < 1: the shortest prefix whose cumulative untempered probability
 *      (softmax of the candidates) reaches top_p;
 *   3. min_p > 0: z >= max z + log(min_p) over the candidates;
 *   p(x) = exp(z_x/T) / sum over the kept ids, 0 for the others.
 * The rules, draws, outputs, limits and fail-closed sequences are those of
 * vsel_spec_accept and vsel_spec_match with these p and q (a drafted token
 * outside the draft's kept set has q = 0 and is accepted by the modified
 * rejection test).  temperature == 0 is greedy and ignores the filters.
 *   0 <= top_k <= VSEL_K_MAX, 0 < top_p <= 1, 0 <= min_p <= 1
 *   workspace: VSEL_OP_SPEC_FILTERED with rows = batch, k = gamma
 */
vsel_status vsel_spec_accept_filtered(const float* target_logits, int64_t ld_t, const float* draft_logits,
                                      int64_t ld_d, int64_t batch, int32_t gamma, int64_t vocab,
                                      float temperature, int32_t top_k, float top_p, float min_p,
                                      const uint32_t* draft_tokens, const float* u_accept,
                                      const float* u_resid, const float* u_bonus, int32_t* out_len_mrs,
                                      uint32_t* out_tok_mrs, int32_t* out_len_aa, uint32_t* out_tok_aa,
                                      float* out_summin, float* out_sumprod, void* workspace, size_t workspace_bytes,
                                      void* stream);

vsel_status vsel_spec_match_filtered(const float* target_logits, int64_t ld_t, const float* draft_logits,
                                     int64_t ld_d, int64_t batch, int32_t gamma, int64_t vocab,
                                     float temperature, int32_t top_k, float top_p, float min_p,
                                     const uint32_t* draft_tokens, const float* u_match, int32_t* out_len,
                                     uint32_t* out_tok, float* out_sumprod, void* workspace,
                                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSEL_H */
