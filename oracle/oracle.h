/*
 * oracle.h -- plain, single-threaded CPU oracle for the speculative-decoding
 * verification step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may call this library.  It shares no code,
 * header, table or helper with the GPU library and never calls it.
 *
 * What it computes (all arithmetic in double, logits read as float32 values,
 * which represent fp32, fp16 and bf16 inputs exactly):
 *
 *  - oracle_sample_seq: the sampling-mode acceptance rule exactly as the
 *    production blog "Speculative Decoding: Faster Generation Without Changing
 *    the Model" states it (section "The acceptance rule"): drafts are examined
 *    left to right, x_i is kept with probability min(1, p(x_i)/q(x_i)); the
 *    first rejection is replaced by a draw from the residual proportional to
 *    max(0, p - q) and the round ends; if every draft survives, one bonus token
 *    is drawn from p at position k+1.  The Cascade Speculative Drafting page
 *    (section "The Vertical Cascade", review function, lenience l = 1) states
 *    the same rule as "accept if q <= p, else reject with probability 1 - p/q",
 *    which also fixes the q(x) = 0 corner: accept.
 *
 *  - oracle_greedy_seq: the greedy collapse of that rule (same blog section):
 *    accept while x_i equals the target argmax, replace the first mismatch by
 *    the argmax; if all k survive the bonus is the argmax at position k+1.
 *
 *  - oracle_greedy_candidates_seq: longest-accepted-candidate selection over C
 *    candidate drafts verified in one pass (Ouroboros page, section 3.4.3
 *    "Lengthening Drafts via Phrases", "Selecting the accepted tokens",
 *    Stage 1 / Stage 2 and the case equation for the accepted suffix length).
 *
 * Conventions fixed here because the pages leave them open (each is a reading,
 * listed again in the design notes):
 *  - p = softmax(z / T), q = softmax(y / T): the temperature is applied to
 *    target and draft alike.
 *  - one uniform u_i per draft position decides acceptance: accept iff
 *    u_i < min(1, p/q) (strict).  A single further uniform u_k drives the one
 *    sampling step of the round (residual or bonus) by inverse CDF: the
 *    smallest token index t whose running sum of weights (ascending t) exceeds
 *    u_k times the total.  If rounding leaves no crossing, the largest t with
 *    positive weight is taken.  A residual whose total is 0 falls back to p.
 *  - argmax: the lowest index among equal maxima; NaN never wins; a row with
 *    no value above -inf yields index 0.  Greedy ignores the temperature.
 *  - a draft token outside [0, V) is rejected (its p and q are taken as 0).
 *  - sampling rows must hold at least one finite logit and no +inf / NaN.
 *
 * Layouts: a logit row is V contiguous floats; consecutive rows of one
 * sequence are `row_stride` floats apart.  Target rows of a sequence: k+1,
 * draft rows: k.  Output tokens: k+1 ints, -1 past the committed count.
 * All buffers are host memory owned by the caller.
 */
#ifndef SPEC_ORACLE_H
#define SPEC_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_MAX_K 63

/* Per-round record of what the sampling oracle decided and how close each
 * decision was to its boundary (used to classify rounding-tie rounds). */
typedef struct {
    int evaluated;                      /* draft positions whose acceptance was decided */
    int num_accepted;                   /* j: accepted drafts */
    int sample_kind;                    /* 0 residual, 1 bonus, 2 residual total was 0 -> p */
    int sampled_token;
    double ratio[ORACLE_MAX_K + 1];     /* min(1, p/q) at evaluated positions (0 if invalid token) */
    double accept_margin[ORACLE_MAX_K + 1]; /* |u_i - ratio_i|; 1 - u_i when q <= p */
    double p_x[ORACLE_MAX_K + 1];       /* p_i(x_i) at evaluated positions */
    double q_x[ORACLE_MAX_K + 1];       /* q_i(x_i) at evaluated positions */
    double sample_total;                /* total weight of the sampled distribution */
    double sample_lo;                   /* CDF(t*-1)/total */
    double sample_hi;                   /* CDF(t*)/total */
    double sample_margin;               /* min(u_k - lo, hi - u_k) */
} oracle_trace;

/* Deliberate mistakes, planted only to show that the statistical pins have the
 * power to catch them.  ORACLE_MUT_NONE is the oracle. */
enum {
    ORACLE_MUT_NONE = 0,
    ORACLE_MUT_RESIDUAL_IS_P = 1,     /* resample from p instead of the residual */
    ORACLE_MUT_RESIDUAL_IS_Q = 2,     /* resample from q */
    ORACLE_MUT_BONUS_FROM_Q = 3,      /* bonus drawn from the last draft row */
    ORACLE_MUT_RATIO_INVERTED = 4,    /* accept with min(1, q/p) */
    ORACLE_MUT_RESIDUAL_SIGN = 5      /* residual max(0, q - p) */
};

/* Status codes: 0 ok, -1 bad arguments, -2 out of memory, -3 a sampling row
 * with no finite logit. */

int oracle_greedy_seq(const float* target, long long row_stride, const int* draft_tokens,
                      int k, int V, int* out_tokens, int* out_num_accepted);

int oracle_sample_seq(const float* target, long long target_row_stride,
                      const float* draft, long long draft_row_stride,
                      const int* draft_tokens, const float* uniforms, double temperature,
                      int k, int V, int* out_tokens, int* out_num_accepted,
                      oracle_trace* trace);

/* Same rule with one planted mistake (tests of the pins only). */
int oracle_sample_seq_mutant(const float* target, long long target_row_stride,
                             const float* draft, long long draft_row_stride,
                             const int* draft_tokens, const float* uniforms, double temperature,
                             int k, int V, int* out_tokens, int* out_num_accepted,
                             oracle_trace* trace, int mutation);

/* Sampling rule with lenience l >= 1 (Cascade Speculative Drafting, "The
 * Vertical Cascade", the review function): accept if q(x) <= l p(x), else
 * reject with probability 1 - l p(x)/q(x), i.e. accept iff u < min(1, l p/q);
 * the residual stays max(0, p - q).  l = 1 is oracle_sample_seq. */
int oracle_sample_lenient(const float* target, long long target_row_stride,
                          const float* draft, long long draft_row_stride,
                          const int* draft_tokens, const float* uniforms, double temperature,
                          double lenience, int B, int k, int V, int* out_tokens,
                          int* out_num_accepted, oracle_trace* traces);

/* Sampling rule on truncated distributions: top-k then top-p applied to the
 * target's and the draft's rows alike (the production blog, "Integration with
 * the serving engine" and "Failure modes": a processor applied to one side
 * and not the other breaks the q the rule relies on; Ouroboros samples with
 * top-p 0.8).  Per row, with w_t = exp(z_t/T - max):
 *   top-k (top_k >= 1, top_k < V): keep t iff fewer than top_k tokens have a
 *     strictly larger logit (ties at the boundary all kept);
 *   top-p (0 < top_p < 1): among the tokens top-k kept, keep t iff the kept
 *     tokens with strictly larger logits hold less than top_p of the kept mass
 *     (the smallest set of top tokens reaching top_p, ties kept together);
 *   p' = w / (sum of w over kept tokens) on kept tokens, 0 elsewhere.
 * top_k = 0 and top_p >= 1 switch the respective step off.  The rule then
 * runs on p' and q'.  trace->sample_* refer to p', q'.  `trunc_margin`, if
 * not NULL, gets per sequence the smallest distance, over every row the round
 * read, between top_p and the kept-mass fraction at either side of the top-p
 * boundary (1 where top-p is off). */
int oracle_sample_truncated(const float* target, long long target_row_stride,
                            const float* draft, long long draft_row_stride,
                            const int* draft_tokens, const float* uniforms, double temperature,
                            int top_k, double top_p, int B, int k, int V, int* out_tokens,
                            int* out_num_accepted, oracle_trace* traces, double* trunc_margin);

/* One truncated row: p' as above (out_p[V]); returns 0 or an error. *margin as
 * above for this row. */
int oracle_truncated_row(const float* z, int V, double temperature, int top_k, double top_p,
                         double* out_p, double* margin);

/* Verification by-products of the greedy pass (Ouroboros section 3.4.4,
 * Eq. 10): v_i = argmax of target row i for i <= k (the target's own token at
 * every position, accepted or not), bit i of the match mask = [x_i == v_i]
 * for i < k, and #Match = the number of set bits. */
int oracle_greedy_matches(const float* target, long long row_stride, const int* draft_tokens,
                          int B, int k, int V, int* out_v, unsigned long long* out_mask,
                          int* out_num_match);

/* Multi-candidate greedy selection over a token tree (Ouroboros section 3.4.3,
 * Figure 3: the target scores every node of the tree once; candidates that
 * share a prefix share its rows).  Sequence b has N node rows; cand_rows
 * [B][C][R] names the node row that scores candidate token (c, i) for i < L,
 * and for R = L+1 the row after the last token.  Otherwise as
 * oracle_greedy_candidates (the flat layout is the tree with every row
 * spelled out).  A row index outside [0, N) never matches and yields the
 * correction token -1. */
int oracle_greedy_tree(const float* nodes, long long row_stride, int N, const int* cand_tokens,
                       const int* cand_rows, int B, int C, int L, int R, int V,
                       int* out_tokens, int* out_num_accepted, int* out_best);

/* The argmax of every row (candidates: the verification token of every
 * candidate position, used to correct unused candidates). */
int oracle_row_argmax(const float* rows, long long row_stride, long long n_rows, int V, int* out);

/* p_i(x_i) and q_i(x_i) for every draft position i < k (0 for an invalid x_i). */
int oracle_token_probs_seq(const float* target, long long target_row_stride,
                           const float* draft, long long draft_row_stride,
                           const int* draft_tokens, double temperature, int k, int V,
                           double* out_p_x, double* out_q_x);

/* rows of one sequence: [C][R][V], candidate tokens [C][L]; R is L or L+1.
 * out_tokens has L+1 entries, -1 past the committed count. */
int oracle_greedy_candidates_seq(const float* target, long long row_stride,
                                 const int* cand_tokens, int C, int L, int R, int V,
                                 int* out_tokens, int* out_num_accepted, int* out_best);

/* Batched forms: sequence b's rows start at row b*(k+1) (target), b*k (draft),
 * b*C*R (candidates); per-sequence outputs are laid out contiguously.
 * `mutation` selects a planted mistake (0 = the oracle). `traces` may be NULL. */
int oracle_greedy(const float* target, long long row_stride, const int* draft_tokens,
                  int B, int k, int V, int* out_tokens, int* out_num_accepted);

int oracle_sample(const float* target, long long target_row_stride,
                  const float* draft, long long draft_row_stride,
                  const int* draft_tokens, const float* uniforms, double temperature,
                  int B, int k, int V, int* out_tokens, int* out_num_accepted,
                  oracle_trace* traces, int mutation);

int oracle_greedy_candidates(const float* target, long long row_stride,
                             const int* cand_tokens, int B, int C, int L, int R, int V,
                             int* out_tokens, int* out_num_accepted, int* out_best);

/* The interval [lo, hi] of cumulative probability (ascending token order)
 * that `token` occupies in the distribution one round draws from: the
 * residual max(0, p - q) normalised when `draft_row` is given (p itself if
 * that residual has no mass), else p.  *weight is the token's probability in
 * that distribution.  A draw with uniform u picks `token` exactly when
 * lo <= u < hi.  Used to check that a draw whose u lies within rounding of a
 * boundary picked one of the tokens on either side. */
int oracle_draw_interval(const float* target_row, const float* draft_row, double temperature,
                         int V, int token, double* lo, double* hi, double* weight);

int oracle_trace_size(void);

#ifdef __cplusplus
}
#endif
#endif
