/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) speculative-decoding
 * verification library (libspecverify.so).
 *
 * The operation.  A speculative-decoding round proposes k draft tokens
 * x_0..x_{k-1} per sequence; the target model scores all of them in one pass
 * and returns logits at k+1 positions.  The library applies the acceptance
 * rule to a batch of B sequences and returns the committed tokens and the
 * accepted length of each:
 *
 *  - sampling (production blog "Speculative Decoding: Faster Generation Without
 *    Changing the Model", section "The acceptance rule"; the review function of
 *    "Cascade Speculative Drafting", section "The Vertical Cascade", with
 *    lenience 1): p_i = softmax(target_i / T), q_i = softmax(draft_i / T);
 *    left to right, x_i is accepted iff u_i < min(1, p_i(x_i) / q_i(x_i))
 *    (q_i(x_i) <= p_i(x_i) always accepts); the first rejected position j is
 *    replaced by a draw from max(0, p_j - q_j) normalised, and the round ends;
 *    if all k are accepted, a bonus token is drawn from p_k.
 *  - greedy (same blog section, last sentences): x_i is accepted while it
 *    equals argmax target_i; the first mismatch is replaced by that argmax; if
 *    all k match, the bonus is argmax target_k.
 *  - greedy candidates (Ouroboros, section 3.4.3, "Selecting the accepted
 *    tokens"): C candidate drafts of L tokens verified in one pass; each
 *    candidate's accepted length is its number of leading tokens equal to the
 *    argmax of their rows; the longest wins (lowest candidate index on ties);
 *    its accepted tokens are committed followed by the argmax correction.
 *
 * Conventions shared by every entry point.
 *  - Pointers marked DEVICE are device memory (hipMalloc / torch tensors on
 *    the GPU); the caller owns every buffer.  The library allocates no device
 *    memory: scratch space comes from the caller's `workspace`.
 *  - Logits are row-major: a row is V contiguous elements of `dtype`
 *    (SV_F32 / SV_F16 / SV_BF16); consecutive rows are `*_row_stride`
 *    ELEMENTS apart (stride >= V).  Target rows of sequence b are rows
 *    b*(k+1) .. b*(k+1)+k; draft rows are b*k .. b*k+k-1.  With 16-byte aligned
 *    base pointers and (stride * element size) % 16 == 0 the 16-byte vector
 *    path runs; otherwise an element-wise path gives identical results.
 *  - Draft tokens are int32.  A token outside [0, V) is rejected at its
 *    position (its p and q are reported as 0); it never causes an
 *    out-of-range read.
 *  - Argmax: the lowest index among equal maxima; -0.0 equals +0.0; a row
 *    whose elements are all -inf gives index 0.  Greedy ignores temperature.
 *  - Sampling logits may hold -inf (masked tokens) but must hold at least one
 *    finite value per row and no +inf or NaN; greedy logits must not hold NaN.
 *    Inputs outside these contracts give unspecified tokens (always in
 *    [0, V)), never a fault.
 *  - Uniforms are float32 in [0, 1): `uniforms[b][i]` (i < k) decides draft
 *    i; `uniforms[b][k]` drives the round's single draw (residual or bonus),
 *    made by inverse CDF over the vocabulary in ascending index order: the
 *    smallest token whose cumulative weight exceeds u times the total.
 *  - Outputs: out_tokens[b] holds the committed tokens followed by -1 up to
 *    its row length; out_num_accepted[b] is the number of accepted draft
 *    tokens.  Sampling and greedy commit out_num_accepted[b] + 1 tokens.
 *  - Asynchrony: every call validates its arguments on the host, then enqueues
 *    its kernels on `hip_stream` (a hipStream_t, NULL = the null stream) and
 *    returns without waiting.  Results are valid once the stream reaches
 *    that point.  No host synchronisation, no host/device copies.
 *  - Errors: argument checks run before anything is enqueued; on an error
 *    nothing is launched and the outputs are untouched.  SV_EINVAL: a NULL
 *    required pointer or a size/stride/temperature out of range; SV_EDTYPE:
 *    an unknown dtype; SV_EWORKSPACE: workspace NULL or smaller than
 *    spec_verify_workspace_bytes(); SV_EHIP: a launch failed (the HIP error
 *    is reported by the runtime's error state); SV_ESCRATCH: a call of
 *    spec_verify_sample_noalloc that needs more than its static scratch.
 *  - Re-entrancy: calls keep no state between them; concurrent calls must use
 *    distinct workspaces (spec_verify_sample_noalloc, which has no workspace
 *    argument, shares one static buffer per device).  Results are deterministic: the same inputs and
 *    shapes give bit-identical outputs (no floating-point atomics).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SV_OK = 0, SV_EINVAL = 1, SV_EDTYPE = 2, SV_EWORKSPACE = 3, SV_EHIP = 4, SV_ESCRATCH = 5 };
enum { SV_F32 = 0, SV_F16 = 1, SV_BF16 = 2 };

#define SV_MAX_K 63
#define SV_MAX_CANDIDATE_TOKENS 64
/* Size of the static scratch of spec_verify_sample_noalloc (per device). */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

/* Library version, major * 10000 + minor * 100 + patch. */
int spec_verify_version(void);

/* Human-readable name of a status code (static storage). */
const char* spec_verify_status_string(int status);

/* Bytes of device workspace a call needs.  `rows_per_seq` is the number of
 * logit rows the call reads per sequence: k+1 for spec_verify_greedy, 2k+1 for
 * spec_verify_sample, C*R for spec_verify_greedy_candidates.  The figure
 * covers every call with those rows; a truncated call on fp32 logits with a
 * top-k of at most 256 on few rows (at most 512; V >= 8192 for at most 64
 * rows, else V >= 32768) needs up to 2 MiB more than the other calls, for
 * the candidates of its row slices.  Pure host
 * function; returns 0 for arguments that any call would reject. */
size_t spec_verify_workspace_bytes(int B, int rows_per_seq, int V, int dtype);

/* Greedy verification (see the header comment).
 *   target_logits  DEVICE [B][k+1][V] dtype, rows `target_row_stride` apart
 *   draft_tokens   DEVICE [B][k] int32
 *   1 <= B, 1 <= k <= 63, 1 <= V
 *   out_tokens       DEVICE [B][k+1] int32 (x_0..x_{j-1}, correction, then -1)
 *   out_num_accepted DEVICE [B] int32, j in [0, k]
 *   workspace        DEVICE, >= spec_verify_workspace_bytes(B, k+1, V, dtype) */
int spec_verify_greedy(const void* target_logits, long long target_row_stride,
                       const int* draft_tokens, int B, int k, int V, int dtype,
                       int* out_tokens, int* out_num_accepted,
                       void* workspace, size_t workspace_bytes, void* hip_stream);

/* Sampling verification (see the header comment).
 *   target_logits DEVICE [B][k+1][V], draft_logits DEVICE [B][k][V], same dtype
 *   draft_tokens  DEVICE [B][k] int32, drawn by the proposer from q = softmax(draft / T)
 *   uniforms      DEVICE [B][k+1] float32 in [0, 1)
 *   temperature   > 0 and finite; applied to target and draft logits alike
 *   out_tokens       DEVICE [B][k+1] int32, out_num_accepted DEVICE [B] int32
 *   out_p_x, out_q_x DEVICE [B][k] float32, optional (NULL skips): p_i(x_i) and
 *                    q_i(x_i) at every draft position (0 for invalid tokens)
 *   workspace        DEVICE, >= spec_verify_workspace_bytes(B, 2k+1, V, dtype) */
int spec_verify_sample(const void* target_logits, long long target_row_stride,
                       const void* draft_logits, long long draft_row_stride,
                       const int* draft_tokens, const float* uniforms, float temperature,
                       int B, int k, int V, int dtype,
                       int* out_tokens, int* out_num_accepted,
                       float* out_p_x, float* out_q_x,
                       void* workspace, size_t workspace_bytes, void* hip_stream);

/* Greedy verification plus the by-products of the same pass that phrase
 * harvesting uses (Ouroboros section 3.4.4, Eq. 10; no extra logit bytes):
 *   out_target_argmax DEVICE [B][k+1] int32 or NULL: v_i = argmax target_i at
 *                     every position, accepted or not (the target's own tokens,
 *                     from which the rejected tail's matching runs are read)
 *   out_match_mask    DEVICE [B] uint64 or NULL: bit i (i < k) = [x_i == v_i]
 *   out_num_match     DEVICE [B] int32 or NULL: #Match, the number of set bits
 *                     (always >= out_num_accepted)
 * Other arguments and errors as spec_verify_greedy. */
int spec_verify_greedy_ext(const void* target_logits, long long target_row_stride,
                           const int* draft_tokens, int B, int k, int V, int dtype,
                           int* out_tokens, int* out_num_accepted, int* out_target_argmax,
                           unsigned long long* out_match_mask, int* out_num_match,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/* Sampling verification with lenience l (Cascade Speculative Drafting,
 * section "The Vertical Cascade", the review function): x_i is accepted if
 * q_i(x_i) <= l p_i(x_i), else rejected with probability 1 - l p/q, i.e.
 * iff u_i < min(1, l p/q); the residual stays max(0, p - q).  l must be >= 1
 * and finite (SV_EINVAL otherwise); l = 1 gives exactly spec_verify_sample's
 * results.  With l > 1 the committed tokens are no longer distributed as p:
 * the cascade applies it only where a draft model reviews another draft.
 * Other arguments and errors as spec_verify_sample. */
int spec_verify_sample_lenient(const void* target_logits, long long target_row_stride,
                               const void* draft_logits, long long draft_row_stride,
                               const int* draft_tokens, const float* uniforms, float temperature,
                               float lenience, int B, int k, int V, int dtype,
                               int* out_tokens, int* out_num_accepted,
                               float* out_p_x, float* out_q_x,
                               void* workspace, size_t workspace_bytes, void* hip_stream);

/* Sampling verification on truncated distributions: top-k, then top-p,
 * applied to every target row and every draft row alike (production blog,
 * "Integration with the serving engine" and "Failure modes": a sampling
 * processor applied to one side only breaks the q the rule relies on;
 * Ouroboros samples with top-p 0.8).  Per row, with w_t = exp((z_t - max)/T):
 *   top_k in [1, V): keep t iff fewer than top_k tokens have a strictly
 *     larger logit (equal logits at the boundary all kept);
 *   top_p in (0, 1): among the tokens top-k kept, keep t iff the kept tokens
 *     with strictly larger logits hold less than top_p of the kept mass (the
 *     smallest set of top logits reaching top_p, equal logits kept together);
 *   p'(t) = w_t / (sum of w over kept tokens) on kept tokens, 0 elsewhere.
 * The rule (spec_verify_sample) then runs on p' and q': out_p_x / out_q_x are
 * p'_i(x_i), q'_i(x_i), the residual is max(0, p' - q') and the bonus is drawn
 * from p'_k.  top_k = 0 or top_k >= V turns top-k off, top_p >= 1 turns top-p
 * off; with both off the call is spec_verify_sample.  Errors: SV_EINVAL for
 * top_k < 0, top_p <= 0 or NaN, and V > 2^23 with truncation on (kept masses
 * are summed as 64-bit fixed-point integers, 2^-40 of the row maximum's
 * weight, so that they are reproducible bit for bit).  Other arguments,
 * layouts and errors as spec_verify_sample; the workspace is the same size. */
int spec_verify_sample_truncated(const void* target_logits, long long target_row_stride,
                                 const void* draft_logits, long long draft_row_stride,
                                 const int* draft_tokens, const float* uniforms, float temperature,
                                 int top_k, float top_p, int B, int k, int V, int dtype,
                                 int* out_tokens, int* out_num_accepted,
                                 float* out_p_x, float* out_q_x,
                                 void* workspace, size_t workspace_bytes, void* hip_stream);

/* Multi-candidate greedy verification (see the header comment).
 *   target_logits DEVICE [B][C][R][V]; row (c, i) scores candidate token (c, i).
 *                 R = L (no row after the last token: a fully accepted candidate
 *                 commits L tokens) or R = L+1 (the last row gives one more
 *                 greedy token).
 *   cand_tokens   DEVICE [B][C][L] int32; 1 <= C, 1 <= L <= 63, C*L <= 64
 *   out_tokens         DEVICE [B][L+1] int32, committed tokens then -1
 *   out_num_accepted   DEVICE [B] int32: accepted length A of the chosen candidate
 *   out_best_candidate DEVICE [B] int32: the chosen candidate c*
 *   workspace          DEVICE, >= spec_verify_workspace_bytes(B, C*R, V, dtype) */
int spec_verify_greedy_candidates(const void* target_logits, long long row_stride,
                                  const int* cand_tokens, int B, int C, int L, int R, int V,
                                  int dtype, int* out_tokens, int* out_num_accepted,
                                  int* out_best_candidate,
                                  void* workspace, size_t workspace_bytes, void* hip_stream);

/* Multi-candidate greedy verification plus the argmax of every scored row:
 *   out_target_argmax DEVICE [B][C][R] int32 or NULL: the target's token v at
 *                     every candidate position (Ouroboros 3.4.4: an unused
 *                     candidate c is corrected to its first token followed by
 *                     v(c, 1..)).
 * Other arguments and errors as spec_verify_greedy_candidates. */
int spec_verify_greedy_candidates_ext(const void* target_logits, long long row_stride,
                                      const int* cand_tokens, int B, int C, int L, int R, int V,
                                      int dtype, int* out_tokens, int* out_num_accepted,
                                      int* out_best_candidate, int* out_target_argmax,
                                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* Multi-candidate greedy verification over a token tree (Ouroboros section
 * 3.4.3, Figure 3): the target scores each node of the candidate tree once,
 * so candidates that share a prefix share its rows and fewer rows are read.
 *   node_logits DEVICE [B][N][V]: row n of sequence b is the target
 *               distribution after the context plus the path to node n
 *   cand_tokens DEVICE [B][C][L] int32
 *   cand_rows   DEVICE [B][C][R] int32: the node row (0 <= row < N) that scores
 *               candidate token (c, i) for i < L, and for R = L+1 the row
 *               after its last token.  A row outside [0, N) is never read: that
 *               position never matches and its correction token is -1.
 *   N >= 1.  Selection, outputs and errors as spec_verify_greedy_candidates;
 *   the result equals spec_verify_greedy_candidates on the flat layout whose
 *   row (c, i) is node row cand_rows[c][i].
 *   workspace   DEVICE, >= spec_verify_workspace_bytes(B, N, V, dtype) */
int spec_verify_greedy_tree(const void* node_logits, long long row_stride, int N,
                            const int* cand_tokens, const int* cand_rows, int B, int C, int L, int R,
                            int V, int dtype, int* out_tokens, int* out_num_accepted,
                            int* out_best_candidate,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/* Early-exit verification: the same results as spec_verify_sample /
 * spec_verify_greedy, bit for bit, while reading only the rows the rule
 * looks at.  The rule examines position i only when every earlier draft was
 * accepted (production blog, "The acceptance rule": left to right, stopping
 * at the first rejection), so positions are taken in windows [0,1), [1,2),
 * [2,4), [4,8), ... (the bonus row k joins the last window rather than
 * forming one of its own) and a window's rows are streamed only for the sequences
 * still undecided after the previous windows (a device-side work list; no
 * host synchronisation).  Rows read per sequence: those up to its first
 * rejection, rounded up to the end of that window, plus the sampled row.
 * Worth it when acceptance is low; with high acceptance it reads as much as
 * the full pass in more launches.  p(x_i) and q(x_i) are not exported (the
 * rows after the first rejection are not read).
 * Arguments, outputs, workspace size and errors as spec_verify_sample /
 * spec_verify_greedy respectively. */
int spec_verify_sample_lazy(const void* target_logits, long long target_row_stride,
                            const void* draft_logits, long long draft_row_stride,
                            const int* draft_tokens, const float* uniforms, float temperature,
                            int B, int k, int V, int dtype, int* out_tokens, int* out_num_accepted,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

int spec_verify_greedy_lazy(const void* target_logits, long long target_row_stride,
                            const int* draft_tokens, int B, int k, int V, int dtype,
                            int* out_tokens, int* out_num_accepted,
                            void* workspace, size_t workspace_bytes, void* hip_stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 * spec_verify_sample without the workspace arguments: the same kernels and
 * the same results, bit for bit, with the scratch taken from a static device
 * buffer of SV_NOALLOC_SCRATCH_BYTES (4 MiB) that the library holds on each
 * device it runs on until the process ends.  The call allocates and frees
 * nothing (no hipMalloc / hipFree, no allocating library routine).
 *  - Limit: shapes whose workspace for spec_verify_sample exceeds
 *    SV_NOALLOC_SCRATCH_BYTES are refused with SV_ESCRATCH before anything
 *    is launched (B = 512, k = 16, V = 128256 needs 0.86 MiB).  That
 *    workspace is at most spec_verify_workspace_bytes(B, 2k+1, V, dtype),
 *    which also counts the room only truncated calls use.
 *  - One buffer per device, shared by every call on it: the buffer keeps
 *    the last call's contents (nothing in it needs clearing), and calls that
 *    overlap on one device race on it, even on different streams.  Issue
 *    them on one stream, or order them.
 *  - The device is the current one; hip_stream (NULL: the null stream) must
 *    belong to it (SV_EINVAL otherwise).  The buffer's address is looked up
 *    on the first call on each device.
 *  Other arguments, outputs and errors as spec_verify_sample. */
int spec_verify_sample_noalloc(const void* target_logits, long long target_row_stride,
                               const void* draft_logits, long long draft_row_stride,
                               const int* draft_tokens, const float* uniforms, float temperature,
                               int B, int k, int V, int dtype,
                               int* out_tokens, int* out_num_accepted,
                               float* out_p_x, float* out_q_x, void* hip_stream);

/* Measurement variants, for callers that time the vocabulary-streaming kernel
 * (the one launch that reads every logit) inside their own timed region.
 * Each does exactly what the entry points named below do, and in addition
 * records the caller's two HIP events on `hip_stream`: `event_begin` right
 * before that kernel and `event_end` right after it.  The events are
 * hipEvent_t handles created and owned by the caller (passed as void*); the
 * library keeps no state, so concurrent calls on different streams with
 * their own events and workspaces do not interact.  Both events are
 * required (SV_EINVAL if either is NULL, nothing launched); a failed event
 * record returns SV_EHIP.  An event pair costs a few microseconds of queue
 * time on the stream.
 *  - spec_verify_sample_timed: spec_verify_sample_truncated's arguments plus
 *    spec_verify_sample_lenient's lenience (>= 1; 1 is the exact rule);
 *    top_k = 0 and top_p >= 1 with lenience 1 is spec_verify_sample.  The
 *    timed kernel is the statistics pass, or the truncation pass when top-k
 *    or top-p is on.
 *  - spec_verify_greedy_timed: spec_verify_greedy_ext's arguments, whose
 *    three by-product outputs may each be NULL (all NULL: spec_verify_greedy).
 *  - spec_verify_candidates_timed: spec_verify_greedy_tree's arguments, where
 *    cand_rows = NULL selects the flat layout of
 *    spec_verify_greedy_candidates (N is then ignored), plus
 *    spec_verify_greedy_candidates_ext's out_target_argmax (NULL = none):
 *    [B][C][R], the argmax of the row that scores each candidate position
 *    (-1 where a tree row is outside [0, N)). */
int spec_verify_sample_timed(const void* target_logits, long long target_row_stride,
                             const void* draft_logits, long long draft_row_stride,
                             const int* draft_tokens, const float* uniforms, float temperature,
                             float lenience, int top_k, float top_p, int B, int k, int V, int dtype,
                             int* out_tokens, int* out_num_accepted, float* out_p_x, float* out_q_x,
                             void* workspace, size_t workspace_bytes, void* hip_stream,
                             void* event_begin, void* event_end);

int spec_verify_greedy_timed(const void* target_logits, long long target_row_stride,
                             const int* draft_tokens, int B, int k, int V, int dtype,
                             int* out_tokens, int* out_num_accepted, int* out_target_argmax,
                             unsigned long long* out_match_mask, int* out_num_match,
                             void* workspace, size_t workspace_bytes, void* hip_stream,
                             void* event_begin, void* event_end);

int spec_verify_candidates_timed(const void* target_logits, long long row_stride,
                                 const int* cand_tokens, const int* cand_rows, int N,
                                 int B, int C, int L, int R, int V, int dtype,
                                 int* out_tokens, int* out_num_accepted, int* out_best_candidate,
                                 int* out_target_argmax,
                                 void* workspace, size_t workspace_bytes, void* hip_stream,
                                 void* event_begin, void* event_end);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
