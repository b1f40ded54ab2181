/*
 * oracle.c -- plain CPU oracle for the speculative-decoding verification step.
 *
 * TEST INFRASTRUCTURE ONLY: called by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library (which shares nothing
 * with this file).  Single-threaded, double precision, no blocking or fusion:
 * each step below is the rule as the pages state it, executed in their order.
 * The rule, its conventions and its sources are described in oracle.h.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- distributions --------------------------------------------------------
 * p = softmax(z / T): the target's distribution at one position (production
 * blog, "The acceptance rule": the target returns its distribution p at every
 * one of the k+1 positions; the draft's q likewise at k positions).
 * Returns 0, or -3 when the row has no finite logit.                        */
static int softmax_row(const float* z, int V, double T, double* p)
{
    double m = -INFINITY;
    for (int t = 0; t < V; ++t) {
        double a = (double)z[t] / T;
        if (a > m) m = a;
    }
    if (!(m > -INFINITY) || !isfinite(m)) return -3;
    double s = 0.0;
    for (int t = 0; t < V; ++t) s += exp((double)z[t] / T - m);
    for (int t = 0; t < V; ++t) p[t] = exp((double)z[t] / T - m) / s;
    return 0;
}

/* ---- truncation (top-k, then top-p) -------------------------------------
 * Tokens are ranked by logit; equal logits share a rank group and are kept
 * or dropped together. */
typedef struct { double z, p; } zp_pair;

static int cmp_desc(const void* a, const void* b)
{
    double x = ((const zp_pair*)a)->z, y = ((const zp_pair*)b)->z;
    return (x < y) - (x > y);
}

static int truncate_row(const float* z, int V, double T, int top_k, double top_p, double* p,
                        double* margin)
{
    *margin = 1.0;
    int rc = softmax_row(z, V, T, p);          /* p: softmax(z / T) */
    if (rc) return rc;
    zp_pair* sorted = (zp_pair*)malloc(sizeof(zp_pair) * (size_t)V);
    if (!sorted) return -2;
    for (int t = 0; t < V; ++t) {
        sorted[t].z = (double)z[t];
        sorted[t].p = p[t];
    }
    qsort(sorted, (size_t)V, sizeof(zp_pair), cmp_desc);
    /* top-k: keep logits >= the top_k-th largest */
    double zk = -INFINITY;
    if (top_k >= 1 && top_k < V) zk = sorted[top_k - 1].z;
    /* top-p over the kept set, groups of equal logits in descending order:
     * a group is kept iff the kept mass strictly above it is below top_p of
     * the kept mass; the first group that fails and every later one drop */
    double zdrop = -INFINITY;                  /* drop logits <= zdrop */
    int dropped = 0;
    if (top_p < 1.0) {
        double M = 0.0;
        for (int i = 0; i < V && sorted[i].z >= zk; ++i) M += sorted[i].p;
        const double budget = top_p * M;
        double greater = 0.0;
        int i = 0;
        while (i < V && sorted[i].z >= zk) {
            const double g = sorted[i].z;
            if (!(greater < budget)) {
                zdrop = g;
                dropped = 1;
                const double m1 = (greater - budget) / M;
                if (m1 < *margin) *margin = m1;
                break;
            }
            const double m0 = (budget - greater) / M;
            if (m0 < *margin) *margin = m0;
            while (i < V && sorted[i].z == g) greater += sorted[i++].p;
        }
    }
    free(sorted);
    double S = 0.0;
    for (int t = 0; t < V; ++t) {
        const double zt = (double)z[t];
        const int kept = zt >= zk && !(dropped && zt <= zdrop);
        if (!kept) p[t] = 0.0;
        S += p[t];
    }
    for (int t = 0; t < V; ++t) p[t] /= S;
    return 0;
}

int oracle_truncated_row(const float* z, int V, double T, int top_k, double top_p, double* out_p,
                         double* margin)
{
    if (!z || !out_p || !margin || V < 1 || top_k < 0 || !(top_p > 0.0)) return -1;
    if (!(T > 0.0) || !isfinite(T)) return -1;
    return truncate_row(z, V, T, top_k, top_p, out_p, margin);
}

/* ---- one draw by inverse CDF ------------------------------------------------
 * Draw from the distribution proportional to w using one uniform u: walk the
 * vocabulary in ascending index order, summing weights, and return the first
 * index whose running sum exceeds u * total.  If rounding leaves no crossing
 * (u * total >= the final sum), return the largest index with positive
 * weight.  Records the boundaries of the chosen token's CDF interval.        */
static int inverse_cdf(const double* w, int V, double u, double* total_out,
                       double* lo_out, double* hi_out)
{
    double total = 0.0;
    for (int t = 0; t < V; ++t) total += w[t];
    double thr = u * total;
    double c = 0.0;
    for (int t = 0; t < V; ++t) {
        double before = c;
        c += w[t];
        if (c > thr) {
            *total_out = total;
            *lo_out = before / total;
            *hi_out = c / total;
            return t;
        }
    }
    int last = 0;
    double before = 0.0, c2 = 0.0;
    for (int t = 0; t < V; ++t) {
        if (w[t] > 0.0) { last = t; before = c2; }
        c2 += w[t];
    }
    *total_out = total;
    *lo_out = before / total;
    *hi_out = 1.0;
    return last;
}

/* ---- argmax -------------------------------------------------------------
 * Index of the largest logit; the lowest index among equal maxima.  Scans
 * ascending and replaces only on a strictly greater value, so NaN (which
 * compares false) never wins and a row with nothing above -inf gives 0.    */
static int argmax_row(const float* z, int V)
{
    double best = -INFINITY;
    int idx = 0;
    for (int t = 0; t < V; ++t) {
        double v = (double)z[t];
        if (v > best) { best = v; idx = t; }
    }
    return idx;
}

int oracle_trace_size(void) { return (int)sizeof(oracle_trace); }

/* ---- greedy ---------------------------------------------------------------
 * Production blog, "The acceptance rule", last sentences: under greedy
 * decoding a draft token is accepted if it equals the target's argmax at
 * that position and the first mismatch is replaced by the target's argmax.
 * If all k drafts survive, the greedy choice at position k+1 is appended.  */
int oracle_greedy_seq(const float* target, long long row_stride, const int* draft_tokens,
                      int k, int V, int* out_tokens, int* out_num_accepted)
{
    if (!target || !draft_tokens || !out_tokens || !out_num_accepted) return -1;
    if (k < 1 || k > ORACLE_MAX_K || V < 1 || row_stride < V) return -1;
    for (int i = 0; i <= k; ++i) out_tokens[i] = -1;
    for (int i = 0; i < k; ++i) {
        int a = argmax_row(target + (long long)i * row_stride, V);
        int x = draft_tokens[i];
        if (x == a) {                     /* an out-of-range x never equals a */
            out_tokens[i] = x;
            continue;
        }
        out_tokens[i] = a;
        *out_num_accepted = i;
        return 0;
    }
    out_tokens[k] = argmax_row(target + (long long)k * row_stride, V);
    *out_num_accepted = k;
    return 0;
}

/* ---- sampling -------------------------------------------------------------
 * Production blog, "The acceptance rule": examine drafts left to right; keep
 * x_i with probability min(1, p(x_i)/q(x_i)); at the first rejection sample a
 * replacement from the residual proportional to max(0, p - q) and stop; if
 * all k are kept, sample one bonus token from p at position k+1.           */
/* p (or q) of one row: softmax(z / T), truncated when top-k or top-p is on;
 * *margin keeps the smallest top-p boundary distance seen. */
static int row_dist(const float* z, int V, double T, int top_k, double top_p, double* p,
                    double* margin)
{
    if ((top_k <= 0 || top_k >= V) && top_p >= 1.0) return softmax_row(z, V, T, p);
    double m = 1.0;
    int rc = truncate_row(z, V, T, top_k, top_p, p, &m);
    if (m < *margin) *margin = m;
    return rc;
}

static int sample_seq(const float* target, long long ts, const float* draft, long long ds,
                      const int* x, const float* u, double T, double l, int top_k, double top_p,
                      int k, int V, int* out_tokens, int* out_num_accepted, oracle_trace* tr,
                      int mut, double* trunc_margin)
{
    double margin_local = 1.0;
    if (!trunc_margin) trunc_margin = &margin_local;
    *trunc_margin = 1.0;
    if (!target || !draft || !x || !u || !out_tokens || !out_num_accepted) return -1;
    if (k < 1 || k > ORACLE_MAX_K || V < 1 || ts < V || ds < V) return -1;
    if (!(T > 0.0) || !isfinite(T)) return -1;
    if (!(l >= 1.0) || !isfinite(l)) return -1;

    oracle_trace local;
    if (!tr) tr = &local;
    memset(tr, 0, sizeof(*tr));
    for (int i = 0; i <= k; ++i) out_tokens[i] = -1;

    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* q = (double*)malloc(sizeof(double) * (size_t)V);
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    if (!p || !q || !w) { free(p); free(q); free(w); return -2; }

    int rc = 0;
    const double u_sample = (double)u[k];
    for (int i = 0; i < k; ++i) {
        if ((rc = row_dist(target + (long long)i * ts, V, T, top_k, top_p, p, trunc_margin)) != 0) goto done;
        if ((rc = row_dist(draft + (long long)i * ds, V, T, top_k, top_p, q, trunc_margin)) != 0) goto done;

        const int tok = x[i];
        const int valid = tok >= 0 && tok < V;
        const double px = valid ? p[tok] : 0.0;
        const double qx = valid ? q[tok] : 0.0;
        double ratio;
        int accept;
        if (!valid) {
            ratio = 0.0;
            accept = 0;
        } else if (mut == ORACLE_MUT_RATIO_INVERTED) {
            ratio = (px <= qx) ? 1.0 : qx / px;
            accept = (double)u[i] < ratio;
        } else if (qx <= l * px) {
            ratio = 1.0;                  /* min(1, l p/q) = 1, q = 0 included */
            accept = 1;
        } else {
            ratio = l * px / qx;
            accept = (double)u[i] < ratio;
        }
        tr->ratio[i] = ratio;
        tr->accept_margin[i] = fabs((double)u[i] - ratio);
        tr->p_x[i] = px;
        tr->q_x[i] = qx;
        tr->evaluated = i + 1;

        if (accept) {
            out_tokens[i] = tok;
            continue;
        }

        /* first rejection: residual max(0, p - q), normalised by its total */
        for (int t = 0; t < V; ++t) {
            double d;
            switch (mut) {
            case ORACLE_MUT_RESIDUAL_IS_P: d = p[t]; break;
            case ORACLE_MUT_RESIDUAL_IS_Q: d = q[t]; break;
            case ORACLE_MUT_RESIDUAL_SIGN: d = q[t] - p[t]; break;
            default: d = p[t] - q[t]; break;
            }
            w[t] = d > 0.0 ? d : 0.0;
        }
        double total = 0.0;
        for (int t = 0; t < V; ++t) total += w[t];
        tr->sample_kind = 0;
        if (!(total > 0.0)) {            /* no residual mass: p itself */
            memcpy(w, p, sizeof(double) * (size_t)V);
            tr->sample_kind = 2;
        }
        int t_star = inverse_cdf(w, V, u_sample, &tr->sample_total, &tr->sample_lo, &tr->sample_hi);
        out_tokens[i] = t_star;
        tr->sampled_token = t_star;
        tr->num_accepted = i;
        *out_num_accepted = i;
        goto margins;
    }

    /* every draft kept: one bonus token from p at position k+1 */
    if (mut == ORACLE_MUT_BONUS_FROM_Q) {
        if ((rc = row_dist(draft + (long long)(k - 1) * ds, V, T, top_k, top_p, p, trunc_margin)) != 0) goto done;
    } else {
        if ((rc = row_dist(target + (long long)k * ts, V, T, top_k, top_p, p, trunc_margin)) != 0) goto done;
    }
    {
        int t_star = inverse_cdf(p, V, u_sample, &tr->sample_total, &tr->sample_lo, &tr->sample_hi);
        out_tokens[k] = t_star;
        tr->sampled_token = t_star;
        tr->sample_kind = 1;
        tr->num_accepted = k;
        *out_num_accepted = k;
    }

margins:
    tr->num_accepted = *out_num_accepted;
    {
        double a = u_sample - tr->sample_lo, b = tr->sample_hi - u_sample;
        tr->sample_margin = a < b ? a : b;
    }
done:
    free(p);
    free(q);
    free(w);
    return rc;
}

int oracle_sample_seq(const float* target, long long target_row_stride,
                      const float* draft, long long draft_row_stride,
                      const int* draft_tokens, const float* uniforms, double temperature,
                      int k, int V, int* out_tokens, int* out_num_accepted,
                      oracle_trace* trace)
{
    return sample_seq(target, target_row_stride, draft, draft_row_stride, draft_tokens,
                      uniforms, temperature, 1.0, 0, 1.0, k, V, out_tokens, out_num_accepted, trace,
                      ORACLE_MUT_NONE, NULL);
}

int oracle_sample_seq_mutant(const float* target, long long target_row_stride,
                             const float* draft, long long draft_row_stride,
                             const int* draft_tokens, const float* uniforms, double temperature,
                             int k, int V, int* out_tokens, int* out_num_accepted,
                             oracle_trace* trace, int mutation)
{
    return sample_seq(target, target_row_stride, draft, draft_row_stride, draft_tokens,
                      uniforms, temperature, 1.0, 0, 1.0, k, V, out_tokens, out_num_accepted, trace,
                      mutation, NULL);
}

/* p_i(x_i), q_i(x_i) at every draft position: the quantities whose ratio the
 * acceptance rule compares (production blog, "The acceptance rule").       */
int oracle_token_probs_seq(const float* target, long long ts, const float* draft, long long ds,
                           const int* x, double T, int k, int V,
                           double* out_p_x, double* out_q_x)
{
    if (!target || !draft || !x || !out_p_x || !out_q_x) return -1;
    if (k < 1 || k > ORACLE_MAX_K || V < 1 || ts < V || ds < V) return -1;
    if (!(T > 0.0) || !isfinite(T)) return -1;
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* q = (double*)malloc(sizeof(double) * (size_t)V);
    if (!p || !q) { free(p); free(q); return -2; }
    int rc = 0;
    for (int i = 0; i < k; ++i) {
        if ((rc = softmax_row(target + (long long)i * ts, V, T, p)) != 0) break;
        if ((rc = softmax_row(draft + (long long)i * ds, V, T, q)) != 0) break;
        int valid = x[i] >= 0 && x[i] < V;
        out_p_x[i] = valid ? p[x[i]] : 0.0;
        out_q_x[i] = valid ? q[x[i]] : 0.0;
    }
    free(p);
    free(q);
    return rc;
}

/* The CDF interval of one token in the distribution a round draws from
 * (residual or p), by the same ascending-index convention as inverse_cdf. */
int oracle_draw_interval(const float* target_row, const float* draft_row, double T, int V,
                         int token, double* lo, double* hi, double* weight)
{
    if (!target_row || !lo || !hi || !weight || V < 1 || token < 0 || token >= V) return -1;
    if (!(T > 0.0) || !isfinite(T)) return -1;
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    if (!p || !w) { free(p); free(w); return -2; }
    int rc = softmax_row(target_row, V, T, p);
    if (rc == 0) {
        double total = 0.0;
        if (draft_row) {
            rc = softmax_row(draft_row, V, T, w);
            if (rc == 0) {
                for (int t = 0; t < V; ++t) {
                    double d = p[t] - w[t];
                    w[t] = d > 0.0 ? d : 0.0;
                    total += w[t];
                }
            }
        }
        if (rc == 0) {
            if (!draft_row || !(total > 0.0)) {
                memcpy(w, p, sizeof(double) * (size_t)V);
                total = 0.0;
                for (int t = 0; t < V; ++t) total += w[t];
            }
            double c = 0.0;
            for (int t = 0; t < token; ++t) c += w[t];
            *lo = c / total;
            *hi = (c + w[token]) / total;
            *weight = w[token] / total;
        }
    }
    free(p);
    free(w);
    return rc;
}

/* ---- multi-candidate greedy --------------------------------------------
 * Ouroboros, section 3.4.3, "Selecting the accepted tokens": the candidates
 * share their first tokens (the base draft) and are verified together.  For
 * each candidate c the accepted length a_c is the number of leading tokens
 * equal to the target's argmax at their position (the case equation for the
 * accepted suffix length); the candidate with the largest a_c is selected and
 * its accepted tokens are committed, followed by the target's correction at
 * the first mismatch.  When the shared prefix already fails, every candidate
 * has the same a_c and this is Stage 1's plain fallback.  Ties go to the
 * lowest candidate index.  With R = L rows per candidate there is no row
 * after the last token, so a fully accepted candidate commits L tokens; with
 * R = L+1 its last row supplies one more greedy token.                      */
int oracle_greedy_candidates_seq(const float* target, long long row_stride,
                                 const int* cand, int C, int L, int R, int V,
                                 int* out_tokens, int* out_num_accepted, int* out_best)
{
    if (!target || !cand || !out_tokens || !out_num_accepted || !out_best) return -1;
    if (C < 1 || L < 1 || C * L > 64 || (R != L && R != L + 1) || V < 1 || row_stride < V)
        return -1;
    int best_c = 0, best_a = -1;
    for (int c = 0; c < C; ++c) {
        int a = L;
        for (int i = 0; i < L; ++i) {
            const float* row = target + ((long long)c * R + i) * row_stride;
            if (cand[c * L + i] != argmax_row(row, V)) { a = i; break; }
        }
        if (a > best_a) { best_a = a; best_c = c; }
    }
    for (int i = 0; i <= L; ++i) out_tokens[i] = -1;
    for (int i = 0; i < best_a; ++i) out_tokens[i] = cand[best_c * L + i];
    if (best_a < L) {
        out_tokens[best_a] = argmax_row(target + ((long long)best_c * R + best_a) * row_stride, V);
    } else if (R == L + 1) {
        out_tokens[L] = argmax_row(target + ((long long)best_c * R + L) * row_stride, V);
    }
    *out_num_accepted = best_a;
    *out_best = best_c;
    return 0;
}

/* ---- batched forms: one sequence after another -------------------------- */
int oracle_greedy(const float* target, long long row_stride, const int* x,
                  int B, int k, int V, int* out_tokens, int* out_num_accepted)
{
    if (B < 0) return -1;
    for (int b = 0; b < B; ++b) {
        int rc = oracle_greedy_seq(target + (long long)b * (k + 1) * row_stride, row_stride,
                                   x + (long long)b * k, k, V, out_tokens + (long long)b * (k + 1),
                                   out_num_accepted + b);
        if (rc) return rc;
    }
    return 0;
}

int oracle_sample(const float* target, long long ts, const float* draft, long long ds,
                  const int* x, const float* u, double T, int B, int k, int V,
                  int* out_tokens, int* out_num_accepted, oracle_trace* traces, int mutation)
{
    if (B < 0) return -1;
    for (int b = 0; b < B; ++b) {
        int rc = sample_seq(target + (long long)b * (k + 1) * ts, ts,
                            draft + (long long)b * k * ds, ds,
                            x + (long long)b * k, u + (long long)b * (k + 1), T, 1.0, 0, 1.0, k, V,
                            out_tokens + (long long)b * (k + 1), out_num_accepted + b,
                            traces ? traces + b : NULL, mutation, NULL);
        if (rc) return rc;
    }
    return 0;
}

/* Lenience l (Cascade Speculative Drafting, "The Vertical Cascade", review
 * function): the acceptance test becomes q <= l p, else reject with
 * probability 1 - l p/q; the residual is unchanged. */
int oracle_sample_lenient(const float* target, long long ts, const float* draft, long long ds,
                          const int* x, const float* u, double T, double l, int B, int k, int V,
                          int* out_tokens, int* out_num_accepted, oracle_trace* traces)
{
    if (B < 0) return -1;
    for (int b = 0; b < B; ++b) {
        int rc = sample_seq(target + (long long)b * (k + 1) * ts, ts,
                            draft + (long long)b * k * ds, ds,
                            x + (long long)b * k, u + (long long)b * (k + 1), T, l, 0, 1.0, k, V,
                            out_tokens + (long long)b * (k + 1), out_num_accepted + b,
                            traces ? traces + b : NULL, ORACLE_MUT_NONE, NULL);
        if (rc) return rc;
    }
    return 0;
}

/* Truncated sampling (top-k then top-p on target and draft alike). */
int oracle_sample_truncated(const float* target, long long ts, const float* draft, long long ds,
                            const int* x, const float* u, double T, int top_k, double top_p,
                            int B, int k, int V, int* out_tokens, int* out_num_accepted,
                            oracle_trace* traces, double* trunc_margin)
{
    if (B < 0 || top_k < 0 || !(top_p > 0.0)) return -1;
    for (int b = 0; b < B; ++b) {
        int rc = sample_seq(target + (long long)b * (k + 1) * ts, ts,
                            draft + (long long)b * k * ds, ds,
                            x + (long long)b * k, u + (long long)b * (k + 1), T, 1.0, top_k, top_p,
                            k, V, out_tokens + (long long)b * (k + 1), out_num_accepted + b,
                            traces ? traces + b : NULL, ORACLE_MUT_NONE,
                            trunc_margin ? trunc_margin + b : NULL);
        if (rc) return rc;
    }
    return 0;
}

/* Ouroboros section 3.4.4, Eq. 10: #Match counts the positions where the
 * draft token equals the target's verification token v_i (its argmax under
 * greedy decoding), whether or not they lie in the accepted prefix. */
int oracle_greedy_matches(const float* target, long long row_stride, const int* x,
                          int B, int k, int V, int* out_v, unsigned long long* out_mask,
                          int* out_num_match)
{
    if (!target || !x || !out_v || !out_mask || !out_num_match) return -1;
    if (B < 0 || k < 1 || k > ORACLE_MAX_K || V < 1 || row_stride < V) return -1;
    for (int b = 0; b < B; ++b) {
        const float* seq = target + (long long)b * (k + 1) * row_stride;
        unsigned long long mask = 0;
        int count = 0;
        for (int i = 0; i <= k; ++i) {
            int v = argmax_row(seq + (long long)i * row_stride, V);
            out_v[(long long)b * (k + 1) + i] = v;
            if (i < k && x[(long long)b * k + i] == v) {
                mask |= 1ull << i;
                count++;
            }
        }
        out_mask[b] = mask;
        out_num_match[b] = count;
    }
    return 0;
}

/* Ouroboros 3.4.3 on a token tree: the same selection as the flat form, each
 * candidate position reading the node row that scores it. */
int oracle_greedy_tree(const float* nodes, long long row_stride, int N, const int* cand,
                       const int* cand_rows, int B, int C, int L, int R, int V,
                       int* out_tokens, int* out_num_accepted, int* out_best)
{
    if (!nodes || !cand || !cand_rows || !out_tokens || !out_num_accepted || !out_best) return -1;
    if (B < 0 || N < 1 || C < 1 || L < 1 || C * L > 64 || (R != L && R != L + 1) || V < 1 ||
        row_stride < V)
        return -1;
    for (int b = 0; b < B; ++b) {
        const float* seq = nodes + (long long)b * N * row_stride;
        const int* rows = cand_rows + (long long)b * C * R;
        const int* cb = cand + (long long)b * C * L;
        int* out = out_tokens + (long long)b * (L + 1);
        int best_c = 0, best_a = -1;
        for (int c = 0; c < C; ++c) {
            int a = L;
            for (int i = 0; i < L; ++i) {
                int r = rows[c * R + i];
                /* a row outside [0, N) scores nothing: a mismatch whatever the token */
                if (r < 0 || r >= N) { a = i; break; }
                if (cb[c * L + i] != argmax_row(seq + (long long)r * row_stride, V)) { a = i; break; }
            }
            if (a > best_a) { best_a = a; best_c = c; }
        }
        for (int i = 0; i <= L; ++i) out[i] = -1;
        for (int i = 0; i < best_a; ++i) out[i] = cb[best_c * L + i];
        int next = -1;
        if (best_a < L || R == L + 1) {
            int r = rows[best_c * R + best_a];
            next = (r >= 0 && r < N) ? argmax_row(seq + (long long)r * row_stride, V) : -1;
            out[best_a] = next;
        }
        out_num_accepted[b] = best_a;
        out_best[b] = best_c;
    }
    return 0;
}

int oracle_row_argmax(const float* rows, long long row_stride, long long n_rows, int V, int* out)
{
    if (!rows || !out || n_rows < 0 || V < 1 || row_stride < V) return -1;
    for (long long r = 0; r < n_rows; ++r) out[r] = argmax_row(rows + r * row_stride, V);
    return 0;
}

int oracle_greedy_candidates(const float* target, long long row_stride, const int* cand,
                             int B, int C, int L, int R, int V,
                             int* out_tokens, int* out_num_accepted, int* out_best)
{
    if (B < 0) return -1;
    for (int b = 0; b < B; ++b) {
        int rc = oracle_greedy_candidates_seq(target + (long long)b * C * R * row_stride, row_stride,
                                              cand + (long long)b * C * L, C, L, R, V,
                                              out_tokens + (long long)b * (L + 1),
                                              out_num_accepted + b, out_best + b);
        if (rc) return rc;
    }
    return 0;
}
