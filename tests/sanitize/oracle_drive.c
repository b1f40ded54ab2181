/* oracle_drive.c -- exercises every entry point of the CPU oracle on seeded
 * random inputs and edge cases (V from 1 up, k = 1 and 63, invalid draft
 * tokens, -inf logits, all -inf rows, both candidate layouts, out-of-range
 * tree rows, truncation settings), for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Exit status 0 when every call returns its
 * documented status and every output lies in range. */
#include <limits.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static unsigned long long state = 88172645463325252ull;
static double unit(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) * (1.0 / 9007199254740992.0);
}

static int failures = 0;
#define CHECK(c, ...)                        \
    do {                                     \
        if (!(c)) {                          \
            fprintf(stderr, __VA_ARGS__);    \
            fprintf(stderr, "\n");           \
            ++failures;                      \
        }                                    \
    } while (0)

static float* logits(long long n, int V, double ninf_frac)
{
    float* z = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1) * (size_t)V);
    for (long long r = 0; r < n; ++r)
        for (int t = 0; t < V; ++t) {
            float v = (float)(6.0 * unit() - 3.0);
            if (unit() < ninf_frac && t != r % V) v = -INFINITY;   /* one finite logit per row */
            z[r * V + t] = v;
        }
    return z;
}

static void tokens_for(int* x, int n, int V)
{
    for (int i = 0; i < n; ++i) {
        const double r = unit();
        x[i] = r < 0.05 ? -1 : r < 0.1 ? V : r < 0.12 ? INT_MIN : (int)(unit() * V);
    }
}

static void out_range(const int* out, int n_acc, int len, int V, const char* what)
{
    CHECK(n_acc >= 0 && n_acc < len, "%s: accepted count %d", what, n_acc);
    for (int i = 0; i <= n_acc && i < len; ++i)
        CHECK(out[i] >= -1 && out[i] < V, "%s: token %d = %d", what, i, out[i]);
    for (int i = n_acc + 1; i < len; ++i) CHECK(out[i] == -1, "%s: padding at %d", what, i);
}

static void chain_case(int B, int k, int V, double ninf)
{
    const int rt = B * (k + 1), rd = B * k;
    float* z = logits(rt, V, ninf);
    float* y = logits(rd, V, ninf);
    int* x = (int*)malloc(sizeof(int) * B * k);
    float* u = (float*)malloc(sizeof(float) * B * (k + 1));
    int* out = (int*)malloc(sizeof(int) * B * (k + 1));
    int* na = (int*)malloc(sizeof(int) * B);
    tokens_for(x, B * k, V);
    for (int i = 0; i < B * (k + 1); ++i) u[i] = (float)(unit() * 0.999999);
    char* traces = (char*)malloc((size_t)oracle_trace_size() * B);

    CHECK(oracle_greedy(z, V, x, B, k, V, out, na) == 0, "greedy B=%d k=%d V=%d", B, k, V);
    for (int b = 0; b < B; ++b) out_range(out + b * (k + 1), na[b], k + 1, V, "greedy");
    for (int mut = 0; mut <= 5; ++mut) {
        CHECK(oracle_sample(z, V, y, V, x, u, 0.8, B, k, V, out, na, (oracle_trace*)traces, mut) == 0,
              "sample mut=%d B=%d k=%d V=%d", mut, B, k, V);
        for (int b = 0; b < B; ++b) out_range(out + b * (k + 1), na[b], k + 1, V, "sample");
    }
    CHECK(oracle_sample_lenient(z, V, y, V, x, u, 1.3, 2.5, B, k, V, out, na, NULL) == 0, "lenient");
    for (int b = 0; b < B; ++b) out_range(out + b * (k + 1), na[b], k + 1, V, "lenient");
    double* margin = (double*)malloc(sizeof(double) * B);
    const int tk[3] = {0, 1, V > 3 ? V / 3 : 1};
    const double tp[3] = {1.0, 0.8, 1e-6};
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            CHECK(oracle_sample_truncated(z, V, y, V, x, u, 0.9, tk[i], tp[j], B, k, V, out, na,
                                          (oracle_trace*)traces, margin) == 0,
                  "truncated top_k=%d top_p=%g", tk[i], tp[j]);
            for (int b = 0; b < B; ++b) out_range(out + b * (k + 1), na[b], k + 1, V, "truncated");
        }
    double* p = (double*)malloc(sizeof(double) * V);
    double m = 0;
    CHECK(oracle_truncated_row(z, V, 1.0, tk[2], 0.5, p, &m) == 0, "truncated_row");
    int* v = (int*)malloc(sizeof(int) * B * (k + 1));
    unsigned long long* mask = (unsigned long long*)malloc(sizeof(unsigned long long) * B);
    int* cnt = (int*)malloc(sizeof(int) * B);
    CHECK(oracle_greedy_matches(z, V, x, B, k, V, v, mask, cnt) == 0, "greedy_matches");
    CHECK(oracle_row_argmax(z, V, rt, V, v) == 0, "row_argmax");
    for (int i = 0; i < rt; ++i) CHECK(v[i] >= 0 && v[i] < V, "row argmax %d", v[i]);
    double* px = (double*)malloc(sizeof(double) * k);
    double* qx = (double*)malloc(sizeof(double) * k);
    CHECK(oracle_token_probs_seq(z, V, y, V, x, 1.0, k, V, px, qx) == 0, "token_probs");
    double lo, hi, w;
    CHECK(oracle_draw_interval(z, y, 1.0, V, V / 2, &lo, &hi, &w) == 0, "draw_interval residual");
    CHECK(oracle_draw_interval(z, NULL, 1.0, V, 0, &lo, &hi, &w) == 0, "draw_interval p");
    CHECK(lo >= 0.0 && hi <= 1.0 + 1e-12 && lo <= hi, "draw interval [%g, %g]", lo, hi);
    free(z); free(y); free(x); free(u); free(out); free(na); free(traces); free(margin);
    free(p); free(v); free(mask); free(cnt); free(px); free(qx);
}

static void candidate_case(int B, int C, int L, int R, int V)
{
    const long long rows = (long long)B * C * R;
    float* z = logits(rows, V, 0.0);
    int* cand = (int*)malloc(sizeof(int) * B * C * L);
    tokens_for(cand, B * C * L, V);
    int* out = (int*)malloc(sizeof(int) * B * (L + 1));
    int* na = (int*)malloc(sizeof(int) * B);
    int* best = (int*)malloc(sizeof(int) * B);
    CHECK(oracle_greedy_candidates(z, V, cand, B, C, L, R, V, out, na, best) == 0,
          "candidates C=%d L=%d R=%d", C, L, R);
    for (int b = 0; b < B; ++b) {
        CHECK(best[b] >= 0 && best[b] < C, "best candidate %d", best[b]);
        out_range(out + b * (L + 1), na[b], L + 1, V, "candidates");
    }
    /* the same rows as a tree over N = C*R nodes, with some row indices out
     * of range (never matched) */
    int* map = (int*)malloc(sizeof(int) * B * C * R);
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < C * R; ++i) map[b * C * R + i] = unit() < 0.1 ? (unit() < 0.5 ? -1 : C * R) : i;
    CHECK(oracle_greedy_tree(z, V, C * R, cand, map, B, C, L, R, V, out, na, best) == 0, "tree");
    for (int b = 0; b < B; ++b) out_range(out + b * (L + 1), na[b], L + 1, V, "tree");
    free(z); free(cand); free(out); free(na); free(best); free(map);
}

int main(void)
{
    const int Vs[6] = {1, 2, 7, 8, 33, 1000};
    for (int i = 0; i < 6; ++i) {
        chain_case(3, 1, Vs[i], 0.0);
        chain_case(2, 5, Vs[i], 0.3);
    }
    chain_case(1, 63, 40, 0.1);
    candidate_case(2, 3, 4, 4, 50);
    candidate_case(2, 3, 4, 5, 50);
    candidate_case(1, 8, 8, 8, 7);
    /* argument errors return -1 without touching the buffers */
    int out[4] = {7, 7, 7, 7}, na = 7;
    float z[4] = {0, 0, 0, 0};
    int x[1] = {0};
    CHECK(oracle_greedy(z, 4, x, 1, 0, 4, out, &na) == -1 && na == 7, "k = 0 rejected");
    CHECK(oracle_greedy(z, 4, x, 1, 1, 0, out, &na) == -1 && na == 7, "V = 0 rejected");
    if (failures) {
        fprintf(stderr, "oracle_drive: %d failures\n", failures);
        return 1;
    }
    printf("oracle_drive: all calls passed\n");
    return 0;
}
