/* sv_client.c -- a plain C99 program using libspecverify.so through
 * include/spec_verify.h alone: no Python, no torch.  Device memory comes from
 * the HIP runtime directly.
 *
 * Without a GPU it checks the host-side part of the boundary (status strings,
 * workspace sizing, argument validation, which never touches a device).
 * With a GPU (argument "gpu") it also runs one greedy and one sampling call
 * on small inputs whose results it works out itself:
 *   - greedy: the drafts equal the target row's first maximum for the first
 *     positions, then differ: the accepted count is that prefix and the
 *     correction is the first maximum (the rule, Blog "The acceptance rule");
 *   - sampling with draft rows equal to the target rows: every ratio is 1, so
 *     every draft is accepted (u < 1), and the bonus is a token of p_k;
 *   - the greedy by-products (every row's first maximum, the match mask and
 *     #Match) against its own scan, and the early-exit entry points against
 *     the full-pass calls, bit for bit.
 * Exit status 0 when every check holds. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "spec_verify.h"

static int failures = 0;

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fputc('\n', stderr);                          \
            ++failures;                                   \
        }                                                 \
    } while (0)

static unsigned lcg_state = 12345u;
static float lcg_unit(void)          /* [0, 1), 24 bits */
{
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return (float)(lcg_state >> 8) * (1.0f / 16777216.0f);
}

static int first_max(const float* row, int V)
{
    int best = 0;
    for (int t = 1; t < V; ++t)
        if (row[t] > row[best]) best = t;
    return best;
}

static void host_checks(void)
{
    CHECK(strncmp(spec_verify_status_string(SV_OK), "SV_OK", 5) == 0, "status string");
    CHECK(spec_verify_version() >= 200, "version");
    CHECK(spec_verify_workspace_bytes(4, 5, 1000, SV_F32) > 0, "workspace size");
    CHECK(spec_verify_workspace_bytes(0, 5, 1000, SV_F32) == 0, "workspace size for B = 0");
    int out[8], na[2];
    float dummy[16];
    int tok[4];
    /* invalid arguments are rejected on the host, before any device work */
    CHECK(spec_verify_greedy(dummy, 4, tok, 1, 0, 4, SV_F32, out, na, dummy, 1 << 20, NULL) == SV_EINVAL,
          "k = 0 rejected");
    CHECK(spec_verify_greedy(dummy, 4, tok, 1, 2, 4, 7, out, na, dummy, 1 << 20, NULL) == SV_EDTYPE,
          "dtype rejected");
    CHECK(spec_verify_sample(dummy, 4, dummy, 4, tok, dummy, 0.0f, 1, 2, 4, SV_F32, out, na, NULL, NULL,
                             dummy, 1 << 20, NULL) == SV_EINVAL,
          "temperature 0 rejected");
    CHECK(spec_verify_greedy(dummy, 4, tok, 1, 2, 4, SV_F32, out, na, dummy, 8, NULL) == SV_EWORKSPACE,
          "small workspace rejected");
}

static void gpu_checks(void)
{
    enum { B = 3, K = 4, V = 1000 };
    const int rows = B * (K + 1);
    float* z = (float*)malloc(sizeof(float) * rows * V);
    int x[B * K];
    float u[B * (K + 1)];
    for (int i = 0; i < rows * V; ++i) z[i] = 4.0f * lcg_unit() - 2.0f;
    for (int i = 0; i < B * (K + 1); ++i) u[i] = lcg_unit();
    /* sequence b: drafts equal the first maximum at positions < b + 1, then differ */
    int want_na[B];
    for (int b = 0; b < B; ++b) {
        want_na[b] = b + 1;
        for (int i = 0; i < K; ++i) {
            const int amax = first_max(z + (size_t)(b * (K + 1) + i) * V, V);
            x[b * K + i] = i < b + 1 ? amax : (amax + 1) % V;
        }
    }

    float *dz = NULL, *du = NULL;
    int *dx = NULL, *dout = NULL, *dna = NULL;
    void* ws = NULL;
    const size_t wsb = spec_verify_workspace_bytes(B, 2 * K + 1, V, SV_F32);
    CHECK(hipMalloc((void**)&dz, sizeof(float) * rows * V) == hipSuccess, "hipMalloc");
    CHECK(hipMalloc((void**)&du, sizeof(u)) == hipSuccess, "hipMalloc");
    CHECK(hipMalloc((void**)&dx, sizeof(x)) == hipSuccess, "hipMalloc");
    CHECK(hipMalloc((void**)&dout, sizeof(int) * B * (K + 1)) == hipSuccess, "hipMalloc");
    CHECK(hipMalloc((void**)&dna, sizeof(int) * B) == hipSuccess, "hipMalloc");
    CHECK(hipMalloc(&ws, wsb) == hipSuccess, "hipMalloc");
    if (failures) return;
    hipMemcpy(dz, z, sizeof(float) * rows * V, hipMemcpyHostToDevice);
    hipMemcpy(du, u, sizeof(u), hipMemcpyHostToDevice);
    hipMemcpy(dx, x, sizeof(x), hipMemcpyHostToDevice);

    int out[B * (K + 1)], na[B];
    CHECK(spec_verify_greedy(dz, V, dx, B, K, V, SV_F32, dout, dna, ws, wsb, NULL) == SV_OK, "greedy call");
    hipDeviceSynchronize();
    hipMemcpy(out, dout, sizeof(out), hipMemcpyDeviceToHost);
    hipMemcpy(na, dna, sizeof(na), hipMemcpyDeviceToHost);
    for (int b = 0; b < B; ++b) {
        const int j = want_na[b];
        CHECK(na[b] == j, "greedy accepted count of sequence %d: %d, want %d", b, na[b], j);
        for (int i = 0; i < j; ++i) CHECK(out[b * (K + 1) + i] == x[b * K + i], "greedy token %d.%d", b, i);
        const int amax = first_max(z + (size_t)(b * (K + 1) + j) * V, V);
        CHECK(out[b * (K + 1) + j] == amax, "greedy correction of sequence %d", b);
        for (int i = j + 1; i <= K; ++i) CHECK(out[b * (K + 1) + i] == -1, "greedy padding %d.%d", b, i);
    }

    /* greedy by-products and early-exit greedy on the same inputs */
    {
        int *dv = NULL, *dcnt = NULL, *dout2 = NULL, *dna2 = NULL;
        unsigned long long* dmask = NULL;
        CHECK(hipMalloc((void**)&dv, sizeof(int) * rows) == hipSuccess, "hipMalloc");
        CHECK(hipMalloc((void**)&dcnt, sizeof(int) * B) == hipSuccess, "hipMalloc");
        CHECK(hipMalloc((void**)&dmask, sizeof(unsigned long long) * B) == hipSuccess, "hipMalloc");
        CHECK(hipMalloc((void**)&dout2, sizeof(int) * B * (K + 1)) == hipSuccess, "hipMalloc");
        CHECK(hipMalloc((void**)&dna2, sizeof(int) * B) == hipSuccess, "hipMalloc");
        if (failures) return;
        CHECK(spec_verify_greedy_ext(dz, V, dx, B, K, V, SV_F32, dout2, dna2, dv, dmask, dcnt, ws, wsb, NULL) ==
                  SV_OK,
              "greedy_ext call");
        hipDeviceSynchronize();
        int v[rows], cnt[B], out2[B * (K + 1)], na2[B];
        unsigned long long mask[B];
        hipMemcpy(v, dv, sizeof(v), hipMemcpyDeviceToHost);
        hipMemcpy(cnt, dcnt, sizeof(cnt), hipMemcpyDeviceToHost);
        hipMemcpy(mask, dmask, sizeof(mask), hipMemcpyDeviceToHost);
        hipMemcpy(out2, dout2, sizeof(out2), hipMemcpyDeviceToHost);
        hipMemcpy(na2, dna2, sizeof(na2), hipMemcpyDeviceToHost);
        for (int b = 0; b < B; ++b) {
            unsigned long long want = 0;
            for (int i = 0; i <= K; ++i) {
                const int amax = first_max(z + (size_t)(b * (K + 1) + i) * V, V);
                CHECK(v[b * (K + 1) + i] == amax, "argmax of row %d.%d", b, i);
                if (i < K && x[b * K + i] == amax) want |= 1ull << i;
            }
            CHECK(mask[b] == want, "match mask of sequence %d", b);
            CHECK(cnt[b] == __builtin_popcountll(want), "#Match of sequence %d", b);
            CHECK(na2[b] == na[b], "greedy_ext accepted count of sequence %d", b);
            for (int i = 0; i <= K; ++i) CHECK(out2[b * (K + 1) + i] == out[b * (K + 1) + i], "greedy_ext token");
        }
        CHECK(spec_verify_greedy_lazy(dz, V, dx, B, K, V, SV_F32, dout2, dna2, ws, wsb, NULL) == SV_OK,
              "greedy_lazy call");
        hipDeviceSynchronize();
        hipMemcpy(out2, dout2, sizeof(out2), hipMemcpyDeviceToHost);
        hipMemcpy(na2, dna2, sizeof(na2), hipMemcpyDeviceToHost);
        CHECK(memcmp(out2, out, sizeof(out)) == 0 && memcmp(na2, na, sizeof(na)) == 0,
              "early-exit greedy equals greedy");
        hipFree(dv);
        hipFree(dcnt);
        hipFree(dmask);
        hipFree(dout2);
        hipFree(dna2);
    }

    /* sampling with the draft rows equal to the target rows: target rows
     * b*(K+1)+i, i < K, double as draft rows with stride (K+1)*V per sequence
     * is not expressible, so copy them into a [B][K][V] buffer */
    float* dy = NULL;
    CHECK(hipMalloc((void**)&dy, sizeof(float) * B * K * V) == hipSuccess, "hipMalloc");
    for (int b = 0; b < B; ++b)
        hipMemcpy(dy + (size_t)b * K * V, dz + (size_t)b * (K + 1) * V, sizeof(float) * K * V,
                  hipMemcpyDeviceToDevice);
    float px[B * K], qx[B * K];
    float *dpx = NULL, *dqx = NULL;
    hipMalloc((void**)&dpx, sizeof(px));
    hipMalloc((void**)&dqx, sizeof(qx));
    CHECK(spec_verify_sample(dz, V, dy, V, dx, du, 1.0f, B, K, V, SV_F32, dout, dna, dpx, dqx, ws, wsb, NULL) ==
              SV_OK,
          "sample call");
    hipDeviceSynchronize();
    hipMemcpy(out, dout, sizeof(out), hipMemcpyDeviceToHost);
    hipMemcpy(na, dna, sizeof(na), hipMemcpyDeviceToHost);
    hipMemcpy(px, dpx, sizeof(px), hipMemcpyDeviceToHost);
    hipMemcpy(qx, dqx, sizeof(qx), hipMemcpyDeviceToHost);
    for (int b = 0; b < B; ++b) {
        CHECK(na[b] == K, "sampling with p = q accepts every draft (sequence %d: %d)", b, na[b]);
        for (int i = 0; i < K; ++i) {
            CHECK(out[b * (K + 1) + i] == x[b * K + i], "sampled token %d.%d", b, i);
            CHECK(px[b * K + i] == qx[b * K + i] && px[b * K + i] > 0.0f, "p(x) = q(x) > 0 at %d.%d", b, i);
        }
        const int bonus = out[b * (K + 1) + K];
        CHECK(bonus >= 0 && bonus < V, "bonus token of sequence %d in range", b);
    }
    /* early-exit sampling on the same inputs: the same tokens, bit for bit */
    {
        int out2[B * (K + 1)], na2[B];
        CHECK(spec_verify_sample_lazy(dz, V, dy, V, dx, du, 1.0f, B, K, V, SV_F32, dout, dna, ws, wsb, NULL) ==
                  SV_OK,
              "sample_lazy call");
        hipDeviceSynchronize();
        hipMemcpy(out2, dout, sizeof(out2), hipMemcpyDeviceToHost);
        hipMemcpy(na2, dna, sizeof(na2), hipMemcpyDeviceToHost);
        CHECK(memcmp(out2, out, sizeof(out2)) == 0 && memcmp(na2, na, sizeof(na2)) == 0,
              "early-exit sampling equals sampling");
    }
    hipFree(dz);
    hipFree(dy);
    hipFree(du);
    hipFree(dx);
    hipFree(dout);
    hipFree(dna);
    hipFree(dpx);
    hipFree(dqx);
    hipFree(ws);
    free(z);
}

int main(int argc, char** argv)
{
    host_checks();
    if (argc > 1 && strcmp(argv[1], "gpu") == 0) gpu_checks();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("sv_client: all checks passed%s\n", argc > 1 ? " (gpu)" : "");
    return 0;
}
