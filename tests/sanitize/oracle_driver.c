/*
 * The float64 oracle (oracle/kda_oracle.c) under AddressSanitizer + UndefinedBehaviorSanitizer,
 * and under ThreadSanitizer for its worker threads (built by tests/test_sanitizers.py).
 *
 * Every buffer is heap memory of exactly the size the call may touch.  Checks, beyond the
 * sanitizers' own reports:
 *   - the result does not depend on the number of worker threads (bit for bit);
 *   - an empty sequence returns its h0 unchanged, and zeros without h0;
 *   - the snapshots of a sequence end with its final state when the length is a multiple of the
 *     stride;
 *   - beta = 0 is pure per-channel decay: S_t = Diag(exp(sum of g up to t)) h0, o_t = S_t^T q_t;
 *   - bad arguments return -2 and write nothing.
 * Exit status 0 when all hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_recurrence_snap(const double *q, const double *k, const double *v, const double *g,
                               const double *beta, const double *h0, const int64_t *cu_seqlens,
                               int64_t num_seqs, int64_t H, int64_t dk, int64_t dv,
                               int gate_is_alpha, double *o, double *hT, int64_t stride,
                               const int64_t *snap_cu, double *snaps, int nthreads);
int kda_oracle_recurrence(const double *q, const double *k, const double *v, const double *g,
                          const double *beta, const double *h0, const int64_t *cu_seqlens,
                          int64_t num_seqs, int64_t H, int64_t dk, int64_t dv,
                          int gate_is_alpha, double *o, double *hT, int nthreads);

static int failures = 0;
#define EXPECT(c)                                                                     \
    do {                                                                              \
        if (!(c)) {                                                                   \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                               \
        }                                                                             \
    } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) /* splitmix64 -> [0, 1) */
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static double *alloc_fill(size_t n, double lo, double hi)
{
    double *p = (double *)malloc(n * sizeof(double) + 1);
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uniform();
    return p;
}

int main(void)
{
    enum { H = 2, DK = 5, DV = 3, N = 4 };
    const int64_t cu[N + 1] = {0, 7, 7, 23, 39}; /* lengths 7, 0, 16, 16 */
    const int64_t Tt = cu[N];
    double *q = alloc_fill((size_t)Tt * H * DK, -1, 1), *k = alloc_fill((size_t)Tt * H * DK, -1, 1);
    double *v = alloc_fill((size_t)Tt * H * DV, -1, 1), *g = alloc_fill((size_t)Tt * H * DK, -5, 0);
    double *beta = alloc_fill((size_t)Tt * H, 0, 1), *h0 = alloc_fill((size_t)N * H * DK * DV, -1, 1);
    const size_t no = (size_t)Tt * H * DV, ns = (size_t)N * H * DK * DV;
    double *o1 = (double *)calloc(no, sizeof(double)), *o4 = (double *)calloc(no, sizeof(double));
    double *h1 = (double *)calloc(ns, sizeof(double)), *h4 = (double *)calloc(ns, sizeof(double));

    EXPECT(kda_oracle_recurrence(q, k, v, g, beta, h0, cu, N, H, DK, DV, 0, o1, h1, 1) == 0);
    EXPECT(kda_oracle_recurrence(q, k, v, g, beta, h0, cu, N, H, DK, DV, 0, o4, h4, 4) == 0);
    EXPECT(memcmp(o1, o4, no * sizeof(double)) == 0);
    EXPECT(memcmp(h1, h4, ns * sizeof(double)) == 0);
    /* sequence 1 is empty: its final state is its h0 */
    EXPECT(memcmp(h1 + (size_t)1 * H * DK * DV, h0 + (size_t)1 * H * DK * DV,
                  (size_t)H * DK * DV * sizeof(double)) == 0);
    /* without h0 the empty sequence ends at zero */
    EXPECT(kda_oracle_recurrence(q, k, v, g, beta, NULL, cu, N, H, DK, DV, 0, o1, h1, 3) == 0);
    for (size_t i = 0; i < (size_t)H * DK * DV; ++i) EXPECT(h1[(size_t)1 * H * DK * DV + i] == 0.0);

    /* snapshots every 8 tokens: 0, 0, 2, 2 per sequence */
    const int64_t scu[N + 1] = {0, 0, 0, 2, 4};
    double *snaps = (double *)calloc((size_t)4 * H * DK * DV, sizeof(double));
    EXPECT(kda_oracle_recurrence_snap(q, k, v, g, beta, h0, cu, N, H, DK, DV, 0, o1, h1, 8, scu,
                                      snaps, 2) == 0);
    for (int n = 2; n < 4; ++n)
        EXPECT(memcmp(snaps + (size_t)(scu[n] + 1) * H * DK * DV, h1 + (size_t)n * H * DK * DV,
                      (size_t)H * DK * DV * sizeof(double)) == 0);

    /* beta = 0: pure decay of h0 */
    double *b0 = (double *)calloc((size_t)Tt * H, sizeof(double));
    EXPECT(kda_oracle_recurrence(q, k, v, g, b0, h0, cu, N, H, DK, DV, 0, o1, h1, 2) == 0);
    double worst = 0;
    for (int n = 0; n < N; ++n)
        for (int h = 0; h < H; ++h) {
            double G[DK] = {0};
            for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
                for (int r = 0; r < DK; ++r) G[r] += g[(t * H + h) * DK + r];
                for (int c = 0; c < DV; ++c) {
                    double acc = 0;
                    for (int r = 0; r < DK; ++r)
                        acc += q[(t * H + h) * DK + r] * exp(G[r]) *
                               h0[(((size_t)n * H + h) * DK + r) * DV + c];
                    worst = fmax(worst, fabs(acc - o1[(t * H + h) * DV + c]));
                }
            }
        }
    EXPECT(worst < 1e-12);

    /* bad arguments: -2, nothing written */
    const int64_t bad_cu[3] = {0, 5, 3};
    double *canary = (double *)calloc(no, sizeof(double));
    EXPECT(kda_oracle_recurrence(q, k, v, g, beta, h0, bad_cu, 2, H, DK, DV, 0, canary, h1, 1) == -2);
    EXPECT(kda_oracle_recurrence(q, k, v, g, beta, h0, NULL, 2, H, DK, DV, 0, canary, h1, 1) == -2);
    EXPECT(kda_oracle_recurrence(q, k, v, g, beta, h0, cu, N, 0, DK, DV, 0, canary, h1, 1) == -2);
    EXPECT(kda_oracle_recurrence(NULL, k, v, g, beta, h0, cu, N, H, DK, DV, 0, canary, h1, 1) == -2);
    EXPECT(kda_oracle_recurrence_snap(q, k, v, g, beta, h0, cu, N, H, DK, DV, 0, canary, h1, 8,
                                      NULL, snaps, 1) == -2);
    for (size_t i = 0; i < no; ++i) EXPECT(canary[i] == 0.0);

    free(q); free(k); free(v); free(g); free(beta); free(h0); free(o1); free(o4); free(h1);
    free(h4); free(snaps); free(b0); free(canary);
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all expectations hold\n");
    return 0;
}
