/*
 * KDA oracle: the plain token-by-token recurrence in float64, on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this; only the tests, the
 * smoke check and the benchmark's CPU-baseline leg load it.  It shares no code, header or
 * constant with the HIP kernels.
 *
 * What it computes (one retention factor per key channel, decay first, then erase-and-write,
 * then read the updated state):
 *
 *   for every sequence n and head h, with S <- h0[n,h] (zeros when h0 is NULL), for each token t
 *   of the sequence in order:
 *       a      = exp(g[t,h,:])                 retention per key channel (alpha_t)
 *       S      = Diag(a) S                     fade
 *       pred   = S^T k[t,h,:]                  what the memory currently returns for k_t
 *       u      = beta[t,h] (v[t,h,:] - pred)   write only the error
 *       S      = S + k[t,h,:] u^T              erase along k_t and write v_t
 *       o[t,h] = S^T q[t,h,:]                  read the updated state
 *   and hT[n,h] = S after the last token.
 *
 * Sources (the pages this follows):
 *  - "Kimi K3's hybrid block, from first principles", section "From linear attention to the delta
 *    rule": the state is a dk x dv matrix; the delta rule reads the current prediction for k_t
 *    and writes only the error, which is one gradient step on 1/2 |S^T k_t - v_t|^2 with step
 *    beta_t; KDA makes the decay one factor per key channel, alpha_t in (0,1)^dk.
 *  - "Kimi K3, explained", section "Kimi Delta Attention: making the radical option work": per
 *    token first weakens what is stored, then clears the entry held for its key, then stores its
 *    value; k and v update S(t-1) and q reads the updated S(t).
 *  - "What's new in Kimi K3", section "KDA in one page": (I - beta k k^T) erases what the memory
 *    holds for the key before writing, and the forget gate alpha_t sits in front of it.
 * Expanding the fade/erase/write steps gives S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T,
 * o_t = S_t^T q_t.  No query scaling is applied (the pages state none; q arrives L2-normalised).
 *
 * gate_is_alpha = 1 (test use) passes alpha itself instead of log(alpha), so that dyadic test
 * inputs avoid the rounding of exp(log(alpha)).
 *
 * Snapshots (kda_oracle_recurrence_snap).  A cached prefix of a KDA layer can be resumed only from
 * a state saved at exactly that boundary, so states are saved every `stride` tokens ("Kimi K3's
 * hybrid block, from first principles", section "Gated MLA without positions", paragraph "The
 * cache, in bytes"; "What's new in Kimi K3", section "What it costs to serve").  After token
 * j * stride of sequence n (counted from the sequence start, j = 1 .. len_n / stride) the state
 * S is copied to snaps[snap_cu[n] + j - 1, h], a [dk, dv] block of snaps [*, H, dk, dv].
 *
 * Layouts (row-major, packed tokens): q,k,g [Ttot,H,dk]; v,o [Ttot,H,dv]; beta [Ttot,H];
 * h0,hT [N,H,dk,dv]; cu_seqlens int64 [N+1] (sequence n owns tokens cu[n] .. cu[n+1]-1).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *h0;
    const int64_t *cu;
    int64_t N, H, dk, dv;
    int gate_is_alpha;
    double *o, *hT;
    int64_t stride;         /* snapshot stride in tokens (0: no snapshots) */
    const int64_t *snap_cu; /* first snapshot index of each sequence */
    double *snaps;
    int64_t next;           /* next (sequence, head) unit to take */
    pthread_mutex_t lock;
    int status;
} job_t;

/* One (sequence, head) unit: the recurrence over the sequence's tokens. */
static int run_unit(job_t *J, int64_t unit, double *S, double *pred, double *u, double *a)
{
    const int64_t n = unit / J->H, h = unit % J->H;
    const int64_t H = J->H, dk = J->dk, dv = J->dv;
    const double *h0 = J->h0 ? J->h0 + (n * H + h) * dk * dv : NULL;
    for (int64_t i = 0; i < dk * dv; ++i) S[i] = h0 ? h0[i] : 0.0;

    for (int64_t t = J->cu[n]; t < J->cu[n + 1]; ++t) {
        const double *qt = J->q + (t * H + h) * dk;
        const double *kt = J->k + (t * H + h) * dk;
        const double *gt = J->g + (t * H + h) * dk;
        const double *vt = J->v + (t * H + h) * dv;
        const double bt = J->beta[t * H + h];
        double *ot = J->o + (t * H + h) * dv;

        /* fade: S <- Diag(alpha_t) S, one factor per key channel (row of S) */
        for (int64_t r = 0; r < dk; ++r) {
            a[r] = J->gate_is_alpha ? gt[r] : exp(gt[r]);
            for (int64_t c = 0; c < dv; ++c) S[r * dv + c] *= a[r];
        }
        /* prediction for k_t and the error term u = beta (v - S^T k) */
        for (int64_t c = 0; c < dv; ++c) pred[c] = 0.0;
        for (int64_t r = 0; r < dk; ++r)
            for (int64_t c = 0; c < dv; ++c) pred[c] += S[r * dv + c] * kt[r];
        for (int64_t c = 0; c < dv; ++c) u[c] = bt * (vt[c] - pred[c]);
        /* erase-and-write: S <- S + k u^T */
        for (int64_t r = 0; r < dk; ++r)
            for (int64_t c = 0; c < dv; ++c) S[r * dv + c] += kt[r] * u[c];
        /* read the updated state */
        for (int64_t c = 0; c < dv; ++c) ot[c] = 0.0;
        for (int64_t r = 0; r < dk; ++r)
            for (int64_t c = 0; c < dv; ++c) ot[c] += S[r * dv + c] * qt[r];
        /* the state that resumes the prefix ending after this token */
        const int64_t done = t - J->cu[n] + 1;
        if (J->stride > 0 && done % J->stride == 0) {
            double *snap = J->snaps + ((J->snap_cu[n] + done / J->stride - 1) * H + h) * dk * dv;
            for (int64_t i = 0; i < dk * dv; ++i) snap[i] = S[i];
        }
    }
    if (J->hT) {
        double *hT = J->hT + (n * H + h) * dk * dv;
        for (int64_t i = 0; i < dk * dv; ++i) hT[i] = S[i];
    }
    return 0;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)(J->dk * J->dv));
    double *pred = (double *)malloc(sizeof(double) * (size_t)J->dv);
    double *u = (double *)malloc(sizeof(double) * (size_t)J->dv);
    double *a = (double *)malloc(sizeof(double) * (size_t)J->dk);
    if (!S || !pred || !u || !a) {
        pthread_mutex_lock(&J->lock);
        J->status = -1;
        pthread_mutex_unlock(&J->lock);
    } else {
        for (;;) {
            pthread_mutex_lock(&J->lock);
            int64_t unit = J->next++;
            pthread_mutex_unlock(&J->lock);
            if (unit >= J->N * J->H) break;
            run_unit(J, unit, S, pred, u, a);
        }
    }
    free(S); free(pred); free(u); free(a);
    return NULL;
}

/* Returns 0 on success, -1 on allocation failure, -2 on bad arguments.  stride = 0 saves no
 * snapshots (snap_cu and snaps may then be NULL). */
int kda_oracle_recurrence_snap(const double *q, const double *k, const double *v, const double *g,
                               const double *beta, const double *h0, const int64_t *cu_seqlens,
                               int64_t num_seqs, int64_t H, int64_t dk, int64_t dv,
                               int gate_is_alpha, double *o, double *hT, int64_t stride,
                               const int64_t *snap_cu, double *snaps, int nthreads)
{
    if (!cu_seqlens || num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return -2;
    if (stride < 0 || (stride > 0 && (!snap_cu || !snaps))) return -2;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -2;
    if (cu_seqlens[num_seqs] > cu_seqlens[0] && (!q || !k || !v || !g || !beta || !o)) return -2;

    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0;
    J.cu = cu_seqlens; J.N = num_seqs; J.H = H; J.dk = dk; J.dv = dv;
    J.gate_is_alpha = gate_is_alpha; J.o = o; J.hT = hT;
    J.stride = stride; J.snap_cu = snap_cu; J.snaps = snaps;
    pthread_mutex_init(&J.lock, NULL);

    int64_t units = num_seqs * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = (int)(units > 0 ? units : 1);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -1;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &J) == 0) ++started;
    }
    if (started == 0) worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.lock);
    return J.status;
}

int kda_oracle_recurrence(const double *q, const double *k, const double *v, const double *g,
                          const double *beta, const double *h0, const int64_t *cu_seqlens,
                          int64_t num_seqs, int64_t H, int64_t dk, int64_t dv,
                          int gate_is_alpha, double *o, double *hT, int nthreads)
{
    return kda_oracle_recurrence_snap(q, k, v, g, beta, h0, cu_seqlens, num_seqs, H, dk, dv,
                                      gate_is_alpha, o, hT, 0, NULL, NULL, nthreads);
}
