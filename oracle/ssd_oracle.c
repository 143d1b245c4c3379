/*
 * ssd_oracle.c -- plain, slow, sequential fp64 reference of the Mamba-2 SSD
 * recurrence.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * What it computes.  "Compiler-First State Space Duality and Portable O(1)
 * Autoregressive Caching for Inference" (section 2, methodology) describes the
 * SSD layer as a per-head diagonal state recurrence that can be cut into
 * fixed-size chunks, with the decay exponentiated in float32, and (section 3)
 * an O(1) per-sequence state cache that decoding updates one token at a time.
 * The page never writes the recurrence out; this file takes the plainest
 * reading consistent with that description -- the Mamba-2 SSD layer with a
 * scalar-times-identity state matrix per head -- as the definition.  For each
 * batch row b and head h, with group g = h / (H / G), starting from the
 * initial state H_0 (zero unless given), for t = 1 .. L:
 *
 *     alpha_t = exp(dt[b,t,h] * A[h])
 *     H_t     = alpha_t * H_{t-1} + dt[b,t,h] * x[b,t,h,:] (outer) B[b,t,g,:]
 *     y[b,t,h,:] = H_t . C[b,t,g,:] + D[h] * x[b,t,h,:]
 *
 * H_t is headdim x dstate (P x N), row p, column n.  The output reads the
 * state *after* the update (token t sees itself).  The final state is H_L.
 * A decode step is exactly one more iteration of the same loop on a cached
 * state (section 2: the on-device O(1) cache).  Everything is fp64; inputs are
 * widened exactly from their stored precision by the caller.
 *
 * Threads only split independent (b, h) pairs; every pair runs its t loop in
 * order, so the result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups;
    const double *x, *dt, *A, *B, *C, *D, *h0;
    double *y, *hL;
    int64_t next;            /* next (b, h) pair to run */
    pthread_mutex_t lock;
} oracle_job;

/* One (b, h) recurrence, t = 0 .. L-1 in order. */
static void run_pair(const oracle_job *j, int64_t b, int64_t h, double *S)
{
    const int64_t L = j->seqlen, H = j->nheads, P = j->headdim, N = j->dstate;
    const int64_t g = h / (H / j->ngroups);
    const double A = j->A[h], D = j->D[h];

    if (j->h0)
        memcpy(S, j->h0 + (b * H + h) * P * N, sizeof(double) * P * N);
    else
        memset(S, 0, sizeof(double) * P * N);

    for (int64_t t = 0; t < L; ++t) {
        const double dt = j->dt[(b * L + t) * H + h];
        const double alpha = exp(dt * A);
        const double *xt = j->x + ((b * L + t) * H + h) * P;
        const double *Bt = j->B + ((b * L + t) * j->ngroups + g) * N;
        const double *Ct = j->C + ((b * L + t) * j->ngroups + g) * N;
        double *yt = j->y + ((b * L + t) * H + h) * P;
        for (int64_t p = 0; p < P; ++p) {
            double *row = S + p * N;
            const double u = dt * xt[p];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                row[n] = alpha * row[n] + u * Bt[n];
                acc += row[n] * Ct[n];
            }
            yt[p] = acc + D * xt[p];
        }
    }
    memcpy(j->hL + (b * H + h) * P * N, S, sizeof(double) * P * N);
}

static void *worker(void *arg)
{
    oracle_job *j = (oracle_job *)arg;
    const int64_t pairs = j->batch * j->nheads;
    double *S = (double *)malloc(sizeof(double) * (size_t)(j->headdim * j->dstate));
    if (!S)
        return (void *)1;
    for (;;) {
        pthread_mutex_lock(&j->lock);
        const int64_t k = j->next++;
        pthread_mutex_unlock(&j->lock);
        if (k >= pairs)
            break;
        run_pair(j, k / j->nheads, k % j->nheads, S);
    }
    free(S);
    return NULL;
}

/*
 * ssd_oracle_scan: run the recurrence over a whole [batch, seqlen] input.
 *   x  [batch, seqlen, nheads, headdim]   dt [batch, seqlen, nheads]
 *   A  [nheads]    D [nheads]             B, C [batch, seqlen, ngroups, dstate]
 *   h0 [batch, nheads, headdim, dstate] or NULL (zero initial state)
 *   y  [batch, seqlen, nheads, headdim]  (out)
 *   hL [batch, nheads, headdim, dstate]  (out, final state)
 * All arrays are contiguous row-major fp64 in host memory.  nthreads <= 0
 * means one thread.  Returns 0, or -1 on bad sizes / allocation failure.
 */
int ssd_oracle_scan(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                    int64_t dstate, int64_t ngroups,
                    const double *x, const double *dt, const double *A,
                    const double *B, const double *C, const double *D,
                    const double *h0, double *y, double *hL, int nthreads)
{
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 ||
        ngroups <= 0 || nheads % ngroups != 0)
        return -1;
    oracle_job j = {batch, seqlen, nheads, headdim, dstate, ngroups,
                    x, dt, A, B, C, D, h0, y, hL, 0, PTHREAD_MUTEX_INITIALIZER};
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads == 1)
        return worker(&j) == NULL ? 0 : -1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid)
        return -1;
    int started = 0, rc = 0;
    for (; started < nthreads; ++started)
        if (pthread_create(&tid[started], NULL, worker, &j) != 0)
            break;
    if (started == 0)
        rc = worker(&j) == NULL ? 0 : -1;
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(tid[i], &r);
        if (r != NULL)
            rc = -1;
    }
    free(tid);
    return rc;
}
