/*
 * ssd_oracle.c -- fp64 CPU oracle for the SSD (state space dual) layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file or the library built from it: only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark use it.  It shares no code, header,
 * table or helper with the HIP library.
 *
 * What it computes (the plain definition, token by token):
 *
 *   "Mamba-2: Attention's Distant Cousin" (docsaid.org), section "Writing an SSM
 *   as a Matrix": the selective SSM recurrence h_t = A_t h_{t-1} + B_t x_t,
 *   y_t = C_t^T h_t.  Section "Reducing A to a Single Number": A_t = a_t I, one
 *   scalar decay per step, which is the SSD case.  Section "The Mamba-2 Block":
 *   heads of dimension P, with B and C shared across the heads of a group.
 *
 *   The pages leave the discretisation open.  The reading taken here: the decay
 *   of head h at step t is a = exp(dt[b,t,h] * A[h]), the input is scaled by
 *   dt[b,t,h], and a per-head skip D[h] * x is added to the output:
 *
 *     S  <- a * S + dt * B_t x_t^T            (S is N x P, one per (b, h))
 *     y_t = C_t^T S + D[h] * x_t              (sum over n in ascending order)
 *
 *   The state entering step 0 is init_state (zeros when none is given), so it
 *   is decayed by a_0 like any other carried state.  Head h reads group
 *   g = h / (H / G) of B and C (contiguous heads share a group).
 *
 * Layouts (row-major, contiguous):
 *   x, y                   [batch][seqlen][nheads][headdim]
 *   dt                     [batch][seqlen][nheads]
 *   A, D                   [nheads]
 *   B, C                   [batch][seqlen][ngroups][dstate]
 *   init_state, final      [batch][nheads][dstate][headdim]
 *   boundary_states        [batch][nheads][nchunks][dstate][headdim]
 *
 * Every (batch, head) pair is an independent sequence; the only parallelism is
 * one POSIX thread per group of such pairs.  Each pair's arithmetic is done in
 * one thread in a fixed order, so results do not depend on the thread count.
 */
#include "ssd_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const ssd_ref_dims* d;
    const double *x, *dt, *A, *B, *C, *D, *init_state;
    double *y, *final_state, *boundary_states;
    int64_t chunk_len;
    int thread_index, nthreads;
    int failed;
} ref_job;

/* One (batch, head) sequence through the recurrence. */
static void run_sequence(const ref_job* j, int64_t b, int64_t h, double* S)
{
    const ssd_ref_dims* d = j->d;
    const int64_t T = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
    const int64_t heads_per_group = H / G;
    const int64_t g = h / heads_per_group;
    const int64_t nchunks = j->chunk_len > 0 ? (T + j->chunk_len - 1) / j->chunk_len : 0;

    if (j->init_state)
        memcpy(S, j->init_state + (b * H + h) * N * P, (size_t)(N * P) * sizeof(double));
    else
        memset(S, 0, (size_t)(N * P) * sizeof(double));

    for (int64_t t = 0; t < T; ++t) {
        const double dt = j->dt[(b * T + t) * H + h];
        const double a = exp(dt * j->A[h]);
        const double* xt = j->x + ((b * T + t) * H + h) * P;
        const double* Bt = j->B + ((b * T + t) * G + g) * N;
        const double* Ct = j->C + ((b * T + t) * G + g) * N;
        double* yt = j->y + ((b * T + t) * H + h) * P;

        /* state update: S = a S + dt B_t x_t^T */
        for (int64_t n = 0; n < N; ++n) {
            const double wb = dt * Bt[n];
            double* Sn = S + n * P;
            for (int64_t p = 0; p < P; ++p)
                Sn[p] = a * Sn[p] + wb * xt[p];
        }
        /* readout: y_t = C_t^T S + D x_t */
        for (int64_t p = 0; p < P; ++p) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n)
                acc += Ct[n] * S[n * P + p];
            yt[p] = acc + j->D[h] * xt[p];
        }
        /* the state at the last step of each chunk (or of the sequence) */
        if (j->boundary_states && ((t + 1) % j->chunk_len == 0 || t == T - 1)) {
            const int64_t c = t / j->chunk_len;
            memcpy(j->boundary_states + ((b * H + h) * nchunks + c) * N * P, S,
                   (size_t)(N * P) * sizeof(double));
        }
    }
    if (j->final_state)
        memcpy(j->final_state + (b * H + h) * N * P, S, (size_t)(N * P) * sizeof(double));
}

static void* ref_worker(void* arg)
{
    ref_job* j = (ref_job*)arg;
    const ssd_ref_dims* d = j->d;
    double* S = (double*)malloc((size_t)(d->dstate * d->headdim) * sizeof(double));
    if (!S) {
        j->failed = 1;
        return NULL;
    }
    const int64_t tasks = d->batch * d->nheads;
    for (int64_t k = j->thread_index; k < tasks; k += j->nthreads)
        run_sequence(j, k / d->nheads, k % d->nheads, S);
    free(S);
    return NULL;
}

int ssd_ref(const ssd_ref_dims* d, const double* x, const double* dt, const double* A,
            const double* B, const double* C, const double* D, const double* init_state,
            int64_t chunk_len, double* y, double* final_state, double* boundary_states,
            int nthreads)
{
    if (!d || !x || !dt || !A || !B || !C || !D || !y)
        return SSD_REF_ERR_NULL;
    if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
        d->ngroups < 1 || d->nheads % d->ngroups != 0)
        return SSD_REF_ERR_DIMS;
    if (boundary_states && chunk_len < 1)
        return SSD_REF_ERR_DIMS;
    if (chunk_len < 0)
        return SSD_REF_ERR_DIMS;

    const int64_t tasks = d->batch * d->nheads;
    if (tasks == 0)
        return SSD_REF_OK;
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > tasks)
        nthreads = (int)tasks;

    ref_job* jobs = (ref_job*)calloc((size_t)nthreads, sizeof(ref_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return SSD_REF_ERR_ALLOC;
    }
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (ref_job){d, x, dt, A, B, C, D, init_state, y, final_state, boundary_states,
                            chunk_len, i, nthreads, 0};
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, ref_worker, &jobs[i]) != 0)
            break;
        started = i;
    }
    /* thread 0's share runs here; shares whose thread failed to start run here too */
    ref_worker(&jobs[0]);
    for (int i = started + 1; i < nthreads; ++i)
        ref_worker(&jobs[i]);
    for (int i = 1; i <= started; ++i)
        pthread_join(th[i], NULL);

    int failed = 0;
    for (int i = 0; i < nthreads; ++i)
        failed |= jobs[i].failed;
    free(jobs);
    free(th);
    return failed ? SSD_REF_ERR_ALLOC : SSD_REF_OK;
}

int ssd_ref_threads_used(const ssd_ref_dims* d, int nthreads)
{
    if (!d)
        return 0;
    const int64_t tasks = d->batch * d->nheads;
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > tasks)
        nthreads = (int)(tasks > 0 ? tasks : 1);
    return nthreads;
}
