/*
 * ssd_oracle.c -- fp64 CPU oracle for the SSD (state space dual) layer, forward and
 * backward.
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

/*
 * ---------------------------------------------------------------------------------
 * Backward: the gradient of a scalar loss L with respect to every input, given
 * dL/dy for every output step and dL/d(final state).  This is reverse-mode
 * differentiation of the recurrence above, one step at a time, written out by hand:
 *
 *   forward   S_t = a_t S_{t-1} + dt_t B_t x_t^T,   a_t = exp(dt_t A),
 *             y_t = C_t^T S_t + D x_t,               S_{-1} = init_state
 *   reverse   Lam_t = dL/dS_t (every use of S_t, i.e. through y_t and S_{t+1}):
 *             Lam_{T-1} = C_{T-1} dy_{T-1}^T + d_final
 *             Lam_t     = C_t dy_t^T + a_{t+1} Lam_{t+1}
 *   then      dx_t  = D dy_t + dt_t Lam_t^T B_t
 *             dB_t += dt_t Lam_t x_t             (summed over the heads of the group)
 *             dC_t += S_t dy_t                   (summed over the heads of the group)
 *             ddt_t = B_t^T Lam_t x_t + A a_t <S_{t-1}, Lam_t>
 *             dA   += dt_t a_t <S_{t-1}, Lam_t>  (summed over batch and time)
 *             dD   += <x_t, dy_t>
 *             d_init = a_0 Lam_0
 * (<U, V> is the sum of the elementwise product of two N x P matrices.)
 *
 * The forward states are needed in reverse order.  They are recomputed segment by
 * segment from checkpoints: the state entering every segment of kSeg steps is kept
 * from one forward sweep, and before a segment is walked backwards its kSeg states
 * are recomputed from that checkpoint with the same arithmetic as the forward.
 *
 * Outputs per (batch, head) task, so that no two threads write the same element:
 *   dx [B][T][H][P], ddt [B][T][H], dB_heads and dC_heads [B][T][H][N] (this head's
 *   share; the caller sums the heads of a group), dA_parts and dD_parts [B][H]
 *   (the caller sums over batch), d_init [B][H][N][P] or NULL, and boundary_grads
 *   [B][H][nchunks][N][P] or NULL: for every chunk, dL/d(the state after the chunk's
 *   last step) through the later steps only -- the gradient of the state that enters
 *   the next chunk (d_final for the last chunk).
 * ---------------------------------------------------------------------------------
 */
enum { kSeg = 64 };

typedef struct {
    const ssd_ref_dims* d;
    const double *x, *dt, *A, *B, *C, *D, *init_state, *dy, *d_final;
    double *dx, *ddt, *dB_heads, *dC_heads, *dA_parts, *dD_parts, *d_init, *boundary_grads;
    int64_t chunk_len;
    int thread_index, nthreads;
    int failed;
} bwd_job;

/* S <- a S + dt B_t x_t^T for one step (the forward update, as in run_sequence) */
static void step_state(double* S, double a, double dt, const double* Bt, const double* xt,
                       int64_t N, int64_t P)
{
    for (int64_t n = 0; n < N; ++n) {
        const double w = dt * Bt[n];
        double* row = S + n * P;
        for (int64_t p = 0; p < P; ++p)
            row[p] = a * row[p] + w * xt[p];
    }
}

static void run_sequence_bwd(const bwd_job* j, int64_t b, int64_t h, double* ckpt, double* seg,
                             double* Lam)
{
    const ssd_ref_dims* d = j->d;
    const int64_t T = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
    const int64_t NP = N * P;
    const int64_t g = h / (H / G);
    const int64_t nseg = (T + kSeg - 1) / kSeg;
    const int64_t nchunks = j->chunk_len > 0 ? (T + j->chunk_len - 1) / j->chunk_len : 0;
    const double Ah = j->A[h], Dh = j->D[h];
#define XT(t) (j->x + ((b * T + (t)) * H + h) * P)
#define DYT(t) (j->dy + ((b * T + (t)) * H + h) * P)
#define BT(t) (j->B + ((b * T + (t)) * G + g) * N)
#define CT(t) (j->C + ((b * T + (t)) * G + g) * N)
#define DTT(t) (j->dt[(b * T + (t)) * H + h])

    /* forward sweep: keep the state entering every segment */
    double* S = seg; /* seg[0] doubles as the running state here */
    if (j->init_state != NULL)
        memcpy(S, j->init_state + (b * H + h) * NP, (size_t)NP * sizeof(double));
    else
        memset(S, 0, (size_t)NP * sizeof(double));
    for (int64_t t = 0; t < T; t++) {
        if (t % kSeg == 0)
            memcpy(ckpt + (t / kSeg) * NP, S, (size_t)NP * sizeof(double));
        step_state(S, exp(DTT(t) * Ah), DTT(t), BT(t), XT(t), N, P);
    }

    /* reverse sweep */
    if (j->d_final)
        memcpy(Lam, j->d_final + (b * H + h) * NP, (size_t)NP * sizeof(double));
    else
        memset(Lam, 0, (size_t)NP * sizeof(double));
    double dA_acc = 0.0, dD_acc = 0.0;
    for (int64_t s = nseg - 1; s >= 0; --s) {
        const int64_t t0 = s * kSeg, t1 = (t0 + kSeg < T) ? t0 + kSeg : T;
        /* seg[k] = state after step t0 + k - 1 (seg[0] = the state entering t0) */
        memcpy(seg, ckpt + s * NP, (size_t)NP * sizeof(double));
        for (int64_t t = t0; t < t1; ++t) {
            double* nxt = seg + (t - t0 + 1) * NP;
            memcpy(nxt, seg + (t - t0) * NP, (size_t)NP * sizeof(double));
            step_state(nxt, exp(DTT(t) * Ah), DTT(t), BT(t), XT(t), N, P);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            /* Lam holds dL/dS_t through the later steps; a chunk's last step records it */
            if (j->boundary_grads && (t % j->chunk_len == j->chunk_len - 1 || t == T - 1)) {
                const int64_t c = t / j->chunk_len;
                memcpy(j->boundary_grads + ((b * H + h) * nchunks + c) * NP, Lam,
                       (size_t)NP * sizeof(double));
            }
            const double* xt = XT(t);
            const double* dyt = DYT(t);
            const double* Bt = BT(t);
            const double* Ct = CT(t);
            const double dtt = DTT(t);
            const double a = exp(dtt * Ah);
            const double* S_prev = seg + (t - t0) * NP;
            const double* S_t = seg + (t - t0 + 1) * NP;
            /* add this step's own use of S_t: y_t = C_t^T S_t */
            for (int64_t n = 0; n < N; ++n)
                for (int64_t p = 0; p < P; ++p)
                    Lam[n * P + p] += Ct[n] * dyt[p];
            /* dC_t (this head) = S_t dy_t */
            double* dCt = j->dC_heads + ((b * T + t) * H + h) * N;
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t p = 0; p < P; ++p)
                    acc += S_t[n * P + p] * dyt[p];
                dCt[n] = acc;
            }
            /* dx_t = D dy_t + dt Lam^T B_t */
            double* dxt = j->dx + ((b * T + t) * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += Bt[n] * Lam[n * P + p];
                dxt[p] = Dh * dyt[p] + dtt * acc;
            }
            /* u = Lam x_t; dB_t (this head) = dt u; the explicit dt term is B_t . u */
            double* dBt = j->dB_heads + ((b * T + t) * H + h) * N;
            double direct = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double u = 0.0;
                for (int64_t p = 0; p < P; ++p)
                    u += Lam[n * P + p] * xt[p];
                dBt[n] = dtt * u;
                direct += Bt[n] * u;
            }
            /* q = <S_{t-1}, Lam_t>: the decay a = exp(dt A) seen from dt and from A */
            double q = 0.0;
            for (int64_t k = 0; k < NP; ++k)
                q += S_prev[k] * Lam[k];
            j->ddt[(b * T + t) * H + h] = direct + Ah * a * q;
            dA_acc += dtt * a * q;
            for (int64_t p = 0; p < P; ++p)
                dD_acc += xt[p] * dyt[p];
            /* on to dL/dS_{t-1} through the later steps */
            for (int64_t k = 0; k < NP; ++k)
                Lam[k] *= a;
        }
    }
    if (j->d_init)
        memcpy(j->d_init + (b * H + h) * NP, Lam, (size_t)NP * sizeof(double));
    j->dA_parts[b * H + h] = dA_acc;
    j->dD_parts[b * H + h] = dD_acc;
#undef XT
#undef DYT
#undef BT
#undef CT
#undef DTT
}

static void* bwd_worker(void* arg)
{
    bwd_job* j = (bwd_job*)arg;
    const ssd_ref_dims* d = j->d;
    const int64_t NP = d->dstate * d->headdim;
    const int64_t nseg = (d->seqlen + kSeg - 1) / kSeg;
    double* ckpt = (double*)malloc((size_t)((nseg > 0 ? nseg : 1) * NP) * sizeof(double));
    double* seg = (double*)malloc((size_t)((kSeg + 1) * NP) * sizeof(double));
    double* Lam = (double*)malloc((size_t)NP * sizeof(double));
    if (!ckpt || !seg || !Lam) {
        j->failed = 1;
    } else {
        const int64_t tasks = d->batch * d->nheads;
        for (int64_t k = j->thread_index; k < tasks; k += j->nthreads)
            run_sequence_bwd(j, k / d->nheads, k % d->nheads, ckpt, seg, Lam);
    }
    free(ckpt);
    free(seg);
    free(Lam);
    return NULL;
}

int ssd_bwd_ref(const ssd_ref_dims* d, const double* x, const double* dt, const double* A,
                const double* B, const double* C, const double* D, const double* init_state,
                const double* dy, const double* d_final, int64_t chunk_len, double* dx,
                double* ddt, double* dB_heads, double* dC_heads, double* dA_parts,
                double* dD_parts, double* d_init, double* boundary_grads, int nthreads)
{
    if (!d || !x || !dt || !A || !B || !C || !D || !dy || !dx || !ddt || !dB_heads ||
        !dC_heads || !dA_parts || !dD_parts)
        return SSD_REF_ERR_NULL;
    if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
        d->ngroups < 1 || d->nheads % d->ngroups != 0)
        return SSD_REF_ERR_DIMS;
    if (chunk_len < 0 || (boundary_grads && chunk_len < 1))
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

    bwd_job* jobs = (bwd_job*)calloc((size_t)nthreads, sizeof(bwd_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return SSD_REF_ERR_ALLOC;
    }
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (bwd_job){d, x, dt, A, B, C, D, init_state, dy, d_final, dx, ddt, dB_heads,
                            dC_heads, dA_parts, dD_parts, d_init, boundary_grads, chunk_len,
                            i, nthreads, 0};
    }
    int started = 0;
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, bwd_worker, &jobs[i]) != 0)
            break;
        started = i;
    }
    bwd_worker(&jobs[0]);
    for (int i = started + 1; i < nthreads; ++i)
        bwd_worker(&jobs[i]);
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
