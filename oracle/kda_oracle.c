/*
 * Plain fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or helper with the HIP
 * library: it is written from the recurrence on the pages, not from the
 * kernels.
 *
 * What it computes, per sequence n and head h, for tokens t in order
 * (state S is dk x dv, outputs read the post-update state):
 *
 *     S_t = (I - b_t k_t k_t^T) Diag(alpha_t) S_{t-1} + b_t k_t v_t^T
 *     o_t = S_t^T q_t,      alpha_t = exp(g_t)   (natural log, per channel)
 *
 *   "Kimi K3.1 Pro 架构完全拆解", §3.1 (single-head recurrence) and §3.2
 *   (the bounded log-decay gate alpha = exp(g)).
 *
 * It evaluates that recurrence in the algebraically identical "u form"
 *
 *     DS = Diag(alpha_t) S_{t-1}
 *     u_t = b_write * v_t - b_erase * DS^T k_t
 *     S_t = DS + k_t u_t^T
 *     o_t = S_t^T q_t
 *
 *   "Kimi K3 的架構" (hao.cnyes.com), §六 FlashKDA 演算法, the alternative
 *   form of the recurrence that the decode kernel follows.
 *
 * For KDA b_erase = b_write = beta.  Keeping the two apart only serves a
 * test that switches the erase term off (plain linear attention,
 * "Kimi K3 的架構" §三).
 *
 * The segment transition follows "部署 Kimi K3：从 KDA Kernel 到 Fleet 调度",
 * §二 (KCP math): M = M_T ... M_1 with M_r = (I - b_r k_r k_r^T) Diag(alpha_r),
 * formed as explicit dk x dk products, and S~ = the recurrence run from S = 0,
 * so that the state after the segment is S~ + M S_in.
 *
 * Layouts (row-major, last index fastest):
 *   q, k, g : [T_total, H, dk]      v, o : [T_total, H, dv]
 *   beta    : [T_total, H]          states : [num_seqs, H, dk, dv]
 *   M       : [num_segs, H, dk, dk]
 * Sequence n owns tokens [cu[n], cu[n+1]).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    int32_t num_seqs;
    const int64_t *cu;
    int32_t H, dk, dv;
    const double *q, *k, *v, *g, *b_erase, *b_write;
    const double *init;   /* may be NULL: zero initial state */
    double *o;            /* may be NULL: outputs not wanted */
    double *final_state;  /* may be NULL */
    double *M;            /* segment mode only: [num_seqs, H, dk, dk] */
    int explicit_m;       /* 1: also form M by explicit products */
    int64_t next_task;    /* shared task counter (guarded by lock) */
    pthread_mutex_t lock;
    int failed;
} oracle_job;

static int64_t take_task(oracle_job *job)
{
    int64_t t;
    pthread_mutex_lock(&job->lock);
    t = job->next_task++;
    pthread_mutex_unlock(&job->lock);
    return t;
}

/* One (sequence, head) task: the u-form recurrence, and optionally the
 * explicit product of per-token transition matrices. */
static int run_task(oracle_job *job, int64_t task)
{
    const int32_t H = job->H, dk = job->dk, dv = job->dv;
    const int32_t n = (int32_t)(task / H), h = (int32_t)(task % H);
    const int64_t t0 = job->cu[n], t1 = job->cu[n + 1];
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *w = (double *)malloc(sizeof(double) * (size_t)dv);
    double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
    double *Mr = NULL, *Mprod = NULL, *Mtmp = NULL;
    if (!S || !w || !alpha) {
        free(S); free(w); free(alpha);
        return -1;
    }
    if (job->explicit_m) {
        Mr = (double *)malloc(sizeof(double) * (size_t)dk * dk);
        Mprod = (double *)malloc(sizeof(double) * (size_t)dk * dk);
        Mtmp = (double *)malloc(sizeof(double) * (size_t)dk * dk);
        if (!Mr || !Mprod || !Mtmp) {
            free(S); free(w); free(alpha); free(Mr); free(Mprod); free(Mtmp);
            return -1;
        }
        for (int32_t i = 0; i < dk; ++i)
            for (int32_t j = 0; j < dk; ++j)
                Mprod[(size_t)i * dk + j] = (i == j) ? 1.0 : 0.0;
    }

    const size_t sidx = ((size_t)n * H + h) * (size_t)dk * dv;
    if (job->init)
        memcpy(S, job->init + sidx, sizeof(double) * (size_t)dk * dv);
    else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);

    for (int64_t t = t0; t < t1; ++t) {
        const size_t row = (size_t)t * H + h;
        const double *qt = job->q ? job->q + row * dk : NULL;
        const double *kt = job->k + row * dk;
        const double *vt = job->v + row * dv;
        const double *gt = job->g + row * dk;
        const double be = job->b_erase[row];
        const double bw = job->b_write[row];

        /* alpha_t = exp(g_t), one retention factor per key channel */
        for (int32_t i = 0; i < dk; ++i)
            alpha[i] = exp(gt[i]);

        /* DS = Diag(alpha) S : the decay scales the rows (key channels) */
        for (int32_t i = 0; i < dk; ++i)
            for (int32_t j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] *= alpha[i];

        /* w = DS^T k */
        for (int32_t j = 0; j < dv; ++j)
            w[j] = 0.0;
        for (int32_t i = 0; i < dk; ++i) {
            const double ki = kt[i];
            for (int32_t j = 0; j < dv; ++j)
                w[j] += ki * S[(size_t)i * dv + j];
        }
        /* u = b_write v - b_erase w ;  S = DS + k u^T */
        for (int32_t j = 0; j < dv; ++j)
            w[j] = bw * vt[j] - be * w[j];
        for (int32_t i = 0; i < dk; ++i) {
            const double ki = kt[i];
            for (int32_t j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] += ki * w[j];
        }
        /* o = S^T q (post-update state) */
        if (job->o && qt) {
            double *ot = job->o + row * dv;
            for (int32_t j = 0; j < dv; ++j)
                ot[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i) {
                const double qi = qt[i];
                for (int32_t j = 0; j < dv; ++j)
                    ot[j] += qi * S[(size_t)i * dv + j];
            }
        }

        if (job->explicit_m) {
            /* M_r = (I - b k k^T) Diag(alpha):  (M_r)_ij = (d_ij - b k_i k_j) alpha_j */
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dk; ++j)
                    Mr[(size_t)i * dk + j] =
                        ((i == j ? 1.0 : 0.0) - be * kt[i] * kt[j]) * alpha[j];
            /* Mprod <- M_r * Mprod  (latest factor on the left) */
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t j = 0; j < dk; ++j) {
                    double acc = 0.0;
                    for (int32_t m = 0; m < dk; ++m)
                        acc += Mr[(size_t)i * dk + m] * Mprod[(size_t)m * dk + j];
                    Mtmp[(size_t)i * dk + j] = acc;
                }
            memcpy(Mprod, Mtmp, sizeof(double) * (size_t)dk * dk);
        }
    }

    if (job->final_state)
        memcpy(job->final_state + sidx, S, sizeof(double) * (size_t)dk * dv);
    if (job->explicit_m && job->M)
        memcpy(job->M + ((size_t)n * H + h) * (size_t)dk * dk, Mprod,
               sizeof(double) * (size_t)dk * dk);

    free(S); free(w); free(alpha); free(Mr); free(Mprod); free(Mtmp);
    return 0;
}

static void *worker(void *arg)
{
    oracle_job *job = (oracle_job *)arg;
    const int64_t ntasks = (int64_t)job->num_seqs * job->H;
    for (;;) {
        int64_t t = take_task(job);
        if (t >= ntasks)
            break;
        if (run_task(job, t) != 0) {
            pthread_mutex_lock(&job->lock);
            job->failed = 1;
            pthread_mutex_unlock(&job->lock);
        }
    }
    return NULL;
}

static int run_job(oracle_job *job, int32_t nthreads)
{
    const int64_t ntasks = (int64_t)job->num_seqs * job->H;
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int32_t)n : 1;
    }
    if (nthreads > ntasks)
        nthreads = ntasks > 0 ? (int32_t)ntasks : 1;
    job->next_task = 0;
    job->failed = 0;
    pthread_mutex_init(&job->lock, NULL);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th)
        return -1;
    int32_t started = 0;
    for (int32_t i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, job) != 0)
            break;
        ++started;
    }
    worker(job);
    for (int32_t i = 1; i <= started; ++i)
        pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&job->lock);
    return job->failed ? -1 : 0;
}

static int check_cu(int32_t num_seqs, const int64_t *cu)
{
    if (num_seqs < 0 || !cu || cu[0] != 0)
        return -1;
    for (int32_t n = 0; n < num_seqs; ++n)
        if (cu[n + 1] < cu[n])
            return -1;
    return 0;
}

/* Returns the number of threads it would use (for reporting). */
int32_t kda_oracle_threads(int32_t nthreads)
{
    if (nthreads > 0)
        return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int32_t)n : 1;
}

/*
 * Per-token recurrence over packed sequences.  q and o may be NULL together
 * (no outputs), init may be NULL (zero state), final_state may be NULL.
 * b_write may be NULL, meaning b_write = b_erase (true KDA).
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int32_t kda_oracle_recurrence(int32_t num_seqs, const int64_t *cu, int32_t H, int32_t dk,
                              int32_t dv, const double *q, const double *k, const double *v,
                              const double *g, const double *b_erase, const double *b_write,
                              const double *init, double *o, double *final_state,
                              int32_t nthreads)
{
    if (check_cu(num_seqs, cu) || H < 1 || dk < 1 || dv < 1 || !k || !v || !g || !b_erase)
        return -1;
    oracle_job job;
    memset(&job, 0, sizeof(job));
    job.num_seqs = num_seqs; job.cu = cu; job.H = H; job.dk = dk; job.dv = dv;
    job.q = q; job.k = k; job.v = v; job.g = g;
    job.b_erase = b_erase; job.b_write = b_write ? b_write : b_erase;
    job.init = init; job.o = o; job.final_state = final_state;
    return run_job(&job, nthreads);
}

/*
 * Segment transition pair (M, S~) for packed segments: M = M_T ... M_1 by
 * explicit dk x dk products, S~ = the state after the segment from S = 0.
 * Either output may be NULL.
 */
int32_t kda_oracle_segment(int32_t num_segs, const int64_t *cu, int32_t H, int32_t dk,
                           int32_t dv, const double *k, const double *v, const double *g,
                           const double *beta, double *M, double *S_tilde, int32_t nthreads)
{
    if (check_cu(num_segs, cu) || H < 1 || dk < 1 || dv < 1 || !k || !v || !g || !beta)
        return -1;
    oracle_job job;
    memset(&job, 0, sizeof(job));
    job.num_seqs = num_segs; job.cu = cu; job.H = H; job.dk = dk; job.dv = dv;
    job.q = NULL; job.k = k; job.v = v; job.g = g;
    job.b_erase = beta; job.b_write = beta;
    job.init = NULL; job.o = NULL; job.final_state = S_tilde;
    job.M = M; job.explicit_m = M ? 1 : 0;
    return run_job(&job, nthreads);
}
