/*
 * kda_oracle.c -- plain fp64 CPU oracle of the KDA gated delta-rule core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the bench's CPU-baseline leg
 * do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (the pages do not print the recurrence; this is the plainest
 * reading of what they do print):
 *
 *   Per sequence b and head h the core carries an FP32 state S of shape
 *   [head_dim (key i), head_dim (value j)], the "K-major [heads, head_dim,
 *   head_dim]" recurrent state of the config page (config.rs,
 *   Glm5NextKdaConfig::recurrent_state_elems).  Each token t brings q_t, k_t
 *   (L2-normalised upstream), a raw v_t, a per-channel log-decay gate_t
 *   (workspace page, field "gate": bounded log-decay) and a scalar beta_t that
 *   has already been through a sigmoid (workspace page, field "beta").
 *
 *   Gated delta rule, decay before the delta correction (kernel-table page,
 *   field recurrent_smem: the decayed state column is what the two state
 *   passes share):
 *       alpha_i  = exp(gate_{t,i})                       per key channel i
 *       S_ij    <- alpha_i * S_ij                         decay
 *       u_j      = sum_i k_{t,i} S_ij                     read-out with the key
 *       delta_j  = beta_t * (v_{t,j} - u_j)               delta-rule error
 *       S_ij    <- S_ij + k_{t,i} delta_j                 rank-1 correction
 *       out_{t,j}= sum_i q_{t,i} S_ij                     post-update state, scale 1
 *   i.e. S_t = (I - beta k k^T) diag(e^g) S_{t-1} + beta k v^T,  o_t = S_t^T q_t.
 *
 *   The chunked form (kernel-table page, fields chunk_prepare / chunk_scan;
 *   layer page, prefill) is the same map computed C rows at a time.  With S0
 *   the state entering a chunk and G_r = sum_{m<=r} g_m (per channel):
 *       A_rs = beta_r sum_i k_ri k_si e^{G_ri - G_si}   (s < r),  T = (I + A)^-1
 *       W = T diag(beta) (e^G o K),   U = T diag(beta) V,   Delta = U - W S0
 *       M_rs = sum_i q_ri k_si e^{G_ri - G_si}           (s <= r)
 *       O = (e^G o Q) S0 + M Delta
 *       S_C = diag(e^{G_last}) S0 + (e^{G_last - G} o K)^T Delta
 *   obtained by unrolling the serial map over the chunk and collecting the
 *   delta_r terms (the delta of row r depends on the earlier deltas of the
 *   chunk only through A).  Every pairwise decay e^{G_ri - G_si} is taken as
 *   one exp of an fp64 difference, so no factor here can overflow.
 *
 * Layouts (token-major, heads inside; row_stride rows per sequence):
 *   q, k, v, gate : float  [B][row_stride][H][D]
 *   beta          : float  [B][row_stride][H]
 *   state         : double [B][H][D][D]            read and updated in place
 *   out           : double [B][T][H][D]            rows t < T
 *   snaps         : double [n_snap][B][H][D][D]    state after row t, t < n_snap
 * All arithmetic is IEEE double; inputs are widened from float on read.
 * Work is split over (b, h) units with POSIX threads; each unit is computed by
 * one thread in a fixed order, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const float *q, *k, *v, *gate, *beta;
    double *state, *out, *snaps;
    int n_snap, B, H, D, T, row_stride, chunk;
    /* work distribution */
    int n_units, n_threads;
    int thread_id;
    int status;
} oracle_job;

static size_t vec_index(const oracle_job* j, int b, int t, int h)
{
    return (((size_t)b * j->row_stride + t) * j->H + h) * (size_t)j->D;
}

static size_t beta_index(const oracle_job* j, int b, int t, int h)
{
    return ((size_t)b * j->row_stride + t) * j->H + h;
}

/* ---- serial (token by token) form -------------------------------------- */

static void serial_unit(const oracle_job* j, int b, int h, double* work)
{
    const int D = j->D;
    double* S = j->state + ((size_t)b * j->H + h) * (size_t)D * D;
    double* alpha = work;          /* [D] */
    double* u = work + D;          /* [D] */
    double* delta = work + 2 * D;  /* [D] */
    for (int t = 0; t < j->T; ++t) {
        const float* qt = j->q + vec_index(j, b, t, h);
        const float* kt = j->k + vec_index(j, b, t, h);
        const float* vt = j->v + vec_index(j, b, t, h);
        const float* gt = j->gate + vec_index(j, b, t, h);
        const double bt = (double)j->beta[beta_index(j, b, t, h)];
        for (int i = 0; i < D; ++i) alpha[i] = exp((double)gt[i]);
        for (int i = 0; i < D; ++i)
            for (int c = 0; c < D; ++c) S[(size_t)i * D + c] *= alpha[i];
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int i = 0; i < D; ++i) acc += (double)kt[i] * S[(size_t)i * D + c];
            u[c] = acc;
        }
        for (int c = 0; c < D; ++c) delta[c] = bt * ((double)vt[c] - u[c]);
        for (int i = 0; i < D; ++i)
            for (int c = 0; c < D; ++c) S[(size_t)i * D + c] += (double)kt[i] * delta[c];
        double* ot = j->out + (((size_t)b * j->T + t) * j->H + h) * (size_t)D;
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int i = 0; i < D; ++i) acc += (double)qt[i] * S[(size_t)i * D + c];
            ot[c] = acc;
        }
        if (t < j->n_snap) {
            double* dst = j->snaps + (((size_t)t * j->B + b) * j->H + h) * (size_t)D * D;
            memcpy(dst, S, sizeof(double) * (size_t)D * D);
        }
    }
}

/* ---- chunked (WY / UT) form ------------------------------------------- */

/* Optional per-chunk intermediates, each row-major with n = rows in chunk. */
typedef struct {
    double *G;      /* [n][D]  cumulative log-decay                   */
    double *A;      /* [n][n]  strictly lower, row-scaled by beta     */
    double *Tinv;   /* [n][n]  (I + A)^-1                              */
    double *W;      /* [n][D]                                          */
    double *U;      /* [n][D]                                          */
    double *M;      /* [n][n]  lower incl. diagonal                    */
    double *Delta;  /* [n][D]                                          */
} chunk_stages;

/* One chunk of n rows starting at token t0 of (b, h); S is the incoming
 * state [D][D], replaced by the outgoing one; O [n][D] receives the outputs.
 * scratch must hold 5*n*D + 3*n*n + 2*n doubles. */
static void chunk_unit(const oracle_job* j, int b, int h, int t0, int n, double* S, double* O,
                       double* scratch, chunk_stages* st)
{
    const int D = j->D;
    double* G = scratch;                 /* n*D  cumulative log-decay        */
    double* Gm = G + (size_t)n * D;      /* n*D  e^{G}                        */
    double* W = Gm + (size_t)n * D;      /* n*D                               */
    double* U = W + (size_t)n * D;       /* n*D                               */
    double* Dl = U + (size_t)n * D;      /* n*D  Delta                        */
    double* A = Dl + (size_t)n * D;      /* n*n                               */
    double* Ti = A + (size_t)n * n;      /* n*n                               */
    double* M = Ti + (size_t)n * n;      /* n*n                               */
    double* bet = M + (size_t)n * n;     /* n                                 */
    double* kt = bet + n;                /* n    one column of e^{G_last-G} k */

    for (int r = 0; r < n; ++r) bet[r] = (double)j->beta[beta_index(j, b, t0 + r, h)];

    /* G_r = sum_{m <= r} g_m per channel, and e^{G_r} */
    for (int i = 0; i < D; ++i) {
        double acc = 0.0;
        for (int r = 0; r < n; ++r) {
            acc += (double)j->gate[vec_index(j, b, t0 + r, h) + i];
            G[(size_t)r * D + i] = acc;
            Gm[(size_t)r * D + i] = exp(acc);
        }
    }
#define KV(arr, r, i) ((double)(arr)[vec_index(j, b, t0 + (r), h) + (i)])
    /* A (strictly lower) and M (lower with diagonal) */
    for (int r = 0; r < n; ++r) {
        for (int s = 0; s < n; ++s) {
            double a = 0.0, m = 0.0;
            if (s <= r) {
                for (int i = 0; i < D; ++i) {
                    const double e = exp(G[(size_t)r * D + i] - G[(size_t)s * D + i]);
                    a += KV(j->k, r, i) * KV(j->k, s, i) * e;
                    m += KV(j->q, r, i) * KV(j->k, s, i) * e;
                }
            }
            A[(size_t)r * n + s] = (s < r) ? bet[r] * a : 0.0;
            M[(size_t)r * n + s] = (s <= r) ? m : 0.0;
        }
    }
    /* T = (I + A)^-1 by forward substitution, one column at a time */
    for (int c = 0; c < n; ++c) {
        for (int r = 0; r < n; ++r) {
            double x = (r == c) ? 1.0 : 0.0;
            for (int m = 0; m < r; ++m) x -= A[(size_t)r * n + m] * Ti[(size_t)m * n + c];
            Ti[(size_t)r * n + c] = x;
        }
    }
    /* W = T diag(beta) (e^G o K),  U = T diag(beta) V */
    for (int r = 0; r < n; ++r) {
        for (int i = 0; i < D; ++i) {
            double w = 0.0, u = 0.0;
            for (int s = 0; s < n; ++s) {
                const double t = Ti[(size_t)r * n + s];
                w += t * bet[s] * Gm[(size_t)s * D + i] * KV(j->k, s, i);
                u += t * bet[s] * KV(j->v, s, i);
            }
            W[(size_t)r * D + i] = w;
            U[(size_t)r * D + i] = u;
        }
    }
    /* Delta = U - W S0 */
    for (int r = 0; r < n; ++r)
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int i = 0; i < D; ++i) acc += W[(size_t)r * D + i] * S[(size_t)i * D + c];
            Dl[(size_t)r * D + c] = U[(size_t)r * D + c] - acc;
        }
    /* O = (e^G o Q) S0 + M Delta */
    for (int r = 0; r < n; ++r)
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int i = 0; i < D; ++i) acc += Gm[(size_t)r * D + i] * KV(j->q, r, i) * S[(size_t)i * D + c];
            for (int s = 0; s < n; ++s) acc += M[(size_t)r * n + s] * Dl[(size_t)s * D + c];
            O[(size_t)r * D + c] = acc;
        }
    /* S_C = diag(e^{G_last}) S0 + (e^{G_last - G} o K)^T Delta */
    for (int i = 0; i < D; ++i) {
        const double gl = G[(size_t)(n - 1) * D + i];
        const double decay = exp(gl);
        for (int s = 0; s < n; ++s) kt[s] = exp(gl - G[(size_t)s * D + i]) * KV(j->k, s, i);
        for (int c = 0; c < D; ++c) {
            double acc = decay * S[(size_t)i * D + c];
            for (int s = 0; s < n; ++s) acc += kt[s] * Dl[(size_t)s * D + c];
            S[(size_t)i * D + c] = acc;
        }
    }
#undef KV
    if (st) {
        if (st->G) memcpy(st->G, G, sizeof(double) * (size_t)n * D);
        if (st->A) memcpy(st->A, A, sizeof(double) * (size_t)n * n);
        if (st->Tinv) memcpy(st->Tinv, Ti, sizeof(double) * (size_t)n * n);
        if (st->W) memcpy(st->W, W, sizeof(double) * (size_t)n * D);
        if (st->U) memcpy(st->U, U, sizeof(double) * (size_t)n * D);
        if (st->M) memcpy(st->M, M, sizeof(double) * (size_t)n * n);
        if (st->Delta) memcpy(st->Delta, Dl, sizeof(double) * (size_t)n * D);
    }
}

static size_t chunk_scratch_doubles(int n, int D)
{
    return 5 * (size_t)n * D + 3 * (size_t)n * n + 2 * (size_t)n;
}

static void chunked_unit(const oracle_job* j, int b, int h, double* scratch, double* O)
{
    const int D = j->D;
    double* S = j->state + ((size_t)b * j->H + h) * (size_t)D * D;
    for (int t0 = 0; t0 < j->T; t0 += j->chunk) {
        const int n = (j->T - t0 < j->chunk) ? j->T - t0 : j->chunk;
        chunk_unit(j, b, h, t0, n, S, O, scratch, NULL);
        for (int r = 0; r < n; ++r)
            memcpy(j->out + (((size_t)b * j->T + t0 + r) * j->H + h) * (size_t)D, O + (size_t)r * D,
                   sizeof(double) * (size_t)D);
    }
}

/* ---- threading --------------------------------------------------------- */

static void* worker(void* arg)
{
    oracle_job* j = (oracle_job*)arg;
    const int D = j->D;
    double* work = NULL;
    double* O = NULL;
    if (j->chunk > 0) {
        work = (double*)malloc(sizeof(double) * chunk_scratch_doubles(j->chunk, D));
        O = (double*)malloc(sizeof(double) * (size_t)j->chunk * D);
    } else {
        work = (double*)malloc(sizeof(double) * 3 * (size_t)D);
    }
    if (!work || (j->chunk > 0 && !O)) {
        free(work);
        free(O);
        j->status = -1;
        return NULL;
    }
    for (int u = j->thread_id; u < j->n_units; u += j->n_threads) {
        const int b = u / j->H, h = u % j->H;
        if (j->chunk > 0) chunked_unit(j, b, h, work, O);
        else serial_unit(j, b, h, work);
    }
    free(work);
    free(O);
    j->status = 0;
    return NULL;
}

int kda_oracle_threads(int requested)
{
    if (requested > 0) return requested;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static int run(oracle_job base, int nthreads)
{
    if (!base.q || !base.k || !base.v || !base.gate || !base.beta || !base.state || !base.out) return -1;
    if (base.B < 1 || base.H < 1 || base.D < 1 || base.T < 1 || base.row_stride < base.T) return -1;
    if (base.n_snap < 0 || base.n_snap > base.T || (base.n_snap > 0 && !base.snaps)) return -1;
    base.n_units = base.B * base.H;
    int nt = kda_oracle_threads(nthreads);
    if (nt > base.n_units) nt = base.n_units;
    oracle_job* jobs = (oracle_job*)calloc((size_t)nt, sizeof(oracle_job));
    pthread_t* tids = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -1;
    }
    int rc = nt;
    for (int i = 0; i < nt; ++i) {
        jobs[i] = base;
        jobs[i].n_threads = nt;
        jobs[i].thread_id = i;
        jobs[i].status = -1;
        if (pthread_create(&tids[i], NULL, worker, &jobs[i]) != 0) {
            /* run the rest on this thread */
            for (int r = i; r < nt; ++r) {
                jobs[r] = base;
                jobs[r].n_threads = nt;
                jobs[r].thread_id = r;
                worker(&jobs[r]);
            }
            for (int w = 0; w < i; ++w) pthread_join(tids[w], NULL);
            for (int w = 0; w < nt; ++w)
                if (jobs[w].status != 0) rc = -1;
            free(jobs);
            free(tids);
            return rc;
        }
    }
    for (int i = 0; i < nt; ++i) pthread_join(tids[i], NULL);
    for (int i = 0; i < nt; ++i)
        if (jobs[i].status != 0) rc = -1;
    free(jobs);
    free(tids);
    return rc;
}

/* Serial form.  Returns the number of threads used, or -1 on bad arguments. */
int kda_oracle_serial(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                      double* state, double* out, double* snaps, int n_snap, int B, int H, int D, int T,
                      int row_stride, int nthreads)
{
    oracle_job j;
    memset(&j, 0, sizeof j);
    j.q = q; j.k = k; j.v = v; j.gate = gate; j.beta = beta;
    j.state = state; j.out = out; j.snaps = snaps; j.n_snap = n_snap;
    j.B = B; j.H = H; j.D = D; j.T = T; j.row_stride = row_stride; j.chunk = 0;
    return run(j, nthreads);
}

/* Chunked (WY/UT) form with chunk width C.  Same layouts and return value. */
int kda_oracle_chunked(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                       double* state, double* out, int B, int H, int D, int T, int row_stride, int C,
                       int nthreads)
{
    if (C < 1) return -1;
    oracle_job j;
    memset(&j, 0, sizeof j);
    j.q = q; j.k = k; j.v = v; j.gate = gate; j.beta = beta;
    j.state = state; j.out = out; j.snaps = NULL; j.n_snap = 0;
    j.B = B; j.H = H; j.D = D; j.T = T; j.row_stride = row_stride; j.chunk = C;
    return run(j, nthreads);
}

/* Intermediates of one chunk (rows [t0, t0+n) of (b, h)) from the incoming
 * state S (double [D][D], replaced by the outgoing state); O gets [n][D].
 * Any stage pointer may be NULL.  Returns 0, or -1 on bad arguments. */
int kda_oracle_chunk_stages(const float* q, const float* k, const float* v, const float* gate,
                            const float* beta, int B, int H, int D, int row_stride, int b, int h, int t0, int n,
                            double* S, double* O, double* G, double* A, double* Tinv, double* W, double* U,
                            double* M, double* Delta)
{
    if (!q || !k || !v || !gate || !beta || !S || !O) return -1;
    if (b < 0 || b >= B || h < 0 || h >= H || n < 1 || t0 < 0 || t0 + n > row_stride || D < 1) return -1;
    oracle_job j;
    memset(&j, 0, sizeof j);
    j.q = q; j.k = k; j.v = v; j.gate = gate; j.beta = beta;
    j.B = B; j.H = H; j.D = D; j.T = t0 + n; j.row_stride = row_stride; j.chunk = n;
    double* scratch = (double*)malloc(sizeof(double) * chunk_scratch_doubles(n, D));
    if (!scratch) return -1;
    chunk_stages st = {G, A, Tinv, W, U, M, Delta};
    chunk_unit(&j, b, h, t0, n, S, O, scratch, &st);
    free(scratch);
    return 0;
}
