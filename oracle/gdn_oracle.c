/*
 * gdn_oracle.c -- plain, slow fp64 CPU oracle for GDN tree verification.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (Trees from Marginals, technical summary, Methodology,
 * "3. Rollback-Free Tree Verification for GDN"):
 *
 *   The Gated DeltaNet state update of that section, written there as
 *   S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T with S of
 *   shape d_k x d_v, is used here in its transposed orientation (S is
 *   d_v x d_k and maps a key to a value):
 *
 *       S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *       o_t = S_t q_t,          alpha_t = exp(g_t).
 *
 *   Tree verification gives every node i the output the recurrence produces
 *   when it is run from the prefix state S0 along the root-to-i path of the
 *   proposal tree (nodes sorted topologically, parent[i] < i, -1 = child of
 *   the prefix state).  The output is taken after node i's own update.
 *
 *   Commit (same section, the delayed state commitment): the state that the
 *   recurrence reaches at the accepted node, i.e. after running the path
 *   root..a; accepted = -1 leaves S0 unchanged.
 *
 * The oracle does exactly that: a sequential replay in fp64, no blocking, no
 * reordering, no BLAS.  The memoised form (S_i = step(S_parent(i), i)) runs
 * the identical sequence of step() calls on identical operands, so it is
 * bit-identical to the per-path replay; the tests assert this.
 *
 * Indexing (row-major):
 *   q, k [B][N][Hk][dk]   v [B][N][Hv][dv]   g, beta [B][N][Hv]
 *   parent [B][N]          S0, S_new [B][Hv][dv][dk]   o [B][N][Hv][dv]
 * Value head h reads key head h / (Hv / Hk) (consecutive grouping).
 *
 * Return codes: 0 ok, -1 bad dims, -2 invalid tree (parent[i] outside
 * [-1, i-1]), -3 invalid accepted node, -4 out of memory.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int B, N, Hk, Hv, dk, dv;
} od_dims;

/* One step of the recurrence on S (dv x dk):
 *   Sk = S k;  S <- a * (S - bt * Sk k^T) + bt * v k^T                      */
static void gdn_step(double *S, int dv, int dk, double a, double bt,
                     const double *k, const double *v, double *Sk)
{
    for (int c = 0; c < dv; ++c) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(size_t)c * dk + j] * k[j];
        Sk[c] = acc;
    }
    for (int c = 0; c < dv; ++c) {
        for (int j = 0; j < dk; ++j) {
            double s = S[(size_t)c * dk + j];
            S[(size_t)c * dk + j] = a * (s - bt * Sk[c] * k[j]) + bt * v[c] * k[j];
        }
    }
}

/* o = S q */
static void gdn_readout(const double *S, int dv, int dk, const double *q, double *o)
{
    for (int c = 0; c < dv; ++c) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(size_t)c * dk + j] * q[j];
        o[c] = acc;
    }
}

static int check_dims(const od_dims *d)
{
    if (d->B < 0 || d->N < 0 || d->Hk <= 0 || d->Hv <= 0 || d->dk <= 0 || d->dv <= 0) return -1;
    if (d->Hv % d->Hk != 0) return -1;
    return 0;
}

/* parent[i] must lie in [-1, i-1] for every node. */
int oracle_check_tree(int B, int N, const int32_t *parent)
{
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < N; ++i) {
            int p = parent[(size_t)b * N + i];
            if (p < -1 || p >= i) return -2;
        }
    return 0;
}

/* Ancestor sets as bit rows (inclusive: bit i of row i is set) and depth
 * (number of nodes on the root..i path, root depth 1).  A node's ancestors
 * are found by following parent links until -1. */
int oracle_ancestors(int B, int N, const int32_t *parent, uint32_t *anc, int32_t *depth)
{
    if (B < 0 || N < 0) return -1;
    int rc = oracle_check_tree(B, N, parent);
    if (rc) return rc;
    int W = (N + 31) / 32;
    memset(anc, 0, sizeof(uint32_t) * (size_t)B * N * (W ? W : 1));
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < N; ++i) {
            uint32_t *row = anc + ((size_t)b * N + i) * W;
            int d = 0;
            for (int s = i; s >= 0; s = parent[(size_t)b * N + s]) {
                row[s / 32] |= 1u << (s % 32);
                ++d;
            }
            depth[(size_t)b * N + i] = d;
        }
    return 0;
}

/* root..i path of node i into path[], returns its length */
static int path_of(const int32_t *par, int i, int *path)
{
    int len = 0;
    for (int s = i; s >= 0; s = par[s]) path[len++] = s;
    for (int l = 0, r = len - 1; l < r; ++l, --r) {
        int t = path[l]; path[l] = path[r]; path[r] = t;
    }
    return len;
}

typedef struct {
    const od_dims *d;
    const double *q, *k, *v, *g, *beta, *S0;
    const int32_t *parent, *accepted;
    double *out;          /* o (verify) or S_new (commit) */
    int memo;
    int mode;             /* 0 verify, 1 commit */
    int next;             /* shared work counter */
    pthread_mutex_t lock;
    int err;
} job_t;

static const double *kvec(const job_t *J, int b, int i, int kh)
{
    const od_dims *d = J->d;
    return J->k + (((size_t)b * d->N + i) * d->Hk + kh) * d->dk;
}
static const double *qvec(const job_t *J, int b, int i, int kh)
{
    const od_dims *d = J->d;
    return J->q + (((size_t)b * d->N + i) * d->Hk + kh) * d->dk;
}
static const double *vvec(const job_t *J, int b, int i, int h)
{
    const od_dims *d = J->d;
    return J->v + (((size_t)b * d->N + i) * d->Hv + h) * d->dv;
}
static double gval(const job_t *J, const double *arr, int b, int i, int h)
{
    return arr[((size_t)b * J->d->N + i) * J->d->Hv + h];
}

/* apply node j's update to S */
static void step_node(const job_t *J, double *S, int b, int j, int h, int kh, double *Sk)
{
    const od_dims *d = J->d;
    gdn_step(S, d->dv, d->dk, exp(gval(J, J->g, b, j, h)), gval(J, J->beta, b, j, h),
             kvec(J, b, j, kh), vvec(J, b, j, h), Sk);
}

static int run_unit(job_t *J, int unit)
{
    const od_dims *d = J->d;
    int b = unit / d->Hv, h = unit % d->Hv;
    int kh = h / (d->Hv / d->Hk);
    size_t ss = (size_t)d->dv * d->dk;
    const double *S0 = J->S0 + ((size_t)b * d->Hv + h) * ss;
    const int32_t *par = J->parent + (size_t)b * d->N;
    double *Sk = malloc(sizeof(double) * d->dv);
    int *path = malloc(sizeof(int) * (d->N ? d->N : 1));
    if (!Sk || !path) { free(Sk); free(path); return -4; }
    int rc = 0;

    if (J->mode == 1) {                       /* commit */
        int a = J->accepted[b];
        double *Snew = J->out + ((size_t)b * d->Hv + h) * ss;
        double *S = malloc(sizeof(double) * ss);
        if (!S) { rc = -4; goto done; }
        memcpy(S, S0, sizeof(double) * ss);
        if (a >= 0) {
            int len = path_of(par, a, path);
            for (int t = 0; t < len; ++t) step_node(J, S, b, path[t], h, kh, Sk);
        }
        memcpy(Snew, S, sizeof(double) * ss);
        free(S);
        goto done;
    }

    if (J->memo) {                           /* S_i = step(S_parent(i)) */
        double *Sall = malloc(sizeof(double) * ss * (d->N ? d->N : 1));
        if (!Sall) { rc = -4; goto done; }
        for (int i = 0; i < d->N; ++i) {
            double *Si = Sall + (size_t)i * ss;
            const double *Sp = par[i] < 0 ? S0 : Sall + (size_t)par[i] * ss;
            memcpy(Si, Sp, sizeof(double) * ss);
            step_node(J, Si, b, i, h, kh, Sk);
            double *o = J->out + (((size_t)b * d->N + i) * d->Hv + h) * d->dv;
            gdn_readout(Si, d->dv, d->dk, qvec(J, b, i, kh), o);
        }
        free(Sall);
    } else {                                 /* per-path replay from S0 */
        double *S = malloc(sizeof(double) * ss);
        if (!S) { rc = -4; goto done; }
        for (int i = 0; i < d->N; ++i) {
            memcpy(S, S0, sizeof(double) * ss);
            int len = path_of(par, i, path);
            for (int t = 0; t < len; ++t) step_node(J, S, b, path[t], h, kh, Sk);
            double *o = J->out + (((size_t)b * d->N + i) * d->Hv + h) * d->dv;
            gdn_readout(S, d->dv, d->dk, qvec(J, b, i, kh), o);
        }
        free(S);
    }
done:
    free(Sk);
    free(path);
    return rc;
}

static void *worker(void *arg)
{
    job_t *J = arg;
    int units = J->d->B * J->d->Hv;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int u = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (u >= units) break;
        int rc = run_unit(J, u);
        if (rc) {
            pthread_mutex_lock(&J->lock);
            J->err = rc;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

static int run_job(job_t *J, int nthreads)
{
    int units = J->d->B * J->d->Hv;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > units) nthreads = units ? units : 1;
    pthread_mutex_init(&J->lock, NULL);
    J->next = 0;
    J->err = 0;
    pthread_t *th = malloc(sizeof(pthread_t) * nthreads);
    if (!th) return -4;
    int started = 0;
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, worker, J) == 0) ++started; else break;
    worker(J);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    free(th);
    pthread_mutex_destroy(&J->lock);
    return J->err;
}

/* o[B][N][Hv][dv] = outputs of every tree node; memo selects the memoised
 * form (bit-identical to the replay). */
int oracle_verify(int B, int N, int Hk, int Hv, int dk, int dv,
                  const double *q, const double *k, const double *v,
                  const double *g, const double *beta, const int32_t *parent,
                  const double *S0, double *o, int memo, int nthreads)
{
    od_dims d = {B, N, Hk, Hv, dk, dv};
    if (check_dims(&d)) return -1;
    int rc = oracle_check_tree(B, N, parent);
    if (rc) return rc;
    job_t J = {0};
    J.d = &d; J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.S0 = S0;
    J.parent = parent; J.out = o; J.memo = memo; J.mode = 0;
    return run_job(&J, nthreads);
}

/* S_new[B][Hv][dv][dk] = state at accepted[b] (S0 when accepted[b] == -1) */
int oracle_commit(int B, int N, int Hk, int Hv, int dk, int dv,
                  const double *k, const double *v, const double *g, const double *beta,
                  const int32_t *parent, const double *S0, const int32_t *accepted,
                  double *S_new, int nthreads)
{
    od_dims d = {B, N, Hk, Hv, dk, dv};
    if (check_dims(&d)) return -1;
    int rc = oracle_check_tree(B, N, parent);
    if (rc) return rc;
    for (int b = 0; b < B; ++b)
        if (accepted[b] < -1 || accepted[b] >= N) return -3;
    job_t J = {0};
    J.d = &d; J.k = k; J.v = v; J.g = g; J.beta = beta; J.S0 = S0;
    J.parent = parent; J.accepted = accepted; J.out = S_new; J.mode = 1;
    return run_job(&J, nthreads);
}
