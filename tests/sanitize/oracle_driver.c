/* oracle_driver.c -- runs every entry point of the fp64 oracle on small
 * seeded trees (uniform, chain, forest; memoised and per-path forms; several
 * thread counts) and on invalid inputs, under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Exit status 0 when every call returns what
 * it should and the memoised and per-path outputs agree bit for bit. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_verify(int B, int N, int Hk, int Hv, int dk, int dv, const double *q, const double *k,
                  const double *v, const double *g, const double *beta, const int32_t *parent,
                  const double *S0, double *o, int memo, int nthreads);
int oracle_commit(int B, int N, int Hk, int Hv, int dk, int dv, const double *k, const double *v,
                  const double *g, const double *beta, const int32_t *parent, const double *S0,
                  const int32_t *accepted, double *S_new, int nthreads);
int oracle_ancestors(int B, int N, const int32_t *parent, uint32_t *anc, int32_t *depth);
int oracle_check_tree(int B, int N, const int32_t *parent);

static uint64_t s_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {   /* xorshift64*, in [0, 1) */
    s_state ^= s_state >> 12; s_state ^= s_state << 25; s_state ^= s_state >> 27;
    return (double)((s_state * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}
static double *darr(size_t n, double lo, double hi) {
    double *p = malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * urand();
    return p;
}

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static void one_case(int B, int N, int Hk, int Hv, int dk, int dv, int kind, int threads) {
    size_t nq = (size_t)B * N * Hk * dk, nv = (size_t)B * N * Hv * dv, ng = (size_t)B * N * Hv;
    size_t ns = (size_t)B * Hv * dv * dk;
    double *q = darr(nq, -1, 1), *k = darr(nq, -0.2, 0.2), *v = darr(nv, -1, 1);
    double *g = darr(ng, -1, 0), *be = darr(ng, 0, 1), *S0 = darr(ns, -0.05, 0.05);
    int32_t *par = malloc(sizeof(int32_t) * (B * N ? B * N : 1));
    int32_t *acc = malloc(sizeof(int32_t) * (B ? B : 1));
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < N; ++i) {
            int p = kind == 0 ? (i ? (int)(urand() * i) : -1) : i - 1;
            if (kind == 2 && urand() < 0.2) p = -1;
            par[b * N + i] = p;
        }
        acc[b] = N ? (int)(urand() * (N + 1)) - 1 : -1;
    }
    double *o1 = calloc(nv ? nv : 1, sizeof(double)), *o2 = calloc(nv ? nv : 1, sizeof(double));
    double *Sn = calloc(ns ? ns : 1, sizeof(double));
    uint32_t *anc = calloc((size_t)B * N * ((N + 31) / 32) + 1, sizeof(uint32_t));
    int32_t *dep = calloc((size_t)B * N + 1, sizeof(int32_t));
    CHECK(oracle_verify(B, N, Hk, Hv, dk, dv, q, k, v, g, be, par, S0, o1, 1, threads) == 0);
    CHECK(oracle_verify(B, N, Hk, Hv, dk, dv, q, k, v, g, be, par, S0, o2, 0, threads) == 0);
    CHECK(memcmp(o1, o2, sizeof(double) * nv) == 0);
    CHECK(oracle_commit(B, N, Hk, Hv, dk, dv, k, v, g, be, par, S0, acc, Sn, threads) == 0);
    CHECK(oracle_ancestors(B, N, par, anc, dep) == 0);
    CHECK(oracle_check_tree(B, N, par) == 0);
    if (B > 0 && N > 1) {
        int keep = par[N - 1];
        par[N - 1] = N - 1;   /* a self edge: not topological */
        CHECK(oracle_check_tree(B, N, par) == -2);
        CHECK(oracle_verify(B, N, Hk, Hv, dk, dv, q, k, v, g, be, par, S0, o1, 1, threads) == -2);
        CHECK(oracle_ancestors(B, N, par, anc, dep) == -2);
        par[N - 1] = keep;
        int ka = acc[0];
        acc[0] = N;
        CHECK(oracle_commit(B, N, Hk, Hv, dk, dv, k, v, g, be, par, S0, acc, Sn, threads) == -3);
        acc[0] = ka;
    }
    /* value heads not a multiple of key heads: rejected before any access */
    CHECK(oracle_verify(B, N, 2, 3, dk, dv, q, k, v, g, be, par, S0, o1, 1, threads) == -1);
    CHECK(oracle_commit(B, N, 0, Hv, dk, dv, k, v, g, be, par, S0, acc, Sn, threads) == -1);
    free(q); free(k); free(v); free(g); free(be); free(S0); free(par); free(acc);
    free(o1); free(o2); free(Sn); free(anc); free(dep);
}

int main(void) {
    one_case(2, 9, 1, 2, 8, 6, 0, 1);
    one_case(3, 33, 2, 4, 4, 5, 0, 3);
    one_case(1, 17, 1, 1, 3, 3, 1, 2);
    one_case(2, 40, 2, 2, 5, 4, 2, 8);
    one_case(1, 1, 1, 1, 2, 2, 0, 4);
    one_case(2, 0, 1, 1, 2, 2, 0, 2);
    one_case(0, 5, 1, 1, 2, 2, 0, 2);
    printf("oracle_driver: %d failed checks\n", fails);
    return fails == 0 ? 0 : 1;
}
