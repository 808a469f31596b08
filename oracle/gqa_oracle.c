/*
 * Plain fp64 CPU oracle for the GQA exp-sum-div graph.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * bench's CPU-baseline leg load this library. The product path never calls
 * it and shares no code with it.
 *
 * What it computes: the kernel graph of the Mirage GQA tutorial page
 * ("Mirage: Define GQA Computation Graph"; the same five operations appear
 * under "Python Superoptimization Example" and in section 1 of the kaispace
 * blog), evaluated in double precision on the exact values of the inputs:
 *
 *   A = matmul(Q, K)        A[b,i,n] = sum_d Q[b,i,d] * K[b,d,n]
 *   E = exp(A)              elementwise
 *   S = reduction(E, 2)     S[b,i]   = sum_n E[b,i,n]   (axis 2 = keys, kept)
 *   D = div(E, S)           D[b,i,n] = E[b,i,n] / S[b,i] (S broadcast)
 *   O = matmul(D, V)        O[b,i,j] = sum_n D[b,i,n] * V[b,n,j]
 *
 * There is no 1/sqrt(d) scale and no max subtraction, because the graph has
 * none. Steps run in the graph's order: the division comes before the second
 * matmul. Rows (b, i) are independent; OpenMP spreads them over threads and
 * nothing else is reordered. Each row keeps its scores in a scratch vector of
 * length N.
 *
 * Layouts (row-major, contiguous, as the graph's inputs are declared):
 *   q [B][M][Dh], k [B][Dh][N] (head-dim-major), v [B][N][Dh], o [B][M][Dh].
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Thread count for later calls (n >= 1); used to time the oracle on one
 * core. Changes no arithmetic: each output row is computed by one thread in
 * the same order whatever the count. */
void mga_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int mga_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One query row: o_row[j] = sum_n (exp(a_n) / sum_m exp(a_m)) * v[n][j]. */
static void oracle_row(const double *q_row, const double *k_b, const double *v_b,
                       double *o_row, long N, long Dh, double *a)
{
    /* A = matmul(Q, K): d outer, n inner, so K is walked along its rows. */
    for (long n = 0; n < N; ++n)
        a[n] = 0.0;
    for (long d = 0; d < Dh; ++d) {
        const double qd = q_row[d];
        const double *k_row = k_b + d * N;
        for (long n = 0; n < N; ++n)
            a[n] += qd * k_row[n];
    }
    /* E = exp(A), in place. */
    for (long n = 0; n < N; ++n)
        a[n] = exp(a[n]);
    /* S = reduction(E, 2): plain running sum over the keys. */
    double s = 0.0;
    for (long n = 0; n < N; ++n)
        s += a[n];
    /* D = div(E, S), in place. */
    for (long n = 0; n < N; ++n)
        a[n] = a[n] / s;
    /* O = matmul(D, V). */
    for (long j = 0; j < Dh; ++j)
        o_row[j] = 0.0;
    for (long n = 0; n < N; ++n) {
        const double w = a[n];
        const double *v_row = v_b + n * Dh;
        for (long j = 0; j < Dh; ++j)
            o_row[j] += w * v_row[j];
    }
}

/*
 * Full graph over all B*M rows. Returns 0 on success, -1 on a bad argument
 * (N < 1 makes S an empty sum and D = 0/0, which the graph leaves undefined),
 * -2 if the scratch allocation fails.
 */
int mga_oracle_gqa_f64(const double *q, const double *k, const double *v, double *o,
                       long B, long M, long N, long Dh)
{
    if (B < 0 || M < 0 || N < 1 || Dh < 1 || !q || !k || !v || !o)
        return -1;
    int failed = 0;
#pragma omp parallel
    {
        double *a = (double *)malloc(sizeof(double) * (size_t)N);
        if (!a) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (long r = 0; r < B * M; ++r) {
            if (!a)
                continue;
            const long b = r / M;
            oracle_row(q + r * Dh, k + b * Dh * N, v + b * N * Dh, o + r * Dh, N, Dh, a);
        }
        free(a);
    }
    return failed ? -2 : 0;
}
