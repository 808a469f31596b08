/* Runs the C oracle on a few small shapes (and the empty-key rejection) so
 * that AddressSanitizer and UndefinedBehaviorSanitizer see its loops. The
 * values are checked elsewhere; this only looks for memory and UB errors. */
#include <stdio.h>
#include <stdlib.h>

int mga_oracle_gqa_f64(const double *q, const double *k, const double *v, double *o, long B, long M,
                       long N, long Dh);

int main(void) {
    const long shapes[][4] = {{1, 1, 1, 4}, {2, 3, 5, 8}, {1, 7, 33, 64}, {3, 2, 130, 128}, {1, 0, 4, 8}};
    int bad = 0;
    for (unsigned s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
        const long B = shapes[s][0], M = shapes[s][1], N = shapes[s][2], D = shapes[s][3];
        double *q = malloc(sizeof(double) * (B * M * D + 1)), *k = malloc(sizeof(double) * B * D * N);
        double *v = malloc(sizeof(double) * B * N * D), *o = malloc(sizeof(double) * (B * M * D + 1));
        for (long i = 0; i < B * M * D; ++i) q[i] = 0.01 * (double)(i % 17) - 0.08;
        for (long i = 0; i < B * D * N; ++i) k[i] = 0.02 * (double)(i % 13) - 0.12;
        for (long i = 0; i < B * N * D; ++i) v[i] = (double)(i % 7) - 3.0;
        if (mga_oracle_gqa_f64(q, k, v, o, B, M, N, D) != 0) ++bad;
        free(q), free(k), free(v), free(o);
    }
    double one = 0.0;
    if (mga_oracle_gqa_f64(&one, &one, &one, &one, 1, 1, 0, 1) == 0) ++bad;  /* N = 0 must be rejected */
    printf("oracle shapes run, bad=%d\n", bad);
    return bad;
}
