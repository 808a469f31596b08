// Drives the host half of the C ABI over a grid of shapes, splits and strides,
// extreme values included, so that AddressSanitizer and UndefinedBehavior-
// Sanitizer see every branch of the argument checks, the split policy, the
// workspace arithmetic and the stride validation. Prints one line per check
// family and the number of calls; exits non-zero on an inconsistency.
#include <stdint.h>
#include <stdio.h>

#include <climits>
#include <vector>

#include "../../include/mga_gqa.h"

static int fails = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++fails;                                                    \
        }                                                               \
    } while (0)

int main() {
    const void *A = (const void *)(uintptr_t)(1 << 20);
    const std::vector<int> Bs = {-1, 0, 1, 2, 16, 128, 65535, 65536, 1 << 20, INT_MAX};
    const std::vector<int> Ms = {-1, 0, 1, 8, 32, 33, 256, 300, 1 << 20, INT_MAX};
    const std::vector<int> Ns = {-5, 0, 1, 3, 8, 1001, 4096, (1 << 23) - 8, (1 << 24) - 8, 1 << 24, INT_MAX};
    const std::vector<int> Ds = {0, 32, 64, 96, 128, 256, -64};
    const std::vector<int> Ss = {-1, 0, 1, 2, 7, 32, INT_MAX};
    long calls = 0;
    for (int B : Bs)
        for (int M : Ms)
            for (int N : Ns)
                for (int D : Ds)
                    for (int s : Ss) {
                        const size_t ws = mga_gqa_workspace_bytes(B, M, N, D, s);
                        const int eff = mga_gqa_effective_splits(B, M, N, D, s);
                        int rows = -1, eff2 = -1;
                        const int rc = mga_gqa_plan(B, M, N, D, s, &rows, &eff2);
                        const int chk = mga_gqa_check_args(A, A, A, A, B, M, N, D, s, A, ws);
                        (void)mga_gqa_choose_splits(B, M, N, D);
                        (void)mga_gqa_qknorm_workspace_bytes(B, M, N, D, s);
                        (void)mga_gqa_qknorm_check_args(A, A, A, A, B, M, N, D, 1e-6f, nullptr, s, A, ws);
                        calls += 7;
                        if (rc == MGA_OK) {
                            CHECK(eff == eff2 && eff >= 1);
                            CHECK(rows == 32 || rows == 64 || rows == 128 || rows == 256);
                        } else {
                            CHECK(eff == -1);
                        }
                        if (chk == MGA_OK && B > 0 && M > 0) CHECK(rc == MGA_OK);
                    }
    printf("shapes: %ld calls\n", calls);

    // Strides: every field at extreme values on two shapes.
    const std::vector<long long> vals = {-8, -1, 0, 1, 7, 8, 64, 128, 4096, 1LL << 30, (1LL << 30) + 8,
                                         1LL << 48, (1LL << 48) + 8, LLONG_MAX / 2, LLONG_MAX};
    long scalls = 0;
    for (int shape = 0; shape < 2; ++shape) {
        const int B = shape ? 3 : 2, M = shape ? 40 : 256, N = shape ? 1001 : 4096, D = shape ? 128 : 64;
        const int64_t base[9] = {(int64_t)M * D, D, (int64_t)D * N, N, 1, (int64_t)N * D, D, (int64_t)M * D, D};
        for (int f = 0; f < 9; ++f)
            for (long long v : vals) {
                int64_t st[9];
                for (int i = 0; i < 9; ++i) st[i] = base[i];
                st[f] = v;
                const int r1 = mga_gqa_check_args_strided(A, A, A, A, B, M, N, D, st, 1, A, 1u << 30);
                const int r2 = mga_gqa_qknorm_check_args(A, A, A, A, B, M, N, D, 1e-6f, st, 1, A, 1u << 30);
                CHECK(r1 == r2 || r2 == MGA_OK || r1 == MGA_OK);
                scalls += 2;
            }
    }
    printf("strides: %ld calls\n", scalls);
    for (int code = -1; code < 8; ++code) CHECK(mga_status_string(code) != nullptr);
    printf("fails: %d\n", fails);
    return fails ? 1 : 0;
}
