// Prints the plan (query rows per workgroup, effective splits) the host half
// of the C ABI picks for each shape given on the command line as B,M,N,D, at
// the chip size the stubbed device query reports (MGA_TEST_CUS).
#include <stdio.h>

#include "../../include/mga_gqa.h"

int main(int argc, char **argv) {
    for (int i = 1; i < argc; ++i) {
        int B, M, N, D;
        if (sscanf(argv[i], "%d,%d,%d,%d", &B, &M, &N, &D) != 4) return 2;
        int rows = 0, splits = 0;
        const int rc = mga_gqa_plan(B, M, N, D, 0, &rows, &splits);
        printf("%d %d %d %d %d %d %d\n", B, M, N, D, rc, rows, splits);
    }
    return 0;
}
