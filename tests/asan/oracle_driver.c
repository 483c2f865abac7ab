/* Host driver for the fp64 oracle (oracle/gdn_oracle.c), built with AddressSanitizer
 * and UndefinedBehaviorSanitizer by tests/test_asan_host.py.  It runs the oracle's
 * prefill and decode over cases that touch every index path -- zero-length and
 * one-token sequences, starts off the grid, exports on the grid, slots in place, slots
 * absent (-1), decode padding rows -- so that any access outside a buffer aborts, and
 * checks that every value written is finite and that a sequence ending on the grid
 * exports exactly its final state. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_prefill(int H_k, int H_v, int d_k, int d_v, int num_seqs, const int32_t* cu_seqlens,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, double scale, double* pool, int num_slots,
                   const int32_t* init_slot, const int32_t* final_slot, const int32_t* start_pos,
                   int export_grid, double* export_states, const int32_t* export_offsets,
                   double* o, double* final_states);
int oracle_decode(int H_k, int H_v, int d_k, int d_v, int num_rows, const double* q,
                  const double* k, const double* v, const double* g, const double* beta,
                  double scale, double* pool, int num_slots, const int32_t* slot_in,
                  const int32_t* slot_out, double* o);

static uint64_t lcg = 12345;
static double rnd(void) {
    lcg = lcg * 6364136223846793005ULL + 1442695040888963407ULL;
    return ((double)(lcg >> 11) / 9007199254740992.0) * 2.0 - 1.0;
}
static double* fill(size_t n, double lo, double hi) {
    double* a = (double*)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * 0.5 * (rnd() + 1.0);
    return a;
}
static int all_finite(const double* a, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

int main(void) {
    const int H_k = 2, H_v = 4, d_k = 16, d_v = 8, N = 6, S = 16;
    const int32_t len[6] = {0, 1, 63, 64, 130, 7};
    const int32_t start[6] = {5, 64, 1, 0, 1000, 57};
    const int grid = 64;
    int32_t cu[7] = {0};
    for (int i = 0; i < N; ++i) cu[i + 1] = cu[i] + len[i];
    const int T = cu[N];
    const size_t SE = (size_t)d_k * d_v;
    double* q = fill((size_t)T * H_k * d_k, -0.3, 0.3);
    double* k = fill((size_t)T * H_k * d_k, -0.3, 0.3);
    double* v = fill((size_t)T * H_v * d_v, -1.0, 1.0);
    double* g = fill((size_t)T * H_v, -1.0, 0.0);
    double* beta = fill((size_t)T * H_v, 0.0, 1.0);
    double* pool = fill((size_t)S * H_v * SE, -0.1, 0.1);
    int32_t init[6] = {3, -1, 4, 5, 6, -1};
    int32_t fin[6] = {3, 7, 8, -1, 9, 10};   /* sequence 0 resumes in place; 3 keeps no state */
    int32_t offs[7] = {0};
    for (int i = 0; i < N; ++i) offs[i + 1] = offs[i] + (start[i] + len[i]) / grid - start[i] / grid;
    const int E = offs[N];
    double* exps = (double*)calloc((size_t)(E > 0 ? E : 1) * H_v * SE, sizeof(double));
    double* o = (double*)calloc((size_t)T * H_v * d_v, sizeof(double));
    double* finals = (double*)calloc((size_t)N * H_v * SE, sizeof(double));
    int bad = 0;
    if (oracle_prefill(H_k, H_v, d_k, d_v, N, cu, q, k, v, g, beta, 0.25, pool, S, init, fin, start, grid, exps,
                       offs, o, finals) != 0) {
        fprintf(stderr, "oracle_prefill failed\n");
        return 1;
    }
    bad |= !all_finite(o, (size_t)T * H_v * d_v) || !all_finite(exps, (size_t)E * H_v * SE) ||
           !all_finite(finals, (size_t)N * H_v * SE) || !all_finite(pool, (size_t)S * H_v * SE);
    /* sequence 3 (64 tokens from 0) ends on the grid: its one export is its final state */
    if (memcmp(exps + (size_t)offs[3] * H_v * SE, finals + (size_t)3 * H_v * SE, H_v * SE * sizeof(double)) != 0) {
        fprintf(stderr, "export at the end of sequence 3 differs from its final state\n");
        bad = 1;
    }
    /* a null export stream and no slots at all are valid too */
    if (oracle_prefill(H_k, H_v, d_k, d_v, N, cu, q, k, v, g, beta, 0.25, NULL, 0, NULL, NULL, NULL, 0, NULL, NULL,
                       o, NULL) != 0) {
        fprintf(stderr, "oracle_prefill without slots failed\n");
        return 1;
    }
    /* decode: rows 1 and 4 are padding */
    const int B = 6;
    int32_t si[6] = {0, -1, 2, 11, -1, 12};
    int32_t so[6] = {0, -1, 13, 11, 1, 14};
    double* od = (double*)calloc((size_t)B * H_v * d_v, sizeof(double));
    if (oracle_decode(H_k, H_v, d_k, d_v, B, q, k, v, g, beta, 0.25, pool, S, si, so, od) != 0) {
        fprintf(stderr, "oracle_decode failed\n");
        return 1;
    }
    bad |= !all_finite(od, (size_t)B * H_v * d_v) || !all_finite(pool, (size_t)S * H_v * SE);
    for (int j = 0; j < H_v * d_v; ++j)
        if (od[(size_t)1 * H_v * d_v + j] != 0.0 || od[(size_t)4 * H_v * d_v + j] != 0.0) bad = 1;
    free(q); free(k); free(v); free(g); free(beta); free(pool); free(exps); free(o); free(finals); free(od);
    if (bad) {
        fprintf(stderr, "oracle driver: a check failed\n");
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
