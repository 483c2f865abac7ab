/*
 * gdn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, sequential fp64 evaluation of the gated delta rule, used to check
 * the GPU library.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load this file's library; the product path never does.  It
 * shares no code, header or table with the GPU library.
 *
 * What it computes.  The pages this project follows name the method but print no
 * formula:
 *   - "[Model] Enable batch-invariant mixed decode and prefill for Qwen GDN",
 *     sections "Why" and "Results": Gated DeltaNet layers keep a recurrent ("SSM")
 *     state per request; cached rows advance it one token at a time.
 *   - "[V1][Hybrid] GatedDeltaNet Automatic Prefix Caching", section "Purpose":
 *     the chunk kernel can also hand back the state reached at each chunk boundary,
 *     flattened into one contiguous stream.
 *   - "[WIP][Kernel] Enable GDN batch-invariant prefix caching", section "Purpose":
 *     prefill chunks and cache hits share one grid, lcm(64, block size).
 * The recurrence itself is read as the published gated delta rule (Yang, Kautz and
 * Hatamizadeh, "Gated Delta Networks", ICLR 2025), written for a state S with d_k
 * rows and d_v columns (d_v fastest in memory).  Per token t of one (sequence,
 * value head):
 *
 *     S   <- exp(g_t) * S                        decay first
 *     u   <- beta_t * (v_t - S^T k_t)            delta-rule prediction error
 *     S   <- S + k_t u^T                         rank-1 write
 *     o_t <- scale * S^T q_t                     read from the updated state
 *
 * which is the product form S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T.
 * Value head h reads key head h / (H_v / H_k) (contiguous GQA groups).
 *
 * Every loop below is the definition written out: no blocking, no reordering, no
 * chunking.  All arithmetic is in double precision; inputs arrive already widened
 * from the exact values the GPU receives.
 *
 * Parity unpinned: the output scale (a parameter), the GQA head map above and the
 * [d_k][d_v] state layout are conventions the pages do not fix; the oracle and the
 * GPU library share them by definition, and no pin can check them.  Everything
 * else is pinned by the tests (brute-force products, exact rationals, closed forms,
 * an independent chunked evaluation, planted mistakes).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

/* One token of the recurrence on a d_k x d_v state held row-major (d_v fastest).
 * u is caller scratch of length d_v.  Writes d_v outputs to o. */
static void oracle_token(int d_k, int d_v, double* S, const double* q, const double* k,
                         const double* v, double g, double beta, double scale,
                         double* u, double* o)
{
    const double alpha = exp(g);
    for (int i = 0; i < d_k; ++i)
        for (int j = 0; j < d_v; ++j)
            S[(size_t)i * d_v + j] *= alpha;

    for (int j = 0; j < d_v; ++j) {
        double pred = 0.0;                       /* (S^T k)_j */
        for (int i = 0; i < d_k; ++i)
            pred += S[(size_t)i * d_v + j] * k[i];
        u[j] = beta * (v[j] - pred);
    }

    for (int i = 0; i < d_k; ++i)
        for (int j = 0; j < d_v; ++j)
            S[(size_t)i * d_v + j] += k[i] * u[j];

    for (int j = 0; j < d_v; ++j) {
        double acc = 0.0;                        /* (S^T q)_j */
        for (int i = 0; i < d_k; ++i)
            acc += S[(size_t)i * d_v + j] * q[i];
        o[j] = scale * acc;
    }
}

/*
 * Prefill over packed variable-length sequences.
 *
 * Layouts (all dense, token-major):
 *   q, k          [T, H_k, d_k]          v, o  [T, H_v, d_v]
 *   g, beta       [T, H_v]               cu_seqlens [num_seqs + 1], cu[0] = 0
 *   pool          [num_slots, H_v, d_k, d_v]   (read at init_slot, written at final_slot)
 *   init_slot[i] < 0 means a zero initial state.  final_slot[i] < 0 means "do not
 *   write the final state back".
 *   start_pos     absolute position of each sequence's first token (NULL = all 0)
 *   export_grid   0 = no export; otherwise the state after absolute position p is
 *                 exported whenever p % export_grid == 0, sequence-major then p
 *                 ascending, at export_states[(export_offsets[i] + m), H_v, d_k, d_v].
 *   final_states  optional [num_seqs, H_v, d_k, d_v] copy of every final state.
 *
 * All initial states are read before any final state is written, so a sequence may
 * resume in place (final_slot == init_slot).
 */
int oracle_prefill(int H_k, int H_v, int d_k, int d_v, int num_seqs, const int32_t* cu_seqlens,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, double scale, double* pool, int num_slots,
                   const int32_t* init_slot, const int32_t* final_slot, const int32_t* start_pos,
                   int export_grid, double* export_states, const int32_t* export_offsets,
                   double* o, double* final_states)
{
    if (H_k <= 0 || H_v <= 0 || d_k <= 0 || d_v <= 0 || num_seqs < 0 || H_v % H_k != 0)
        return ORACLE_EINVAL;
    if (export_grid < 0 || (export_grid > 0 && (!export_states || !export_offsets)))
        return ORACLE_EINVAL;

    const int group = H_v / H_k;
    const size_t state_elems = (size_t)d_k * d_v;
    const int units = num_seqs * H_v;
    double* states = (double*)calloc((size_t)(units > 0 ? units : 1) * state_elems, sizeof(double));
    if (!states) return ORACLE_EINVAL;

    for (int i = 0; i < num_seqs; ++i)
        if (init_slot && init_slot[i] >= 0 && pool)
            memcpy(states + (size_t)i * H_v * state_elems,
                   pool + (size_t)init_slot[i] * H_v * state_elems,
                   (size_t)H_v * state_elems * sizeof(double));

    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int unit = 0; unit < units; ++unit) {
        const int i = unit / H_v;
        const int h = unit % H_v;
        const int kh = h / group;
        double* S = states + (size_t)unit * state_elems;
        double* u = (double*)malloc((size_t)d_v * sizeof(double));
        if (!u) { status = ORACLE_EINVAL; continue; }
        const int64_t pos0 = start_pos ? start_pos[i] : 0;
        int m = 0;
        for (int32_t t = cu_seqlens[i]; t < cu_seqlens[i + 1]; ++t) {
            oracle_token(d_k, d_v, S,
                         q + ((size_t)t * H_k + kh) * d_k,
                         k + ((size_t)t * H_k + kh) * d_k,
                         v + ((size_t)t * H_v + h) * d_v,
                         g[(size_t)t * H_v + h], beta[(size_t)t * H_v + h], scale, u,
                         o + ((size_t)t * H_v + h) * d_v);
            const int64_t p = pos0 + (t - cu_seqlens[i]) + 1;   /* tokens consumed so far */
            if (export_grid > 0 && p % export_grid == 0) {
                memcpy(export_states + ((size_t)(export_offsets[i] + m) * H_v + h) * state_elems,
                       S, state_elems * sizeof(double));
                ++m;
            }
        }
        free(u);
    }

    for (int i = 0; i < num_seqs; ++i) {
        const double* src = states + (size_t)i * H_v * state_elems;
        if (final_slot && final_slot[i] >= 0 && pool)
            memcpy(pool + (size_t)final_slot[i] * H_v * state_elems, src,
                   (size_t)H_v * state_elems * sizeof(double));
        if (final_states)
            memcpy(final_states + (size_t)i * H_v * state_elems, src,
                   (size_t)H_v * state_elems * sizeof(double));
    }
    free(states);
    (void)num_slots;
    return status;
}

/*
 * Single-token decode for a packed batch of cached rows: row b reads its state from
 * pool[slot_in[b]], advances it by one token and writes it to pool[slot_out[b]].
 * A row with slot_in[b] < 0 is padding: it is skipped and its output is zero.
 * This is the same recurrence as the prefill with one-token sequences.
 *   q, k [B, H_k, d_k]; v, o [B, H_v, d_v]; g, beta [B, H_v].
 */
int oracle_decode(int H_k, int H_v, int d_k, int d_v, int num_rows, const double* q,
                  const double* k, const double* v, const double* g, const double* beta,
                  double scale, double* pool, int num_slots, const int32_t* slot_in,
                  const int32_t* slot_out, double* o)
{
    if (H_k <= 0 || H_v <= 0 || d_k <= 0 || d_v <= 0 || num_rows < 0 || H_v % H_k != 0)
        return ORACLE_EINVAL;
    const int group = H_v / H_k;
    const size_t state_elems = (size_t)d_k * d_v;
    const int units = num_rows * H_v;
    double* states = (double*)calloc((size_t)(units > 0 ? units : 1) * state_elems, sizeof(double));
    if (!states) return ORACLE_EINVAL;
    for (int b = 0; b < num_rows; ++b)
        if (slot_in[b] >= 0)
            memcpy(states + (size_t)b * H_v * state_elems,
                   pool + (size_t)slot_in[b] * H_v * state_elems,
                   (size_t)H_v * state_elems * sizeof(double));

    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int unit = 0; unit < units; ++unit) {
        const int b = unit / H_v;
        const int h = unit % H_v;
        const int kh = h / group;
        double* ob = o + ((size_t)b * H_v + h) * d_v;
        if (slot_in[b] < 0) {
            for (int j = 0; j < d_v; ++j) ob[j] = 0.0;
            continue;
        }
        double* u = (double*)malloc((size_t)d_v * sizeof(double));
        if (!u) { status = ORACLE_EINVAL; continue; }
        oracle_token(d_k, d_v, states + (size_t)unit * state_elems,
                     q + ((size_t)b * H_k + kh) * d_k, k + ((size_t)b * H_k + kh) * d_k,
                     v + ((size_t)b * H_v + h) * d_v, g[(size_t)b * H_v + h],
                     beta[(size_t)b * H_v + h], scale, u, ob);
        free(u);
    }

    for (int b = 0; b < num_rows; ++b)
        if (slot_in[b] >= 0 && slot_out[b] >= 0)
            memcpy(pool + (size_t)slot_out[b] * H_v * state_elems,
                   states + (size_t)b * H_v * state_elems,
                   (size_t)H_v * state_elems * sizeof(double));
    free(states);
    (void)num_slots;
    return status;
}

/* Number of OpenMP threads the parallel loops above will use (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { if (n > 0) omp_set_num_threads(n); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif
