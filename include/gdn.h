/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule library, libgdn.so.
 *
 * The library runs the two halves of the Gated DeltaNet hot path on one GPU:
 *
 *   - packed single-token recurrent decode over cached per-request fp32 states
 *     ("[Model] Enable batch-invariant mixed decode and prefill for Qwen GDN",
 *     sections "What" and "How": cached rows take the packed recurrent decode path);
 *   - chunked prefill over 64-token chunks that returns outputs, final states and,
 *     optionally, the states reached on an export grid
 *     ("[V1][Hybrid] GatedDeltaNet Automatic Prefix Caching", section "Purpose":
 *     intermediate chunk states flattened into one contiguous stream;
 *     "[WIP][Kernel] Enable GDN batch-invariant prefix caching", section "Purpose":
 *     one grid lcm(64, block size) shared by prefill chunks and cache hits);
 *
 * and a mixed step that sends cached rows at the front of a step through the very
 * same decode launcher and the fresh prefills through the prefill launcher (the
 * route of the first page's "How" section), so that a decode row's bits never
 * depend on what else shares its step.
 *
 * The recurrence (the pages name it; the reading is the published gated delta rule):
 * per request and value head the state S has d_k rows and d_v columns, and each
 * token does
 *     S <- exp(g) S;   u = beta (v - S^T k);   S <- S + k u^T;   o = scale S^T q.
 * Value head h reads key head h / (num_v_heads / num_k_heads).
 *
 * Conventions for every entry point
 *   Memory      All tensor arguments are DEVICE pointers to caller-owned memory,
 *               dense and token-major:
 *                 q, k   [T, num_k_heads, d_k]      v, o  [T, num_v_heads, d_v]
 *                 g, beta [T, num_v_heads] fp32      state pool [num_slots, num_v_heads, d_k, d_v] fp32
 *               q, k, v and o share one dtype (gdn_dtype); g (natural-log decay),
 *               beta and all states are fp32.  Pointers must be 16-byte aligned.
 *               The library keeps no reference after a call returns and allocates
 *               no memory; scratch space is the caller's workspace argument.
 *   Streams     Each call only enqueues work on `stream` and never synchronises,
 *               so it may be captured into a HIP graph.  Inputs must stay valid
 *               until the stream reaches the work.
 *   Slots       Device index arrays are not read by the host.  A slot outside
 *               [0, num_slots) (for example -1) marks a padding row or "no state":
 *               the kernels bounds-check every slot and never touch such a slot.
 *               Within one call no slot may be written by one row and read or
 *               written by another (in-place use of a row's own slot is fine).
 *   Errors      Host arguments are validated before anything is enqueued.  A bad
 *               value returns GDN_ERR_INVALID_ARGUMENT or GDN_ERR_UNSUPPORTED and
 *               sets a thread-local message naming it (gdn_last_error); a failed
 *               launch returns GDN_ERR_HIP.  Nothing falls back to another path.
 *   Arithmetic  No argument changes the per-element arithmetic of a row: a decode
 *               row's output and state are bitwise identical whatever the batch
 *               size, its position in the batch, or the prefills sharing its step;
 *               a prefill sequence's results do not depend on its batch-mates.
 *   Range       bf16 prefills feed the matrix cores fp16 operands for q, k, the
 *               state and the per-token updates: q and k are expected L2-normalised
 *               (as the rule uses them), and states, values and outputs must stay
 *               below 2^15 in magnitude.  fp32 inputs and decode have no such limit.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Chunk length of the prefill.  Fixed: the pages' chunk kernel uses 64 tokens, and
 * the prefix-cache grid is lcm(64, block size). */
#define GDN_CHUNK 64

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARGUMENT = 1,
    GDN_ERR_UNSUPPORTED = 2,
    GDN_ERR_HIP = 3
} gdn_status;

/* Element type of q, k, v and o.  g, beta and every state are always fp32. */
typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Head layout shared by all entry points.  Supported: d_k, d_v in {64, 128};
 * num_v_heads a positive multiple of num_k_heads; dtype GDN_F32 or GDN_BF16;
 * scale finite (callers normally pass 1/sqrt(d_k)). */
typedef struct {
    int32_t num_k_heads;
    int32_t num_v_heads;
    int32_t d_k;
    int32_t d_v;
    int32_t dtype;   /* a gdn_dtype value */
    float scale;
} gdn_shape;

/* Bytes of device workspace that gdn_chunk_prefill / gdn_mixed_step need for
 * num_seqs sequences holding total_tokens tokens.  The current kernels keep every
 * intermediate in LDS and registers, so this is 0 (the argument is kept so that a
 * future kernel can take scratch without an ABI change); it is also 0 for an
 * unsupported shape. */
size_t gdn_chunk_prefill_workspace_size(const gdn_shape* shape, int32_t num_seqs,
                                        int64_t total_tokens);

/*
 * Packed recurrent decode: one token for each of num_rows cached rows.
 *   Defined by: "[Model] Enable batch-invariant mixed decode and prefill for Qwen GDN",
 *   sections "Why" and "How" (cached rows advance their recurrent state through the
 *   packed recurrent decode path); "[V1][Hybrid] GatedDeltaNet Automatic Prefix
 *   Caching", section "Purpose" (decode copies the last computed state into the newly
 *   scheduled slot: slot_out may differ from slot_in).
 *   q, k       device [num_rows, num_k_heads, d_k]      (dtype)
 *   v          device [num_rows, num_v_heads, d_v]      (dtype)
 *   g, beta    device [num_rows, num_v_heads]           fp32
 *   o          device [num_rows, num_v_heads, d_v]      (dtype), written
 *   state_pool device [num_slots, num_v_heads, d_k, d_v] fp32, read at slot_in[b] and
 *              written at slot_out[b]
 *   slot_in, slot_out  device [num_rows] int32.  Row b is padding when slot_in[b] is
 *              outside [0, num_slots): it is skipped and its o row is set to zero.  A
 *              valid slot_in with slot_out outside the range computes o and keeps
 *              the state unwritten.
 *   num_rows == 0 is a no-op returning GDN_OK.
 */
gdn_status gdn_recurrent_decode(const gdn_shape* shape, int32_t num_rows,
                                const void* q, const void* k, const void* v,
                                const float* g, const float* beta, void* o,
                                float* state_pool, int32_t num_slots,
                                const int32_t* slot_in, const int32_t* slot_out,
                                hipStream_t stream);

/*
 * Chunked prefill over num_seqs packed variable-length sequences.
 *   Defined by: "[Model] Enable batch-invariant mixed decode and prefill for Qwen GDN",
 *   section "Why" (fresh prefill rows go through chunk prefill); "[V1][Hybrid]
 *   GatedDeltaNet Automatic Prefix Caching", section "Purpose" (optional per-chunk
 *   intermediate states, flattened into one contiguous stream); "[WIP][Kernel] Enable
 *   GDN batch-invariant prefix caching", section "Purpose" (chunks and cache hits on
 *   one lcm(64, block) grid; a block size that is not a multiple of 64 is rejected).
 *   cu_seqlens device [num_seqs + 1] int32, cu[0] = 0, non-decreasing, cu[num_seqs] =
 *              total_tokens; sequence i owns tokens [cu[i], cu[i+1]).
 *   q, k, v, g, beta, o  as for decode with total_tokens rows.
 *   init_slot  device [num_seqs] int32: the initial state is state_pool[init_slot[i]],
 *              or zero when the slot is outside [0, num_slots).
 *   final_slot device [num_seqs] int32: the final state is written to
 *              state_pool[final_slot[i]] (skipped when outside the range).  It may
 *              equal the sequence's own init_slot (resume in place).
 *   start_pos  device [num_seqs] int32 or NULL (= all 0): absolute position of each
 *              sequence's first token, >= 0 (a negative value is outside the contract:
 *              the device cannot be checked without a sync).  Chunks lie on the absolute
 *              64-token grid: a sequence starting off the grid begins with a short chunk,
 *              and one ending off the grid ends with one.
 *   export_grid 0 = no export.  Otherwise a positive multiple of 64 (for example 64,
 *              or 1088 = lcm(64, 1088)); the state after every absolute position p with
 *              p % export_grid == 0 and start_pos < p <= start_pos + length is written
 *              to export_states[export_offsets[i] + m] (m counts sequence i's grid
 *              points in ascending order).
 *   export_states  device [sum of export counts, num_v_heads, d_k, d_v] fp32, written;
 *              unused (may be NULL) when export_slots is given.
 *   export_offsets device [num_seqs + 1] int32, the exclusive prefix sum of the
 *              per-sequence export counts (floor((s+L)/grid) - floor(s/grid)).
 *   export_slots   device [num_export_states] int32 or NULL.  When given, export idx
 *              is written straight into the cache: state_pool[export_slots[idx]]
 *              (skipped when the slot is outside [0, num_slots)), so a caller's block
 *              table can route each grid state into its prefix-cache block ("[V1][Hybrid]
 *              GatedDeltaNet Automatic Prefix Caching", section "Purpose": the returned
 *              chunk history is replayed into persistent cache blocks).  Export slots
 *              must differ from every slot the call reads (init_slot; in a mixed step
 *              also slot_in) and from each other.
 *   num_export_states  how many exports export_states (or export_slots) holds; an
 *              export whose index would reach it is dropped (the kernels never write
 *              past the buffer).
 *   workspace  device scratch of at least gdn_chunk_prefill_workspace_size() bytes,
 *              256-byte aligned, contents need no initialisation; may be NULL when
 *              that size is 0.
 *   num_seqs == 0 is a no-op returning GDN_OK.  A zero-length sequence copies its
 *   initial state (zeros without one) to its final slot; with total_tokens == 0 every
 *   sequence is empty and does just that.
 *
 *   Splitting a prompt across calls.  A resume at an absolute position that is a
 *   multiple of 64, from the state exported there, continues with the unsplit run's
 *   arithmetic, so its outputs and final state are bitwise those of the unsplit run.
 *   A split at any other token t is made bitwise the same way: a partial last chunk
 *   gives its rows the bits the full chunk would (within a chunk a row combines only
 *   rows at or before it), so the call that ends at t returns the unsplit run's
 *   outputs up to t; the next call starts at t0 = 64 floor(t / 64) from the state
 *   after t0 (an export on a 64 grid, or the initial state when no grid point was
 *   crossed) and re-feeds the t - t0 < 64 tokens since, whose outputs come out
 *   bitwise equal again and may be discarded.
 */
gdn_status gdn_chunk_prefill(const gdn_shape* shape, int32_t num_seqs, int64_t total_tokens,
                             const int32_t* cu_seqlens, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, void* o,
                             float* state_pool, int32_t num_slots, const int32_t* init_slot,
                             const int32_t* final_slot, const int32_t* start_pos,
                             int32_t export_grid, float* export_states,
                             const int32_t* export_offsets, const int32_t* export_slots,
                             int64_t num_export_states, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * One mixed decode-plus-prefill step: tokens [0, num_decode_rows) are cached decode
 * rows (one token each, states at slot_in / slot_out) and the prefill sequences
 * follow, described by cu_seqlens_prefill relative to token num_decode_rows.
 *   Defined by: "[Model] Enable batch-invariant mixed decode and prefill for Qwen GDN",
 *   sections "What", "Why" and "How": cached decode rows at the front of a mixed step
 *   go through the same packed decode helper as a decode-only step; fresh prefill rows
 *   go through chunk prefill.  This entry point is exactly gdn_recurrent_decode on the
 *   first rows followed by gdn_chunk_prefill on the rest, through the same internal
 *   launchers and kernels, on one stream; decode and prefill slots must be disjoint.
 *   Arguments have the meanings given above; q, k, v, g, beta and o hold
 *   num_decode_rows + prefill_tokens rows.
 */
gdn_status gdn_mixed_step(const gdn_shape* shape, int32_t num_decode_rows,
                          const int32_t* slot_in, const int32_t* slot_out,
                          int32_t num_prefill_seqs, int64_t prefill_tokens,
                          const int32_t* cu_seqlens_prefill, const void* q, const void* k,
                          const void* v, const float* g, const float* beta, void* o,
                          float* state_pool, int32_t num_slots, const int32_t* init_slot,
                          const int32_t* final_slot, const int32_t* start_pos,
                          int32_t export_grid, float* export_states,
                          const int32_t* export_offsets, const int32_t* export_slots,
                          int64_t num_export_states, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * Multi-token verify rows: each of num_rows cached rows advances by tokens_per_row
 * tokens in order, as tokens_per_row successive decode steps of that row, and the state
 * after each token is kept so that a caller can roll the row back to any accepted
 * prefix of the tokens.
 *   Context: speculative decoding is left out of the mixed-step route ("[Model] Enable
 *   batch-invariant mixed decode and prefill for Qwen GDN", section "Out of scope") and
 *   of prefix caching ("[V1][Hybrid] GatedDeltaNet Automatic Prefix Caching", section
 *   "TODOs"); this is the recurrent path such rows would take.
 *   q, k       device [num_rows * tokens_per_row, num_k_heads, d_k]: row b's tokens are
 *              rows b * tokens_per_row .. b * tokens_per_row + tokens_per_row - 1.
 *   v, o       device [num_rows * tokens_per_row, num_v_heads, d_v] (o written).
 *   g, beta    device [num_rows * tokens_per_row, num_v_heads] fp32.
 *   slot_in    device [num_rows] int32: the row's state before its first token; a slot
 *              outside [0, num_slots) marks a padding row (outputs zero-filled, no state
 *              written).
 *   token_slots device [num_rows * tokens_per_row] int32: the state after token t of
 *              row b is written to state_pool[token_slots[b * tokens_per_row + t]];
 *              a slot outside [0, num_slots) keeps that state nowhere.  A token slot may
 *              equal slot_in (then the state is read before any write).
 *   With tokens_per_row = 1 this is gdn_recurrent_decode (token_slots = slot_out), on
 *   the same kernel; a verify row is bitwise equal to its tokens decoded one call at a
 *   time.  tokens_per_row < 1 returns GDN_ERR_INVALID_ARGUMENT.
 */
gdn_status gdn_recurrent_verify(const gdn_shape* shape, int32_t num_rows, int32_t tokens_per_row,
                                const void* q, const void* k, const void* v, const float* g,
                                const float* beta, void* o, float* state_pool, int32_t num_slots,
                                const int32_t* slot_in, const int32_t* token_slots,
                                hipStream_t stream);

/* Message describing the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the thread's next call into the library. */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
