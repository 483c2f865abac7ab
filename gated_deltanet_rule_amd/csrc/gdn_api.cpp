// gdn_api.cpp -- the C ABI of libgdn.so: host-side validation and dispatch to the
// gfx950 launchers.  Every scalar and pointer the host can see is checked before any
// work is enqueued; a bad value returns an error status and a message naming it
// (fail closed, no fallback path), following the rule the second page's review
// applies to block sizes: a size that is not a multiple of the chunk is rejected and
// the message states the chunk size ("[V1][Hybrid] GatedDeltaNet Automatic Prefix
// Caching", review of the backend's size check).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

gdn_status check_shape(const gdn_shape* s) {
    if (!s) return fail(GDN_ERR_INVALID_ARGUMENT, "shape is NULL");
    if (s->num_k_heads <= 0 || s->num_v_heads <= 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "head counts must be positive (num_k_heads %d, num_v_heads %d)",
                    s->num_k_heads, s->num_v_heads);
    if (s->num_v_heads > 65535)
        return fail(GDN_ERR_UNSUPPORTED, "num_v_heads %d exceeds 65535", s->num_v_heads);
    if (s->num_v_heads % s->num_k_heads != 0)
        return fail(GDN_ERR_UNSUPPORTED, "num_v_heads %d is not a multiple of num_k_heads %d",
                    s->num_v_heads, s->num_k_heads);
    if ((s->d_k != 64 && s->d_k != 128) || (s->d_v != 64 && s->d_v != 128))
        return fail(GDN_ERR_UNSUPPORTED, "head dims d_k %d, d_v %d: each must be 64 or 128", s->d_k,
                    s->d_v);
    if (s->dtype != GDN_F32 && s->dtype != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "dtype %d is neither GDN_F32 (0) nor GDN_BF16 (1)", s->dtype);
    if (!std::isfinite(s->scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "scale is not finite");
    return GDN_OK;
}

struct Ptr {
    const char* name;
    const void* p;
    size_t align;
};

gdn_status check_ptrs(std::initializer_list<Ptr> ps) {
    for (const Ptr& x : ps) {
        if (!x.p) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is NULL", x.name);
        if (!aligned(x.p, x.align))
            return fail(GDN_ERR_INVALID_ARGUMENT, "%s (%p) is not %zu-byte aligned", x.name, x.p, x.align);
    }
    return GDN_OK;
}

gdn_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return GDN_OK;
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

gdn_status check_decode(const gdn_shape* shape, int32_t num_rows, const void* q, const void* k,
                        const void* v, const float* g, const float* beta, void* o,
                        float* state_pool, int32_t num_slots, const int32_t* slot_in,
                        const int32_t* slot_out) {
    gdn_status st = check_shape(shape);
    if (st != GDN_OK) return st;
    if (num_rows < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "num_rows %d is negative", num_rows);
    if (num_slots < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "num_slots %d is negative", num_slots);
    if (num_rows == 0) return GDN_OK;
    // one workgroup per 64 value columns of each (row, value head)
    if ((int64_t)num_rows * shape->num_v_heads * (shape->d_v / 64) > 0x7fffffffLL)
        return fail(GDN_ERR_UNSUPPORTED, "num_rows %d x num_v_heads %d x d_v / 64 exceeds the launch grid",
                    num_rows, shape->num_v_heads);
    return check_ptrs({{"q", q, 16}, {"k", k, 16}, {"v", v, 16}, {"g", g, 4}, {"beta", beta, 4},
                       {"o", o, 16}, {"state_pool", state_pool, 16}, {"slot_in", slot_in, 4},
                       {"slot_out", slot_out, 4}});
}

gdn_status check_prefill(const gdn_shape* shape, int32_t num_seqs, int64_t total_tokens,
                         const int32_t* cu_seqlens, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, void* o, float* state_pool,
                         int32_t num_slots, const int32_t* init_slot, const int32_t* final_slot,
                         const int32_t* start_pos, int32_t export_grid, float* export_states,
                         const int32_t* export_offsets, const int32_t* export_slots,
                         int64_t num_export_states, void* workspace, size_t workspace_bytes) {
    gdn_status st = check_shape(shape);
    if (st != GDN_OK) return st;
    if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs %d is negative", num_seqs);
    if (total_tokens < 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "total_tokens %lld is negative", (long long)total_tokens);
    if (total_tokens > 0x7fffffffLL - 2 * GDN_CHUNK)
        return fail(GDN_ERR_UNSUPPORTED, "total_tokens %lld exceeds the supported 2^31 - 129",
                    (long long)total_tokens);
    if (num_slots < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "num_slots %d is negative", num_slots);
    if (export_grid < 0 || export_grid % GDN_CHUNK != 0)
        return fail(GDN_ERR_INVALID_ARGUMENT,
                    "export_grid %d is not a multiple of chunk size %d (use 0 for no export)", export_grid,
                    GDN_CHUNK);
    if (num_export_states < 0)
        return fail(GDN_ERR_INVALID_ARGUMENT, "num_export_states %lld is negative",
                    (long long)num_export_states);
    if (num_seqs == 0) return GDN_OK;
    if ((int64_t)num_seqs * shape->num_v_heads > 0x7fffffffLL)
        return fail(GDN_ERR_UNSUPPORTED, "problem too large for one launch (num_seqs %d, total_tokens %lld)",
                    num_seqs, (long long)total_tokens);
    st = check_ptrs({{"cu_seqlens", cu_seqlens, 4}, {"init_slot", init_slot, 4},
                     {"final_slot", final_slot, 4}});
    if (st != GDN_OK) return st;
    if (start_pos && !aligned(start_pos, 4))
        return fail(GDN_ERR_INVALID_ARGUMENT, "start_pos is not 4-byte aligned");
    if (num_slots > 0) {
        st = check_ptrs({{"state_pool", state_pool, 16}});
        if (st != GDN_OK) return st;
    }
    if (total_tokens > 0) {
        st = check_ptrs({{"q", q, 16}, {"k", k, 16}, {"v", v, 16}, {"g", g, 4}, {"beta", beta, 4},
                         {"o", o, 16}});
        if (st != GDN_OK) return st;
    }
    if (export_grid > 0) {
        st = check_ptrs({{"export_offsets", export_offsets, 4}});
        if (st != GDN_OK) return st;
        if (num_export_states > 0) {
            st = export_slots ? check_ptrs({{"export_slots", export_slots, 4}})
                              : check_ptrs({{"export_states", export_states, 16}});
            if (st != GDN_OK) return st;
        }
    }
    const size_t need = gdn::prefill_workspace_bytes(shape->num_v_heads, shape->dtype, num_seqs, total_tokens);
    if (workspace_bytes < need)
        return fail(GDN_ERR_INVALID_ARGUMENT, "workspace_bytes %zu is smaller than the %zu bytes required",
                    workspace_bytes, need);
    if (need > 0) {
        st = check_ptrs({{"workspace", workspace, 256}});
        if (st != GDN_OK) return st;
    }
    return GDN_OK;
}

gdn::DecodeArgs decode_args(const gdn_shape* s, int32_t num_rows, const void* q, const void* k,
                            const void* v, const float* g, const float* beta, void* o, float* pool,
                            int32_t num_slots, const int32_t* slot_in, const int32_t* slot_out) {
    gdn::DecodeArgs a;
    a.H_k = s->num_k_heads;
    a.H_v = s->num_v_heads;
    a.d_k = s->d_k;
    a.d_v = s->d_v;
    a.dtype = s->dtype;
    a.scale = s->scale;
    a.num_rows = num_rows;
    a.tokens_per_row = 1;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.o = o;
    a.pool = pool;
    a.num_slots = num_slots;
    a.slot_in = slot_in;
    a.slot_out = slot_out;
    return a;
}

gdn::PrefillArgs prefill_args(const gdn_shape* s, int32_t num_seqs, int64_t total_tokens,
                              const int32_t* cu_seqlens, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, void* o, float* pool, int32_t num_slots,
                              const int32_t* init_slot, const int32_t* final_slot,
                              const int32_t* start_pos, int32_t export_grid, float* export_states,
                              const int32_t* export_offsets, const int32_t* export_slots,
                              int64_t num_export_states, void* workspace) {
    gdn::PrefillArgs a;
    a.H_k = s->num_k_heads;
    a.H_v = s->num_v_heads;
    a.d_k = s->d_k;
    a.d_v = s->d_v;
    a.dtype = s->dtype;
    a.scale = s->scale;
    a.num_seqs = num_seqs;
    a.total_tokens = total_tokens;
    a.cu_seqlens = cu_seqlens;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.o = o;
    a.pool = pool;
    a.num_slots = num_slots;
    a.init_slot = init_slot;
    a.final_slot = final_slot;
    a.start_pos = start_pos;
    a.export_grid = export_grid;
    a.export_slots = export_grid > 0 ? export_slots : nullptr;
    a.export_states = export_grid > 0 && !export_slots ? export_states : nullptr;
    a.export_offsets = export_grid > 0 ? export_offsets : nullptr;
    a.export_capacity = export_grid > 0 && (a.export_states || a.export_slots) ? num_export_states : 0;
    a.workspace = workspace;
    return a;
}

}  // namespace

extern "C" {

size_t gdn_chunk_prefill_workspace_size(const gdn_shape* shape, int32_t num_seqs, int64_t total_tokens) {
    if (check_shape(shape) != GDN_OK || num_seqs < 0 || total_tokens < 0) return 0;
    return gdn::prefill_workspace_bytes(shape->num_v_heads, shape->dtype, num_seqs, total_tokens);
}

gdn_status gdn_recurrent_decode(const gdn_shape* shape, int32_t num_rows, const void* q, const void* k,
                                const void* v, const float* g, const float* beta, void* o,
                                float* state_pool, int32_t num_slots, const int32_t* slot_in,
                                const int32_t* slot_out, hipStream_t stream) {
    g_last_error.clear();
    gdn_status st = check_decode(shape, num_rows, q, k, v, g, beta, o, state_pool, num_slots, slot_in,
                                 slot_out);
    if (st != GDN_OK || num_rows == 0) return st;
    return hip_status(gdn::launch_decode(decode_args(shape, num_rows, q, k, v, g, beta, o, state_pool,
                                                     num_slots, slot_in, slot_out),
                                         stream),
                      "decode launch");
}

gdn_status gdn_chunk_prefill(const gdn_shape* shape, int32_t num_seqs, int64_t total_tokens,
                             const int32_t* cu_seqlens, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, void* o, float* state_pool,
                             int32_t num_slots, const int32_t* init_slot, const int32_t* final_slot,
                             const int32_t* start_pos, int32_t export_grid, float* export_states,
                             const int32_t* export_offsets, const int32_t* export_slots,
                             int64_t num_export_states, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    g_last_error.clear();
    gdn_status st = check_prefill(shape, num_seqs, total_tokens, cu_seqlens, q, k, v, g, beta, o,
                                  state_pool, num_slots, init_slot, final_slot, start_pos, export_grid,
                                  export_states, export_offsets, export_slots, num_export_states,
                                  workspace, workspace_bytes);
    if (st != GDN_OK || num_seqs == 0) return st;
    return hip_status(gdn::launch_prefill(prefill_args(shape, num_seqs, total_tokens, cu_seqlens, q, k, v,
                                                       g, beta, o, state_pool, num_slots, init_slot,
                                                       final_slot, start_pos, export_grid, export_states,
                                                       export_offsets, export_slots, num_export_states,
                                                       workspace),
                                          stream),
                      "prefill launch");
}

gdn_status gdn_mixed_step(const gdn_shape* shape, int32_t num_decode_rows, const int32_t* slot_in,
                          const int32_t* slot_out, int32_t num_prefill_seqs, int64_t prefill_tokens,
                          const int32_t* cu_seqlens_prefill, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, void* o, float* state_pool, int32_t num_slots,
                          const int32_t* init_slot, const int32_t* final_slot, const int32_t* start_pos,
                          int32_t export_grid, float* export_states, const int32_t* export_offsets,
                          const int32_t* export_slots, int64_t num_export_states, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    gdn_status st = check_decode(shape, num_decode_rows, q, k, v, g, beta, o, state_pool, num_slots,
                                 slot_in, slot_out);
    if (st != GDN_OK) return st;
    // the prefill part starts num_decode_rows tokens into every token-major tensor
    const size_t esz = shape->dtype == GDN_BF16 ? 2 : 4;
    const size_t B = (size_t)num_decode_rows;
    const char* qp = static_cast<const char*>(q) + B * shape->num_k_heads * shape->d_k * esz;
    const char* kp = static_cast<const char*>(k) + B * shape->num_k_heads * shape->d_k * esz;
    const char* vp = static_cast<const char*>(v) + B * shape->num_v_heads * shape->d_v * esz;
    char* op = static_cast<char*>(o) + B * shape->num_v_heads * shape->d_v * esz;
    const float* gp = g + B * shape->num_v_heads;
    const float* bp = beta + B * shape->num_v_heads;
    st = check_prefill(shape, num_prefill_seqs, prefill_tokens, cu_seqlens_prefill, qp, kp, vp, gp, bp, op,
                       state_pool, num_slots, init_slot, final_slot, start_pos, export_grid, export_states,
                       export_offsets, export_slots, num_export_states, workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    // cached rows first, through the same launcher and kernel as a decode-only step
    if (num_decode_rows > 0) {
        st = hip_status(gdn::launch_decode(decode_args(shape, num_decode_rows, q, k, v, g, beta, o,
                                                       state_pool, num_slots, slot_in, slot_out),
                                           stream),
                        "mixed-step decode launch");
        if (st != GDN_OK) return st;
    }
    if (num_prefill_seqs == 0) return GDN_OK;
    return hip_status(gdn::launch_prefill(prefill_args(shape, num_prefill_seqs, prefill_tokens,
                                                       cu_seqlens_prefill, qp, kp, vp, gp, bp, op, state_pool,
                                                       num_slots, init_slot, final_slot, start_pos,
                                                       export_grid, export_states, export_offsets,
                                                       export_slots, num_export_states, workspace),
                                          stream),
                      "mixed-step prefill launch");
}

gdn_status gdn_recurrent_verify(const gdn_shape* shape, int32_t num_rows, int32_t tokens_per_row,
                                const void* q, const void* k, const void* v, const float* g, const float* beta,
                                void* o, float* state_pool, int32_t num_slots, const int32_t* slot_in,
                                const int32_t* token_slots, hipStream_t stream) {
    g_last_error.clear();
    if (tokens_per_row < 1)
        return fail(GDN_ERR_INVALID_ARGUMENT, "tokens_per_row %d is less than 1", tokens_per_row);
    if ((int64_t)num_rows * tokens_per_row > 0x7fffffffLL)
        return fail(GDN_ERR_UNSUPPORTED, "num_rows %d x tokens_per_row %d is too large", num_rows, tokens_per_row);
    gdn_status st = check_decode(shape, num_rows, q, k, v, g, beta, o, state_pool, num_slots, slot_in,
                                 token_slots);
    if (st != GDN_OK || num_rows == 0) return st;
    gdn::DecodeArgs a = decode_args(shape, num_rows, q, k, v, g, beta, o, state_pool, num_slots, slot_in,
                                    token_slots);
    a.tokens_per_row = tokens_per_row;
    return hip_status(gdn::launch_decode(a, stream), "verify launch");
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
