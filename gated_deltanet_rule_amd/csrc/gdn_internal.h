// gdn_internal.h -- launcher interface between the C ABI layer (gdn_api.cpp) and the
// gfx950 kernels (gdn_decode.hip, gdn_prefill.hip, gdn_prefill_bf16.hip).  Host-side declarations only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Packed decode over cached rows: tokens_per_row tokens per row (1 for decode,
// more for verify rows); slot_out holds one slot per token.
struct DecodeArgs {
    int H_k, H_v, d_k, d_v, dtype;
    float scale;
    int num_rows;
    int tokens_per_row;
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    void* o;
    float* pool;
    int num_slots;
    const int32_t* slot_in;
    const int32_t* slot_out;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Chunked prefill over packed variable-length sequences.
struct PrefillArgs {
    int H_k, H_v, d_k, d_v, dtype;
    float scale;
    int num_seqs;
    int64_t total_tokens;
    const int32_t* cu_seqlens;
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    void* o;
    float* pool;
    int num_slots;
    const int32_t* init_slot;
    const int32_t* final_slot;
    const int32_t* start_pos;
    int export_grid;
    float* export_states;
    const int32_t* export_offsets;
    const int32_t* export_slots;     // when set, exports go to pool[export_slots[idx]]
    int64_t export_capacity;
    void* workspace;
};

// Device scratch the prefill needs (none: every chunk's intermediates stay in LDS
// and registers).
size_t prefill_workspace_bytes(int H_v, int dtype, int num_seqs, int64_t total_tokens);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// The bf16 kernel (gdn_prefill_bf16.hip); launch_prefill routes bf16 calls to it.
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
// Compute units of the current device, read once per device (gdn_prefill_bf16.hip):
// the prefill launchers pick their workgroup shape by it.
int device_cus();

}  // namespace gdn
