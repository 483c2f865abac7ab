// gdn_device.h -- device helpers shared by the prefill kernels: chunk geometry on the
// absolute 64-token grid, a wave prefix sum, and an LDS-only workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {
namespace dev {

constexpr int kC = 64;   // chunk length

// Chunks of a sequence lie on the absolute 64-token grid: with a = start_pos % 64,
// chunk c covers local tokens [max(0, 64c - a), min(L, 64(c+1) - a)).
__device__ __forceinline__ int seq_chunks(int L, int a) { return L > 0 ? (a + L + kC - 1) / kC : 0; }

__device__ __forceinline__ void chunk_span(int c, int a, int len, int& b0, int& e0) {
    b0 = c * kC - a < 0 ? 0 : c * kC - a;
    e0 = (c + 1) * kC - a > len ? len : (c + 1) * kC - a;
}

// Token range of sequence i, clamped into [0, T] so that a malformed cu_seqlens can
// only give wrong results, never an access outside the tensors.
__device__ __forceinline__ void seq_range(const int32_t* cu, int i, int64_t T, int& lo, int& len) {
    int64_t b = cu[i], e = cu[i + 1];
    b = b < 0 ? 0 : (b > T ? T : b);
    e = e < b ? b : (e > T ? T : e);
    lo = (int)b;
    len = (int)(e - b);
}

// Inclusive prefix sum over the 64 lanes of a wave, in a fixed order: shifted adds
// within each row of 16 lanes (DPP row_shr 1, 2, 4, 8), then the last lane of row 0
// and of row 2 added to rows 1 and 3 (row_bcast:15), then lane 31 added to rows 2
// and 3 (row_bcast:31).  Lanes that a shift or broadcast does not reach add zero.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_term(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_term<0x111, 0xf>(x);   // row_shr:1
    x += dpp_term<0x112, 0xf>(x);   // row_shr:2
    x += dpp_term<0x114, 0xf>(x);   // row_shr:4
    x += dpp_term<0x118, 0xf>(x);   // row_shr:8
    x += dpp_term<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_term<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for every
// outstanding global load (its release fence drains vmcnt), which would expose the
// latency of the next chunk's prefetch at the first barrier after it is issued.  The
// kernels share data between waves only through LDS, so waiting for LDS operations
// is enough; the memory clobber keeps the compiler from moving accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace dev
}  // namespace gdn
