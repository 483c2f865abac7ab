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

// Inclusive prefix sum over the 64 lanes of a wave (Hillis-Steele, fixed order).
__device__ __forceinline__ float wave_inclusive_sum(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
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
