// gdn_probe.hip -- memory-pattern reference kernels for the benchmark (libgdn_probe.so).
//
// Not part of the gated delta rule: these two kernels measure what the MI355X's HBM
// delivers for the access patterns of the decode kernel, so that the decode's state
// bandwidth can be reported against an achievable figure as well as the 8 TB/s peak.
//   gdn_probe_stream_copy   a plain streaming copy, one 16-byte vector per thread, with
//                           non-temporal loads and stores: the ceiling for moving bytes.
//   gdn_probe_state_rmw     the decode's dependency pattern without its arithmetic: one
//                           workgroup of 1024 threads per 64 KiB fp32 state (d_k = d_v =
//                           128), every element loaded, the column sums over the 128
//                           rows formed in a fixed order through LDS, and every element
//                           stored back in place only after its column's sum is known
//                           (x + 1e-30 sum: the same bits in practice, but a true data
//                           dependency).  Units are (slot, head) pairs of a state pool.
// Both only enqueue on the given stream and return the launch status.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                          size_t n4) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n4) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

constexpr int kRmwThreads = 1024;

__global__ __launch_bounds__(kRmwThreads) void state_rmw_kernel(float* pool, const int32_t* slots, int heads,
                                                                int num_slots) {
    constexpr int DV = 128, DK = 128, TPR = DV / 4, RG = kRmwThreads / TPR, R = DK / RG;
    const int unit = blockIdx.x;
    const int b = unit / heads, h = unit - b * heads;
    const int sl = slots[b];
    if (sl < 0 || sl >= num_slots) return;
    const int tid = threadIdx.x, c4 = tid % TPR, rg = tid / TPR;
    float* base = pool + ((size_t)sl * heads + h) * (size_t)(DK * DV);
    f32x4 s[R];
#pragma unroll
    for (int m = 0; m < R; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base + (size_t)(rg + RG * m) * DV) + c4);
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < R; ++m) p += s[m];
    __shared__ f32x4 red[RG][TPR];
    red[rg][c4] = p;
    __syncthreads();
    f32x4 tot = red[0][c4];
#pragma unroll
    for (int r = 1; r < RG; ++r) tot += red[r][c4];
#pragma unroll
    for (int m = 0; m < R; ++m)
        __builtin_nontemporal_store(s[m] + 1e-30f * tot,
                                    reinterpret_cast<f32x4*>(base + (size_t)(rg + RG * m) * DV) + c4);
}

}  // namespace

extern "C" {

// Copy n_bytes (a multiple of 16, both pointers 16-byte aligned) from src to dst.
int gdn_probe_stream_copy(const void* src, void* dst, size_t n_bytes, hipStream_t stream) {
    if (!src || !dst || n_bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(dst) % 16 != 0)
        return (int)hipErrorInvalidValue;
    const size_t n4 = n_bytes / 16;
    if (n4 == 0) return (int)hipSuccess;
    const size_t blocks = (n4 + 255) / 256;
    if (blocks > 0x7fffffffULL) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), n4);
    return (int)hipGetLastError();
}

// The decode's read-reduce-write pattern over num_rows x heads states of 128 x 128
// fp32 in pool [num_slots, heads, 128, 128], row b's states at slots[b] (device int32;
// a slot outside [0, num_slots) is skipped).
int gdn_probe_state_rmw(float* pool, int num_slots, int heads, const int32_t* slots, int num_rows,
                        hipStream_t stream) {
    if (!pool || !slots || heads <= 0 || num_rows < 0 || num_slots < 0 ||
        (int64_t)num_rows * heads > 0x7fffffffLL || reinterpret_cast<uintptr_t>(pool) % 16 != 0)
        return (int)hipErrorInvalidValue;
    if (num_rows == 0) return (int)hipSuccess;
    hipLaunchKernelGGL(state_rmw_kernel, dim3((unsigned)(num_rows * heads)), dim3(kRmwThreads), 0, stream, pool,
                       slots, heads, num_slots);
    return (int)hipGetLastError();
}

}  // extern "C"
