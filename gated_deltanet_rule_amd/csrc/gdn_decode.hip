// gdn_decode.hip -- packed recurrent decode for gfx950 (MI355X).
//
// A workgroup of 256 threads advances 64 value columns of the state of one (row, value
// head) by one token ("[Model] Enable batch-invariant mixed decode and prefill for Qwen GDN",
// sections "Why" and "How": cached rows take the packed recurrent decode path), or by
// tokens_per_row tokens in order for a multi-token verify row: the state stays in
// registers between the row's tokens and is written after each token to that token's
// slot.  The work is bound by HBM: each state (d_k x d_v fp32, 64 KiB at d = 128) is
// read once and written once per kept token, so the kernel streams it with 16-byte
// coalesced loads into registers, does the whole update there, and streams it back:
//
//     S <- exp(g) S;   u = beta (v - S^T k);   S <- S + k u^T;   o = scale S^T q
//
// The value columns of S, u and o are independent (both reductions run over d_k), so a
// state is split by columns over d_v / 64 workgroups.  Thread layout: a state row's 64
// columns are covered by 16 threads holding one float4 each; the 256 threads form 16
// row groups, and row group r holds rows r, r + 16, r + 32, ...  Small workgroups (32
// KiB of state each, eight to a compute unit) start and finish one by one, so loads
// and stores of different workgroups stay interleaved; one workgroup of 1024 threads
// per 64 KiB state ran 2-3 % slower.  The two reductions over d_k (S^T k and S^T q)
// are per-thread partial sums followed by a fixed-order sum over the row groups through
// LDS, so the result does not depend on anything but the row's own data: a row's
// output and state are bitwise the same in any batch, at any position, and a verify
// row equals the same tokens decoded one call at a time.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

template <typename T>
__device__ __forceinline__ float4 load4(const T* p);

template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}

template <>
__device__ __forceinline__ float4 load4<__bf16>(const __bf16* p) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v);

template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) {
    *reinterpret_cast<float4*>(p) = v;
}

template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, float4 v) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 x;
    x[0] = (__bf16)v.x;   // round to nearest even (v_cvt_pk_bf16_f32)
    x[1] = (__bf16)v.y;
    x[2] = (__bf16)v.z;
    x[3] = (__bf16)v.w;
    *reinterpret_cast<bf16x4*>(p) = x;
}

constexpr int kThreads = 256;
constexpr int kCols = 64;            // value columns per workgroup

// State traffic is touched once per call: stream it with non-temporal loads and
// stores so it neither evicts nor waits on cache lines other work could reuse.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_state(const float* p) {
    const f32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store_state(float* p, float4 v) {
    const f32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4_t*>(p));
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    constexpr int TPR = kCols / 4;       // threads per state row slice
    constexpr int RG = kThreads / TPR;   // row groups
    constexpr int R = DK / RG;           // rows per thread
    constexpr int NCW = DV / kCols;      // workgroups per (row, head)
    static_assert(R * RG == DK && TPR * RG == kThreads && NCW * kCols == DV && 2 * DK <= kThreads,
                  "bad decode tiling");

    const int unit = blockIdx.x / NCW;
    const int col0 = kCols * (blockIdx.x - unit * NCW);
    const int b = unit / a.H_v;
    const int h = unit - b * a.H_v;
    const int kh = h / (a.H_v / a.H_k);
    const int tid = threadIdx.x;
    const int c4 = tid % TPR;
    const int rg = tid / TPR;
    const int NTOK = a.tokens_per_row;

    const int sin = a.slot_in[b];
    if (sin < 0 || sin >= a.num_slots) {          // padding row
        for (int t = 0; t < NTOK; ++t) {
            T* o = static_cast<T*>(a.o) + ((size_t)(b * NTOK + t) * a.H_v + h) * DV;
            if (tid < kCols) o[col0 + tid] = from_f32<T>(0.f);
        }
        return;
    }

    // Issue the state loads first: they are the only large transfer.
    const float* src = a.pool + ((size_t)sin * a.H_v + h) * (size_t)(DK * DV);
    float4 s[R];
#pragma unroll
    for (int m = 0; m < R; ++m)
        s[m] = load_state(src + (size_t)(rg + RG * m) * DV + col0 + 4 * c4);

    __shared__ float kq[2][DK];
    __shared__ float4 red[2][RG][TPR];
    // The row's tokens in order, the state kept in registers between them.  Every
    // LDS array is rewritten only after the barrier that follows its last read.
    for (int t = 0; t < NTOK; ++t) {
        const size_t row = (size_t)b * NTOK + t;
        T* o = static_cast<T*>(a.o) + (row * a.H_v + h) * DV;
        const T* kp = static_cast<const T*>(a.k) + (row * a.H_k + kh) * DK;
        const T* qp = static_cast<const T*>(a.q) + (row * a.H_k + kh) * DK;
        if (tid < DK) kq[0][tid] = to_f32(kp[tid]);
        else if (tid < 2 * DK) kq[1][tid - DK] = to_f32(qp[tid - DK]);
        const float4 vv = load4<T>(static_cast<const T*>(a.v) + row * a.H_v * DV + (size_t)h * DV + col0 + 4 * c4);
        const float alpha = expf(a.g[row * a.H_v + h]);
        const float beta = a.beta[row * a.H_v + h];
        __syncthreads();

        // decay, then the partial prediction S^T k over this thread's rows
        float4 p = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int m = 0; m < R; ++m) {
            s[m].x *= alpha; s[m].y *= alpha; s[m].z *= alpha; s[m].w *= alpha;
            const float kr = kq[0][rg + RG * m];
            p.x = fmaf(s[m].x, kr, p.x); p.y = fmaf(s[m].y, kr, p.y);
            p.z = fmaf(s[m].z, kr, p.z); p.w = fmaf(s[m].w, kr, p.w);
        }
        red[0][rg][c4] = p;
        __syncthreads();
        float4 tot = red[0][0][c4];
#pragma unroll
        for (int r = 1; r < RG; ++r) {
            const float4 x = red[0][r][c4];
            tot.x += x.x; tot.y += x.y; tot.z += x.z; tot.w += x.w;
        }
        const float4 u = make_float4(beta * (vv.x - tot.x), beta * (vv.y - tot.y),
                                     beta * (vv.z - tot.z), beta * (vv.w - tot.w));

        // rank-1 write, then the partial read S^T q from the updated state
        float4 po = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const float kr = kq[0][rg + RG * m];
            const float qr = kq[1][rg + RG * m];
            s[m].x = fmaf(kr, u.x, s[m].x); s[m].y = fmaf(kr, u.y, s[m].y);
            s[m].z = fmaf(kr, u.z, s[m].z); s[m].w = fmaf(kr, u.w, s[m].w);
            po.x = fmaf(s[m].x, qr, po.x); po.y = fmaf(s[m].y, qr, po.y);
            po.z = fmaf(s[m].z, qr, po.z); po.w = fmaf(s[m].w, qr, po.w);
        }
        const int sout = a.slot_out[row];
        if (sout >= 0 && sout < a.num_slots) {
            float* dst = a.pool + ((size_t)sout * a.H_v + h) * (size_t)(DK * DV);
#pragma unroll
            for (int m = 0; m < R; ++m)
                store_state(dst + (size_t)(rg + RG * m) * DV + col0 + 4 * c4, s[m]);
        }
        red[1][rg][c4] = po;
        __syncthreads();
        if (rg == 0) {
            float4 to = red[1][0][c4];
#pragma unroll
            for (int r = 1; r < RG; ++r) {
                const float4 x = red[1][r][c4];
                to.x += x.x; to.y += x.y; to.z += x.z; to.w += x.w;
            }
            const float sc = a.scale;
            store4<T>(o + col0 + 4 * c4, make_float4(sc * to.x, sc * to.y, sc * to.z, sc * to.w));
        }
    }
}

template <typename T, int DK, int DV>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    const unsigned blocks = (unsigned)a.num_rows * (unsigned)a.H_v * (unsigned)(DV / kCols);
    hipLaunchKernelGGL((decode_kernel<T, DK, DV>), dim3(blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dims(const DecodeArgs& a, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_typed<T, 128, 128>(a, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_typed<T, 128, 64>(a, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_typed<T, 64, 128>(a, stream);
    return launch_typed<T, 64, 64>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.num_rows == 0) return hipSuccess;
    if (a.dtype == 1) return launch_dims<__bf16>(a, stream);
    return launch_dims<float>(a, stream);
}

}  // namespace gdn
