// gdn_prefill.hip -- chunked prefill of the gated delta rule for gfx950 (MI355X).
//
// Defined by: "[Model] Enable batch-invariant mixed decode and prefill for Qwen GDN",
// section "Why" (fresh prefill rows go through a 64-token chunk prefill);
// "[V1][Hybrid] GatedDeltaNet Automatic Prefix Caching", section "Purpose" (states at
// chunk boundaries returned as one flat stream); "[WIP][Kernel] Enable GDN
// batch-invariant prefix caching", section "Purpose" (one lcm(64, block) grid).
//
// Within a chunk of L <= 64 tokens (rows r, s) with start state S0 (d_k x d_v) the
// token recurrence S <- e^g (I - beta k k^T) S + beta k v^T is evaluated in the
// chunked WY/UT form:
//     G   = inclusive cumsum of g inside the chunk,  gamma = e^G
//     A   = strictly lower part of diag(beta) (K K^T) o D,   D[r][s] = e^(G_r - G_s)
//     T   = (I + A)^-1
//     U~  = (T diag(beta)) V,   W = (T diag(beta gamma)) K,   U = U~ - W S0
//     O   = scale (diag(gamma) Q S0 + (Q K^T o D o lower-incl-diagonal) U)
//     S1  = gamma_last S0 + K^T (diag(e^(G_last - G)) U)
// Three kernels:
//   prep_kernel   one workgroup: per-sequence chunk counts on the absolute 64-token
//                 grid, their prefix sum, and the chunk table (sequence, first token,
//                 length).
//   tsolve_kernel one wave per (chunk, value head), all chunks at once: K K^T on
//                 MFMA, the decay mask, and T by forward substitution in fp32 (lane j
//                 owns column j).  T goes to the workspace in fp32.
//   chain_kernel  one workgroup per (sequence, value head): the chunks of a sequence
//                 in order.  Each wave owns a 32-column strip of d_v and keeps its
//                 part of S in MFMA accumulator registers (fp32) for the whole
//                 sequence; every product is an MFMA with fp32 accumulation.  The
//                 d_v columns of S, U and O are independent, so the strips never
//                 exchange data; shared operands (W, P, K, Q, T) go through LDS.
// Precision.  For bf16 inputs the MFMAs are 16x16x32 bf16.  q, k and v are exact in
// bf16; the derived operands that carry most of the rounding error -- T (folded with
// beta or beta gamma) and U (folded with the decay) -- enter as a hi + lo pair of
// bf16 values (x = hi + lo to about 2^-17), i.e. two MFMAs against the exact
// operand.  W, P and S enter as single bf16 values.  For fp32 inputs the MFMAs are
// 16x16x4 fp32 and nothing is split.  States, accumulators, gates and T's solve
// are fp32.  A sequence's work never depends on the other sequences of the call, so
// its results are bitwise independent of its batch-mates.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kC = 64;   // chunk length

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- MFMA traits
//
// 16x16 output tiles.  Lane l holds A[l % 16][k...] and B[k...][l % 16]; the C/D tile
// is held as C[4 (l / 16) + i][l % 16], i = 0..3.  Which k a lane element stands for
// only has to agree between A and B, so two k orders are used:
//   natural   element e of lane group g is k = KSTEP*ks + (bf16: 8g + e; fp32: g)
//   from-C    the order in which a C tile's registers already sit, so that an fp32
//             accumulator tile can feed the next MFMA as its B operand without an
//             LDS round trip: bf16 step ks covers rows 32ks..32ks+31 with element e<4
//             = row 32ks + 4g + e and e>=4 = row 32ks + 16 + 4g + (e-4); fp32 step
//             ks is register (ks & 3) of C tile (ks >> 2), i.e. row 16(ks>>2) + 4g + (ks&3).
template <typename E>
struct Mma;

template <>
struct Mma<__bf16> {
    static constexpr int KSTEP = 32;
    typedef bf16x8 frag;
    struct pair { frag hi, lo; };

    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // A split, B exact: hi then lo
    static __device__ __forceinline__ f32x4 mma_sa(const pair& a, frag b, f32x4 c) {
        c = mma(a.hi, b, c);
        return mma(a.lo, b, c);
    }
    // A exact, B split: hi then lo
    static __device__ __forceinline__ f32x4 mma_sb(frag a, const pair& b, f32x4 c) {
        c = mma(a, b.hi, c);
        return mma(a, b.lo, c);
    }
    static __device__ __forceinline__ int nat(int ks, int g, int e) { return 32 * ks + 8 * g + e; }
    static __device__ __forceinline__ int fromc(int ks, int g, int e) {
        return 32 * ks + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
    }
    static __device__ __forceinline__ pair split(const float* x) {
        pair p;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const __bf16 h = (__bf16)x[e];
            p.hi[e] = h;
            p.lo[e] = (__bf16)(x[e] - (float)h);   // exact difference, rounded once
        }
        return p;
    }
    static __device__ __forceinline__ frag round(const float* x) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (__bf16)x[e];
        return f;
    }
    // natural fragment from a row-major LDS row
    static __device__ __forceinline__ frag row_nat(const __bf16* row, int ks, int g) {
        return *reinterpret_cast<const bf16x8*>(row + 32 * ks + 8 * g);
    }
    // from-C ordered fragment from a row-major LDS row
    static __device__ __forceinline__ frag row_fromc(const __bf16* row, int ks, int g) {
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 32 * ks + 4 * g);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 32 * ks + 16 + 4 * g);
        frag f;
        f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
        f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
        return f;
    }
    // natural fragment down a column of a row-major LDS matrix
    static __device__ __forceinline__ frag col_nat(const __bf16* m, int ld, int col, int ks, int g) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = m[nat(ks, g, e) * ld + col];
        return f;
    }
    // from-C ordered fragment down a column
    static __device__ __forceinline__ frag col_fromc(const __bf16* m, int ld, int col, int ks, int g) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = m[fromc(ks, g, e) * ld + col];
        return f;
    }
    // natural fragment of an fp32 LDS row scaled per k, split into hi + lo
    static __device__ __forceinline__ pair row_nat_scaled_split(const float* row, int ks, int g,
                                                                const float* scale) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = row[nat(ks, g, e)] * scale[nat(ks, g, e)];
        return split(x);
    }
    // B fragment (from-C order, step ks) out of 16-row accumulator tiles tiles[x * stride]
    static __device__ __forceinline__ frag acc_fromc(const f32x4* tiles, int ks, int stride) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = tiles[(2 * ks) * stride][i];
            x[4 + i] = tiles[(2 * ks + 1) * stride][i];
        }
        return round(x);
    }
    // the same, each row r scaled by scale[r] (or not, when scale is null), split
    static __device__ __forceinline__ pair acc_fromc_split(const f32x4* tiles, int ks, int stride, int g,
                                                           const float* scale) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = tiles[(2 * ks) * stride][i];
            x[4 + i] = tiles[(2 * ks + 1) * stride][i];
            if (scale) {
                x[i] *= scale[32 * ks + 4 * g + i];
                x[4 + i] *= scale[32 * ks + 16 + 4 * g + i];
            }
        }
        return split(x);
    }
};

template <>
struct Mma<float> {
    static constexpr int KSTEP = 4;
    typedef float frag;
    struct pair { float hi; };

    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mma_sa(const pair& a, frag b, f32x4 c) { return mma(a.hi, b, c); }
    static __device__ __forceinline__ f32x4 mma_sb(frag a, const pair& b, f32x4 c) { return mma(a, b.hi, c); }
    static __device__ __forceinline__ int nat(int ks, int g, int) { return 4 * ks + g; }
    static __device__ __forceinline__ int fromc(int ks, int g, int) { return 16 * (ks >> 2) + 4 * g + (ks & 3); }
    static __device__ __forceinline__ frag row_nat(const float* row, int ks, int g) { return row[nat(ks, g, 0)]; }
    static __device__ __forceinline__ frag row_fromc(const float* row, int ks, int g) { return row[fromc(ks, g, 0)]; }
    static __device__ __forceinline__ frag col_nat(const float* m, int ld, int col, int ks, int g) {
        return m[nat(ks, g, 0) * ld + col];
    }
    static __device__ __forceinline__ frag col_fromc(const float* m, int ld, int col, int ks, int g) {
        return m[fromc(ks, g, 0) * ld + col];
    }
    static __device__ __forceinline__ pair row_nat_scaled_split(const float* row, int ks, int g,
                                                                const float* scale) {
        return pair{row[nat(ks, g, 0)] * scale[nat(ks, g, 0)]};
    }
    static __device__ __forceinline__ frag acc_fromc(const f32x4* tiles, int ks, int stride) {
        return tiles[(ks >> 2) * stride][ks & 3];
    }
    static __device__ __forceinline__ pair acc_fromc_split(const f32x4* tiles, int ks, int stride, int g,
                                                           const float* scale) {
        float x = tiles[(ks >> 2) * stride][ks & 3];
        if (scale) x *= scale[fromc(ks, g, 0)];
        return pair{x};
    }
};

template <typename E>
struct Pad;   // LDS row padding in elements (keeps 16-byte row alignment, spreads banks)
template <>
struct Pad<__bf16> { static constexpr int value = 8; };
template <>
struct Pad<float> { static constexpr int value = 4; };

template <typename E>
struct Vec { static constexpr int N = 16 / sizeof(E); };   // elements per 16-byte vector

__device__ __forceinline__ void copy16(void* dst, const void* src) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}
__device__ __forceinline__ void zero16(void* dst) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------- prep kernel

// Chunks of sequence i lie on the absolute 64-token grid: with a = start_pos % 64,
// chunk c covers local tokens [max(0, 64c - a), min(L, 64(c+1) - a)).
__device__ __forceinline__ int seq_chunks(int L, int a) { return L > 0 ? (a + L + kC - 1) / kC : 0; }

// Token range of sequence i, clamped into [0, T] so that a malformed cu_seqlens can
// only give wrong results, never an access outside the tensors.
__device__ __forceinline__ void seq_range(const int32_t* cu, int i, int64_t T, int& lo, int& len) {
    int64_t b = cu[i], e = cu[i + 1];
    b = b < 0 ? 0 : (b > T ? T : b);
    e = e < b ? b : (e > T ? T : e);
    lo = (int)b;
    len = (int)(e - b);
}

__global__ __launch_bounds__(256) void prep_kernel(const int32_t* cu, const int32_t* start_pos, int N,
                                                   int64_t T, int nc_max, int4* table,
                                                   int32_t* seq_off) {
    __shared__ int scan[256];
    __shared__ int carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int i = base + tid;
        int n = 0, lo = 0, len = 0, a = 0;
        if (i < N) {
            seq_range(cu, i, T, lo, len);
            a = start_pos ? (start_pos[i] & (kC - 1)) : 0;
            n = seq_chunks(len, a);
        }
        scan[tid] = n;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {   // inclusive Hillis-Steele scan
            const int t = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += t;
            __syncthreads();
        }
        const int first = carry + scan[tid] - n;
        if (i < N) {
            seq_off[i] = first;
            for (int c = 0; c < n; ++c) {
                const int idx = first + c;
                if (idx >= nc_max) break;
                const int b0 = c * kC - a < 0 ? 0 : c * kC - a;
                const int e0 = (c + 1) * kC - a > len ? len : (c + 1) * kC - a;
                table[idx] = make_int4(i, lo + b0, e0 - b0, c);
            }
        }
        __syncthreads();
        if (tid == 255) carry += scan[255];
        __syncthreads();
    }
    if (tid == 0) seq_off[N] = carry;
}

// ---------------------------------------------------------------- gates and T = (I + A)^-1

// Per (chunk, value head) gate vectors written by the transform and read by the scan.
constexpr int kGates = 5;
enum { GATE_G = 0, GATE_GAM = 1, GATE_BET = 2, GATE_BG = 3, GATE_KDEC = 4 };

// Inclusive prefix sum over the 64 lanes of a wave (Hillis-Steele, fixed order).
__device__ __forceinline__ float wave_inclusive_sum(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// One wave per (chunk, value head).  Writes the chunk's gate vectors (G, e^G, beta,
// beta e^G, e^(G_last - G)) and T = (I + A)^-1 in fp32.  T is formed blockwise: the
// four 16x16 diagonal blocks by forward substitution (lane 16b + j owns column j of
// block b), then the off-diagonal blocks column block by column block,
//     T_ij = -T_ii sum_{k=j..i-1} A_ik T_kj,
// on fp32 MFMA, each T_ij overwriting A_ij (whose last use it is).
template <typename E, int DK>
__global__ __launch_bounds__(64) void tsolve_kernel(PrefillArgs a, const int4* table,
                                                     const int32_t* seq_off, int nc_max, float* tws,
                                                     float* gws) {
    using M = Mma<E>;
    constexpr int KLD = DK + Pad<E>::value;
    constexpr int ALD = kC + 4;
    constexpr int KBYTES = kC * KLD * (int)sizeof(E);
    constexpr int ABYTES = kC * ALD * (int)sizeof(float);
    // one buffer holds K while K K^T is formed, then A, then T (in place)
    __shared__ __attribute__((aligned(16))) char buf[KBYTES > ABYTES ? KBYTES : ABYTES];
    __shared__ float Gs[kC], bl[kC];
    E* ks = reinterpret_cast<E*>(buf);
    float* as = reinterpret_cast<float*>(buf);

    const int c = blockIdx.x;
    const int h = blockIdx.y;
    const int total = min(seq_off[a.num_seqs], nc_max);
    if (c >= total) return;
    const int4 ent = table[c];
    const int tok = ent.y, L = ent.z;
    const int kh = h / (a.H_v / a.H_k);
    const int lane = threadIdx.x;
    const int li = lane & 15, g4 = lane >> 4;

    // K rows of the chunk -> LDS (zero past L)
    constexpr int VPR = DK / Vec<E>::N;
    const E* kg = static_cast<const E*>(a.k);
    for (int idx = lane; idx < kC * VPR; idx += 64) {
        const int r = idx / VPR, vi = idx - r * VPR;
        E* dst = ks + r * KLD + vi * Vec<E>::N;
        if (r < L) copy16(dst, kg + ((size_t)(tok + r) * a.H_k + kh) * DK + vi * Vec<E>::N);
        else zero16(dst);
    }
    // gates: lane s holds token s (g = beta = 0 past L, so G is flat there)
    const float gs = lane < L ? a.g[(size_t)(tok + lane) * a.H_v + h] : 0.f;
    const float bs = lane < L ? a.beta[(size_t)(tok + lane) * a.H_v + h] : 0.f;
    const float G = wave_inclusive_sum(gs, lane);
    const float G_last = __shfl(G, kC - 1, 64);
    const float gam = expf(G);
    float* gout = gws + ((size_t)c * a.H_v + h) * (kGates * kC);
    gout[GATE_G * kC + lane] = G;
    gout[GATE_GAM * kC + lane] = gam;
    gout[GATE_BET * kC + lane] = bs;
    gout[GATE_BG * kC + lane] = bs * gam;
    gout[GATE_KDEC * kC + lane] = expf(G_last - G);
    Gs[lane] = G;
    bl[lane] = bs;
    __syncthreads();

    // K K^T for the 10 lower 16x16 tiles, kept in registers (products of exact inputs)
    f32x4 kk_t[10];
    {
        int t = 0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt <= mt; ++nt, ++t) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
                for (int kk = 0; kk < DK / M::KSTEP; ++kk)
                    acc = M::mma(M::row_nat(ks + (16 * mt + li) * KLD, kk, g4),
                                 M::row_nat(ks + (16 * nt + li) * KLD, kk, g4), acc);
                kk_t[t] = acc;
            }
    }
    __syncthreads();   // K no longer needed: the buffer becomes A
    for (int idx = lane; idx < kC * ALD; idx += 64) as[idx] = 0.f;
    __syncthreads();
    {
        int t = 0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt <= mt; ++nt, ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + 4 * g4 + i, s = 16 * nt + li;
                    if (s < r) as[r * ALD + s] = bl[r] * kk_t[t][i] * expf(Gs[r] - Gs[s]);
                }
    }
    __syncthreads();

    // diagonal blocks: lane (b, j) forms column j of (I + A_bb)^-1
    {
        const int b = g4, j = li;
        const float* Ab = as + (16 * b) * ALD + 16 * b;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s) acc = fmaf(-Ab[r * ALD + s], t[s], acc);
            t[r] = r < j ? 0.f : (r == j ? 1.f : acc);
        }
        __syncthreads();
        float* Tb = as + (16 * b) * ALD + 16 * b;
#pragma unroll
        for (int r = 0; r < 16; ++r) Tb[r * ALD + j] = t[r];
    }
    __syncthreads();

    // off-diagonal blocks on fp32 MFMA (16x16x4): X = sum_k A_ik T_kj, then T_ij = -T_ii X
#pragma unroll
    for (int jb = 0; jb < 3; ++jb) {
#pragma unroll
        for (int ib = jb + 1; ib < 4; ++ib) {
            f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = jb; kb < ib; ++kb)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    X = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        as[(16 * ib + li) * ALD + 16 * kb + 4 * q + g4],     // A_ik[m][4q + g]
                        as[(16 * kb + 4 * q + g4) * ALD + 16 * jb + li],     // T_kj[4q + g][n]
                        X, 0, 0, 0);
            f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q)   // B from X's registers: element q is row 4g + q
                Y = __builtin_amdgcn_mfma_f32_16x16x4f32(as[(16 * ib + li) * ALD + 16 * ib + 4 * g4 + q], X[q],
                                                         Y, 0, 0, 0);
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i) as[(16 * ib + 4 * g4 + i) * ALD + 16 * jb + li] = -Y[i];
            __syncthreads();
        }
    }

    float* out = tws + ((size_t)c * a.H_v + h) * (kC * kC);
    for (int idx = lane; idx < kC * kC / 4; idx += 64) {
        const int r = idx >> 4, s4 = (idx & 15) * 4;
        *reinterpret_cast<float4*>(out + r * kC + s4) = *reinterpret_cast<const float4*>(as + r * ALD + s4);
    }
}

// ---------------------------------------------------------------- the chunk chain

template <typename E, int DK, int DV>
struct ChainSmem {
    static constexpr int QLD = DK + Pad<E>::value;      // Q rows
    static constexpr int TTLD = kC + Pad<E>::value;     // K^T rows (one per d_k index, tokens along)
    static constexpr int VLD = DV + Pad<E>::value;      // V rows
    static constexpr int WLD = DK + Pad<E>::value;      // -W rows
    static constexpr int TLD = kC + 4;                  // fp32 T rows
    static constexpr int PLD = kC + Pad<E>::value;      // P rows
    E q[kC * QLD];
    E kt[DK * TTLD];
    union {
        E v[kC * VLD];    // V (until U~ is formed)
        E w[kC * WLD];    // then -W
    };
    float t[kC * TLD];
    E p[kC * PLD];
    float gate[kGates * kC];
};

// smallest k index that step ks of each order covers
template <typename M>
__device__ __forceinline__ int kmin_nat(int ks) { return ks * M::KSTEP; }
template <typename M>
__device__ __forceinline__ int kmin_fromc(int ks) { return M::KSTEP == 32 ? 32 * ks : 16 * (ks >> 2); }

template <typename E, int DK, int DV>
__global__ __launch_bounds__(DV * 2) __attribute__((amdgpu_waves_per_eu(2)))
void chain_kernel(PrefillArgs a, const int4* table, const int32_t* seq_off, int nc_max, const float* tws,
                  const float* gws) {
    using M = Mma<E>;
    using S = ChainSmem<E, DK, DV>;
    constexpr int NW = DV / 32;            // waves; wave w owns columns [32w, 32w + 32)
    constexpr int NT = NW * 64;            // threads
    constexpr int MT_S = DK / 16;          // 16-row tiles of the state
    constexpr int KS_DK = DK / M::KSTEP;   // k steps over d_k
    constexpr int KS_C = kC / M::KSTEP;    // k steps over the chunk
    constexpr int VN = Vec<E>::N;
    __shared__ __attribute__((aligned(16))) S sm;

    const int seq = blockIdx.x / a.H_v;
    const int h = blockIdx.x - seq * a.H_v;
    const int kh = h / (a.H_v / a.H_k);
    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    const int lane = tid & 63;
    const int li = lane & 15, g4 = lane >> 4;
    const int col0 = 32 * wv;
    const float* bet = sm.gate + GATE_BET * kC;
    const float* bg = sm.gate + GATE_BG * kC;
    const float* gam = sm.gate + GATE_GAM * kC;
    const float* Gv = sm.gate + GATE_G * kC;
    const float* kdec = sm.gate + GATE_KDEC * kC;

    const size_t SE = (size_t)DK * DV;
    // state strip in accumulator layout: Sacc[mt][nt] holds S[16mt + 4g + i][col0 + 16nt + li]
    f32x4 Sacc[MT_S][2];
    const int isl = a.init_slot ? a.init_slot[seq] : -1;
    if (isl >= 0 && isl < a.num_slots) {
        const float* src = a.pool + ((size_t)isl * a.H_v + h) * SE;
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sacc[mt][nt][i] = src[(size_t)(16 * mt + 4 * g4 + i) * DV + col0 + 16 * nt + li];
    } else {
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) Sacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int total = min(seq_off[a.num_seqs], nc_max);
    const int c_begin = min(seq_off[seq], total);
    const int c_end = min(seq_off[seq + 1], total);
    const int64_t pos0 = a.start_pos ? a.start_pos[seq] : 0;
    int seq_tok0 = 0;
    if (c_begin < c_end) seq_tok0 = table[c_begin].y;

    const E* qg = static_cast<const E*>(a.q);
    const E* kg = static_cast<const E*>(a.k);
    const E* vg = static_cast<const E*>(a.v);
    E* og = static_cast<E*>(a.o);

    for (int c = c_begin; c < c_end; ++c) {
        const int4 ent = table[c];
        const int tok = ent.y, L = ent.z;
        __syncthreads();   // the previous chunk is done with LDS

        // ---- loads: Q rows, K transposed, V rows, T, gates
        for (int idx = tid; idx < kC * (DK / VN); idx += NT) {
            const int r = idx / (DK / VN), d0 = (idx - r * (DK / VN)) * VN;
            E* dq = sm.q + r * S::QLD + d0;
            if (r < L) copy16(dq, qg + ((size_t)(tok + r) * a.H_k + kh) * DK + d0);
            else zero16(dq);
        }
        // K: consecutive threads take consecutive tokens, so the transposed LDS writes
        // of a wave fall in consecutive addresses
        for (int idx = tid; idx < kC * (DK / VN); idx += NT) {
            const int r = idx & (kC - 1), d0 = (idx >> 6) * VN;
            E kv[VN];
            if (r < L) {
                *reinterpret_cast<uint4*>(kv) =
                    *reinterpret_cast<const uint4*>(kg + ((size_t)(tok + r) * a.H_k + kh) * DK + d0);
            } else {
                *reinterpret_cast<uint4*>(kv) = make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int e = 0; e < VN; ++e) sm.kt[(d0 + e) * S::TTLD + r] = kv[e];
        }
        for (int idx = tid; idx < kC * (DV / VN); idx += NT) {
            const int r = idx / (DV / VN), vi = idx - r * (DV / VN);
            E* dv = sm.v + r * S::VLD + vi * VN;
            if (r < L) copy16(dv, vg + ((size_t)(tok + r) * a.H_v + h) * DV + vi * VN);
            else zero16(dv);
        }
        {
            const float* tsrc = tws + ((size_t)c * a.H_v + h) * (kC * kC);
            for (int idx = tid; idx < kC * kC / 4; idx += NT) {
                const int r = idx >> 4, s4 = (idx & 15) * 4;
                copy16(sm.t + r * S::TLD + s4, tsrc + r * kC + s4);
            }
            const float* gsrc = gws + ((size_t)c * a.H_v + h) * (kGates * kC);
            for (int idx = tid; idx < kGates * kC / 4; idx += NT) copy16(sm.gate + 4 * idx, gsrc + 4 * idx);
        }
        __syncthreads();

        // ---- phase A1: U~ = (T diag(beta)) V for this wave's strip (T is lower triangular:
        //      steps wholly above the diagonal are skipped)
        f32x4 Uacc[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            Uacc[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            Uacc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS_C; ++kk) {
                if (kmin_nat<M>(kk) > 16 * mt + 15) continue;
                const typename M::pair ta = M::row_nat_scaled_split(sm.t + (16 * mt + li) * S::TLD, kk, g4, bet);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    Uacc[mt][nt] = M::mma_sa(ta, M::col_nat(sm.v, S::VLD, col0 + 16 * nt + li, kk, g4),
                                             Uacc[mt][nt]);
            }
        }
        __syncthreads();   // V is dead: its space takes -W

        // ---- phase A2 + B (shared, split over the waves):
        //      -W = -(T diag(beta gamma)) K  and  P = (Q K^T) o D o lower-incl-diagonal
        for (int t = wv; t < 4 * (DK / 16); t += NW) {
            const int mt = t / (DK / 16), nt = t - mt * (DK / 16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS_C; ++kk) {
                if (kmin_nat<M>(kk) > 16 * mt + 15) continue;
                acc = M::mma_sa(M::row_nat_scaled_split(sm.t + (16 * mt + li) * S::TLD, kk, g4, bg),
                                M::row_nat(sm.kt + (16 * nt + li) * S::TTLD, kk, g4), acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sm.w[(16 * mt + 4 * g4 + i) * S::WLD + 16 * nt + li] = (E)(-acc[i]);
        }
        for (int t = wv; t < 16; t += NW) {
            const int mt = t >> 2, nt = t & 3;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (nt <= mt) {
#pragma unroll 4
                for (int kk = 0; kk < KS_DK; ++kk)
                    acc = M::mma(M::row_nat(sm.q + (16 * mt + li) * S::QLD, kk, g4),
                                 M::col_nat(sm.kt, S::TTLD, 16 * nt + li, kk, g4), acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * g4 + i, s = 16 * nt + li;
                const float val = s <= r ? acc[i] * expf(Gv[r] - Gv[s]) : 0.f;
                sm.p[r * S::PLD + s] = (E)val;
            }
        }
        __syncthreads();

        // ---- phase C: U = U~ + (-W) S
#pragma unroll
        for (int kk = 0; kk < KS_DK; ++kk) {
            const typename M::frag sb0 = M::acc_fromc(&Sacc[0][0], kk, 2);
            const typename M::frag sb1 = M::acc_fromc(&Sacc[0][1], kk, 2);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const typename M::frag wa = M::row_fromc(sm.w + (16 * mt + li) * S::WLD, kk, g4);
                Uacc[mt][0] = M::mma(wa, sb0, Uacc[mt][0]);
                Uacc[mt][1] = M::mma(wa, sb1, Uacc[mt][1]);
            }
        }

        // ---- phase D: O = gamma o (Q S) + P U, one 16-column tile at a time
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x4 Oacc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) Oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS_DK; ++kk) {
                const typename M::frag sb = M::acc_fromc(&Sacc[0][nt], kk, 2);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    Oacc[mt] = M::mma(M::row_fromc(sm.q + (16 * mt + li) * S::QLD, kk, g4), sb, Oacc[mt]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) Oacc[mt][i] *= gam[16 * mt + 4 * g4 + i];
#pragma unroll
            for (int kk = 0; kk < KS_C; ++kk) {
                const typename M::pair ub = M::acc_fromc_split(&Uacc[0][nt], kk, 2, g4, nullptr);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (kmin_fromc<M>(kk) > 16 * mt + 15) continue;
                    Oacc[mt] = M::mma_sb(M::row_fromc(sm.p + (16 * mt + li) * S::PLD, kk, g4), ub, Oacc[mt]);
                }
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + 4 * g4 + i;
                    if (r < L)
                        og[((size_t)(tok + r) * a.H_v + h) * DV + col0 + 16 * nt + li] = (E)(a.scale * Oacc[mt][i]);
                }
        }

        // ---- phase E: S = gamma_last S + K^T (diag(e^(G_last - G)) U)
        const float gl_last = gam[kC - 1];
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Sacc[mt][0][i] *= gl_last;
                Sacc[mt][1][i] *= gl_last;
            }
#pragma unroll
        for (int kk = 0; kk < KS_C; ++kk) {
            const typename M::pair ub0 = M::acc_fromc_split(&Uacc[0][0], kk, 2, g4, kdec);
            const typename M::pair ub1 = M::acc_fromc_split(&Uacc[0][1], kk, 2, g4, kdec);
#pragma unroll
            for (int mt = 0; mt < MT_S; ++mt) {
                const typename M::frag ka = M::row_fromc(sm.kt + (16 * mt + li) * S::TTLD, kk, g4);
                Sacc[mt][0] = M::mma_sb(ka, ub0, Sacc[mt][0]);
                Sacc[mt][1] = M::mma_sb(ka, ub1, Sacc[mt][1]);
            }
        }

        // ---- export on the grid
        if (a.export_grid > 0) {
            const int64_t p_end = pos0 + (tok + L - seq_tok0);
            if (p_end % a.export_grid == 0) {
                const int64_t m = p_end / a.export_grid - pos0 / a.export_grid - 1;
                const int64_t idx = (int64_t)a.export_offsets[seq] + m;
                if (idx >= 0 && idx < a.export_capacity) {
                    float* dst = a.export_states + ((size_t)idx * a.H_v + h) * SE;
#pragma unroll
                    for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                dst[(size_t)(16 * mt + 4 * g4 + i) * DV + col0 + 16 * nt + li] = Sacc[mt][nt][i];
                }
            }
        }
    }

    const int fsl = a.final_slot ? a.final_slot[seq] : -1;
    if (fsl >= 0 && fsl < a.num_slots) {
        float* dst = a.pool + ((size_t)fsl * a.H_v + h) * SE;
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[(size_t)(16 * mt + 4 * g4 + i) * DV + col0 + 16 * nt + li] = Sacc[mt][nt][i];
    }
}

// ---------------------------------------------------------------- workspace layout

struct Layout {
    size_t table, seq_off, tws, gws, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(int H_v, int num_seqs, int64_t total_tokens) {
    const int64_t nc = max_chunks(num_seqs, total_tokens);
    Layout l;
    l.table = 0;
    l.seq_off = align256(l.table + (size_t)nc * sizeof(int4));
    l.tws = align256(l.seq_off + (size_t)(num_seqs + 1) * sizeof(int32_t));
    l.gws = align256(l.tws + (size_t)nc * H_v * kC * kC * sizeof(float));
    l.total = align256(l.gws + (size_t)nc * H_v * kGates * kC * sizeof(float));
    return l;
}

// stage bit 1: prep + tsolve (fills the workspace); stage bit 2: the chunk chain
template <typename E, int DK, int DV>
hipError_t launch_typed(const PrefillArgs& a, int stages, hipStream_t stream) {
    const Layout l = layout(a.H_v, a.num_seqs, a.total_tokens);
    char* ws = static_cast<char*>(a.workspace);
    int4* table = reinterpret_cast<int4*>(ws + l.table);
    int32_t* seq_off = reinterpret_cast<int32_t*>(ws + l.seq_off);
    float* tws = reinterpret_cast<float*>(ws + l.tws);
    float* gws = reinterpret_cast<float*>(ws + l.gws);
    const int nc_max = (int)max_chunks(a.num_seqs, a.total_tokens);

    if (stages & 1) {
        hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens, a.start_pos,
                           a.num_seqs, a.total_tokens, nc_max, table, seq_off);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL((tsolve_kernel<E, DK>), dim3(nc_max, a.H_v), dim3(64), 0, stream, a, table,
                           seq_off, nc_max, tws, gws);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (stages & 2) {
        hipLaunchKernelGGL((chain_kernel<E, DK, DV>), dim3(a.num_seqs * a.H_v), dim3(DV * 2), 0, stream,
                           a, table, seq_off, nc_max, tws, gws);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename E>
hipError_t launch_dims(const PrefillArgs& a, int stages, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_typed<E, 128, 128>(a, stages, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_typed<E, 128, 64>(a, stages, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_typed<E, 64, 128>(a, stages, stream);
    return launch_typed<E, 64, 64>(a, stages, stream);
}

}  // namespace

int64_t max_chunks(int num_seqs, int64_t total_tokens) {
    // each sequence adds at most one partial chunk at each end
    return (total_tokens + kC - 1) / kC + 2 * (int64_t)num_seqs;
}

size_t prefill_workspace_bytes(int H_v, int dtype, int num_seqs, int64_t total_tokens) {
    (void)dtype;
    return layout(H_v, num_seqs, total_tokens).total;
}

hipError_t launch_prefill(const PrefillArgs& a, int stages, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.dtype == 1) return launch_dims<__bf16>(a, stages, stream);
    return launch_dims<float>(a, stages, stream);
}

}  // namespace gdn
