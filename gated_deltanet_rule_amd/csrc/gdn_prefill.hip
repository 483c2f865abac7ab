// gdn_prefill.hip -- chunked prefill of the gated delta rule for fp32 inputs on gfx950
// (MI355X), and the prefill launcher, which sends bf16 inputs to the kernel in
// gdn_prefill_bf16.hip.
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
//     T1  = T diag(beta),   T2 = T diag(beta gamma)
//     U   = T1 V - T2 (K S0)                       (= U~ - W S0 with W = T2 K)
//     O   = scale (diag(gamma) Q S0 + (Q K^T o D o lower-incl-diagonal) U)
//     S1  = gamma_last S0 + K^T (diag(e^(G_last - G)) U)
//
// One kernel.  A workgroup owns one sequence and one value head and walks the
// sequence's chunks in order.  Per value head, d_v is split into 32-column
// strips, one wave each; a wave keeps its strip of S (d_k x 32, fp32) in MFMA
// accumulator registers for the whole sequence.  The d_v columns of S, U and O are
// independent, so strips never exchange data.  Per chunk:
//   load     Q and K rows from the registers they were
//            prefetched into during the previous chunk; V fragments likewise
//   phase 1  gates by a wave scan; K K^T and Q K^T (lower tiles) and Z = K S for
//            each strip, on MFMA
//   phase 2  A for each head into LDS (fp32)
//   phase 3  T = (I + A)^-1 in place, one wave per head: the 16x16 diagonal blocks by
//            forward substitution (lane 16b + j owns column j of block b), then
//            T_ij = -T_ii sum_{k=j..i-1} A_ik T_kj column block by column block on
//            fp32 MFMA, each T_ij overwriting A_ij (its last use)
//   phase 4  T1 and -T2, split once per chunk into LDS (all threads)
//   phase 5  P into LDS; U = T1 V + (-T2) Z; O = gamma o (Q S) + P U; the state
//            update; the grid export
// Precision.  The MFMAs are 16x16x4 fp32 and nothing is rounded below fp32: states,
// accumulators, gates and T's solve are fp32.  A sequence's work never
// depends on the other sequences of the call, so its results are bitwise
// independent of its batch-mates; the chunks lie on the absolute 64-token grid, so
// a resume from an exported grid state continues with the same arithmetic.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kC = 64;   // chunk length

typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- MFMA traits
//
// 16x16 output tiles.  Lane l holds A[l % 16][k...] and B[k...][l % 16]; the C/D tile
// is held as C[4 (l / 16) + i][l % 16], i = 0..3.  Which k a lane element stands for
// only has to agree between A and B, so two k orders are used (16x16x4 fp32, one
// element per lane and step):
//   natural   lane group g holds k = 4 ks + g
//   from-C    the order in which a C tile's registers already sit, so that an fp32
//             accumulator tile can feed the next MFMA as its B operand without an
//             LDS round trip: step ks is register (ks & 3) of C tile (ks >> 2), i.e.
//             row 16 (ks >> 2) + 4 g + (ks & 3).
template <typename E>
struct Mma;

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
struct Pad<float> { static constexpr int value = 4; };

template <typename E>
struct Vec { static constexpr int N = 16 / sizeof(E); };   // elements per 16-byte vector

__device__ __forceinline__ void copy16(void* dst, const void* src) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}
__device__ __forceinline__ void zero16(void* dst) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(0u, 0u, 0u, 0u);
}


// ---------------------------------------------------------------- chunk geometry

// Chunks of a sequence lie on the absolute 64-token grid: with a = start_pos % 64,
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

// Inclusive prefix sum over the 64 lanes of a wave (Hillis-Steele, fixed order).
__device__ __forceinline__ float wave_inclusive_sum(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

constexpr int kGates = 5;
enum { GATE_G = 0, GATE_GAM = 1, GATE_BET = 2, GATE_BG = 3, GATE_KDEC = 4 };

template <typename E>
struct NSplit { static constexpr int value = 2; };   // bf16: hi + lo
template <>
struct NSplit<float> { static constexpr int value = 1; };

template <typename E, int DK, int DV, int HG>
struct ScanSmem {
    static constexpr int QLD = DK + Pad<E>::value;      // Q and K rows
    static constexpr int ALD = kC + 4;                  // fp32 A / T rows
    static constexpr int TLD = kC + Pad<E>::value;      // T1, T2 rows (operand type)
    static constexpr int PLD = kC + Pad<E>::value;      // P rows
    static constexpr int VLD = DV + Pad<E>::value;      // V rows
    static constexpr int NS = NSplit<E>::value;
    E q[kC * QLD];
    E k[kC * QLD];
    struct Head {
        union {
            E v[kC * VLD];        // V rows (staging to phase 1)
            float a[kC * ALD];    // A, then T in place (phases 2-4)
            E p[kC * PLD];        // then P (phase 5)
        };
        E t1[NS][kC * TLD];       // T diag(beta), hi [+ lo]
        E t2[NS][kC * TLD];       // -T diag(beta gamma), hi [+ lo]
        float gate[kGates * kC];
        float graw[kC];
        float braw[kC];
    } hd[HG];
};

// store an fp32 value as the operand type (fp32: as it is; the lo part is unused)
template <typename E>
__device__ __forceinline__ void split_store(E* hi, E* lo, int idx, float x);
template <>
__device__ __forceinline__ void split_store<float>(float* hi, float*, int idx, float x) {
    hi[idx] = x;
}

template <typename E>
__device__ __forceinline__ typename Mma<E>::pair row_pair_nat(const E* hi, const E* lo, int ks, int g) {
    typename Mma<E>::pair p;
    p.hi = Mma<E>::row_nat(hi, ks, g);
    if constexpr (NSplit<E>::value == 2) p.lo = Mma<E>::row_nat(lo, ks, g);
    return p;
}
template <typename E>
__device__ __forceinline__ typename Mma<E>::pair row_pair_fromc(const E* hi, const E* lo, int ks, int g) {
    typename Mma<E>::pair p;
    p.hi = Mma<E>::row_fromc(hi, ks, g);
    if constexpr (NSplit<E>::value == 2) p.lo = Mma<E>::row_fromc(lo, ks, g);
    return p;
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for every
// outstanding global load (its release fence drains vmcnt), which would expose the
// latency of the next chunk's prefetch at the first barrier after it is issued.  The
// scan shares data between waves only through LDS, so waiting for LDS operations is
// enough; the memory clobber keeps the compiler from moving accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// smallest k index that step ks of each order covers
template <typename M>
__device__ __forceinline__ int kmin_nat(int ks) { return ks * M::KSTEP; }
template <typename M>
__device__ __forceinline__ int kmin_fromc(int ks) { return M::KSTEP == 32 ? 32 * ks : 16 * (ks >> 2); }

// ---------------------------------------------------------------- the scan kernel

template <typename E, int DK, int DV, int HG>
__global__ __launch_bounds__(HG * DV * 2) void scan_kernel(PrefillArgs a) {
    using M = Mma<E>;
    using SM = ScanSmem<E, DK, DV, HG>;
    constexpr int NWH = DV / 32;             // waves per value head
    constexpr int NW = HG * NWH;             // waves
    constexpr int NT = NW * 64;              // threads
    constexpr int MT_S = DK / 16;            // 16-row tiles of the state
    constexpr int KS_DK = DK / M::KSTEP;     // k steps over d_k
    constexpr int KS_C = kC / M::KSTEP;      // k steps over the chunk
    constexpr int VN = Vec<E>::N;            // elements per 16-byte vector
    constexpr int VPR = DK / VN;             // 16-byte vectors per Q/K row
    constexpr int NPF = 2 * kC * VPR / NT;   // prefetched Q/K vectors per thread
    constexpr int VPRV = DV / VN;            // 16-byte vectors per V row
    constexpr int NPV = HG * kC * VPRV / NT; // prefetched V vectors per thread
    constexpr int TPW = (16 + NW - 1) / NW;  // 16x16 tiles of a 64x64 matrix per wave
    constexpr int NVF = KS_C * 2;            // V fragments per wave
    static_assert(NPF * NT == 2 * kC * VPR, "Q/K prefetch must divide evenly");
    static_assert(NPV * NT == HG * kC * VPRV, "V prefetch must divide evenly");
    __shared__ __attribute__((aligned(16))) SM sm;

    const int G = a.H_v / a.H_k;
    const int GG = G / HG;
    const int seq = blockIdx.x / (a.H_k * GG);
    const int rem = blockIdx.x - seq * (a.H_k * GG);
    const int kh = rem / GG;
    const int h0 = kh * G + (rem - kh * GG) * HG;
    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    int lane = tid & 63;
    const int hh = wv / NWH;                 // this wave's head within the group
    const int h = h0 + hh;
    const int col0 = 32 * (wv - hh * NWH);
    typename SM::Head& hd = sm.hd[hh];

    const size_t SE = (size_t)DK * DV;
    // state strip in accumulator layout: Sacc[mt][nt] holds S[16mt + 4g + i][col0 + 16nt + li]
    f32x4 Sacc[MT_S][2];
    const int isl = a.init_slot ? a.init_slot[seq] : -1;
    if (isl >= 0 && isl < a.num_slots) {
        const int li = lane & 15, g4 = lane >> 4;
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

    int lo, len;
    seq_range(a.cu_seqlens, seq, a.total_tokens, lo, len);
    const int64_t pos0 = a.start_pos ? a.start_pos[seq] : 0;
    const int off64 = (int)(pos0 & (kC - 1));
    const int nchunks = seq_chunks(len, off64);

    const E* qg = static_cast<const E*>(a.q);
    const E* kg = static_cast<const E*>(a.k);
    const E* vg = static_cast<const E*>(a.v);
    E* og = static_cast<E*>(a.o);

    // ---- prefetch registers: Q/K row vectors, V row vectors, g/beta (16-byte vector
    //      loads that nothing consumes until the next chunk is staged)
    uint4 pf[NPF];
    uint4 pv[NPV];
    float gbpf = 0.f;
    auto chunk_bounds = [&](int c, int& tok, int& L, int& e0) {
        const int b0 = c * kC - off64 < 0 ? 0 : c * kC - off64;
        e0 = (c + 1) * kC - off64 > len ? len : (c + 1) * kC - off64;
        tok = lo + b0;
        L = e0 - b0;
    };
    // load 16 bytes at a uniform base plus an unsigned 32-bit byte offset (the
    // scalar-base + vector-offset form of the global load)
    auto ld16 = [](const void* base, uint32_t off) {
        return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + off);
    };
    auto prefetch = [&](int c, int t) {
        int tok, L, e0;
        chunk_bounds(c, tok, L, e0);
        const E* qb = qg + (size_t)tok * a.H_k * DK;
        const E* kb = kg + (size_t)tok * a.H_k * DK;
        const E* vb = vg + (size_t)tok * a.H_v * DV;
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int i = t + NT * j;
            const int which = i / (kC * VPR);            // 0: Q, 1: K
            const int r = (i / VPR) % kC, vi = i % VPR;
            const uint32_t off = (uint32_t)((r * a.H_k + kh) * DK + vi * VN) * (uint32_t)sizeof(E);
            pf[j] = r < L ? ld16(which == 0 ? qb : kb, off) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
            const int i = t + NT * j;
            const int hx = i / (kC * VPRV);
            const int r = (i / VPRV) % kC, vi = i % VPRV;
            const uint32_t off = (uint32_t)((r * a.H_v + h0 + hx) * DV + vi * VN) * (uint32_t)sizeof(E);
            pv[j] = r < L ? ld16(vb, off) : make_uint4(0u, 0u, 0u, 0u);
        }
        if (t < 2 * kC * HG) {                            // g then beta for each head
            const int hx = t / (2 * kC), which = (t / kC) & 1, s = t % kC;
            const float* src = (which == 0 ? a.g : a.beta) + (size_t)tok * a.H_v;
            const uint32_t off = (uint32_t)(s * a.H_v + h0 + hx) * 4u;
            gbpf = s < L ? *reinterpret_cast<const float*>(reinterpret_cast<const char*>(src) + off) : 0.f;
        }
    };
    if (nchunks > 0) prefetch(0, tid);

    for (int c = 0; c < nchunks; ++c) {
        int tok, L, e0;
        chunk_bounds(c, tok, L, e0);
        // Keep lane-derived addresses inside the loop: without this the compiler hoists
        // every unrolled access's address out of the chunk loop and runs out of registers.
        int tid_l = tid;
        asm volatile("" : "+v"(lane), "+v"(tid_l));
        const int li = lane & 15, g4 = lane >> 4;
        lds_barrier();   // the previous chunk is done with LDS

        // ---- stage this chunk's inputs; prefetch the next chunk
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int i = tid + NT * j;
            const int which = i / (kC * VPR);
            const int r = (i / VPR) % kC, vi = i % VPR;
            E* dst = (which == 0 ? sm.q : sm.k) + r * SM::QLD + vi * VN;
            *reinterpret_cast<uint4*>(dst) = pf[j];
        }
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
            const int i = tid + NT * j;
            const int hx = i / (kC * VPRV);
            const int r = (i / VPRV) % kC, vi = i % VPRV;
            *reinterpret_cast<uint4*>(sm.hd[hx].v + r * SM::VLD + vi * VN) = pv[j];
        }
        if (tid < 2 * kC * HG) {
            const int hx = tid / (2 * kC), which = (tid / kC) & 1, s = tid % kC;
            (which == 0 ? sm.hd[hx].graw : sm.hd[hx].braw)[s] = gbpf;
        }
        lds_barrier();
        // the staged inputs are in LDS: fetch the next chunk's behind this chunk's compute
        if (c + 1 < nchunks) prefetch(c + 1, tid_l);

        // ---- phase 1: this wave's V fragments; gates; K K^T lower tiles
        typename M::frag vcur[NVF];
#pragma unroll
        for (int kk = 0; kk < KS_C; ++kk)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                vcur[kk * 2 + nt] = M::col_nat(hd.v, SM::VLD, col0 + 16 * nt + li, kk, g4);
        if (wv - hh * NWH == 0) {                          // first wave of each head
            const float gs = hd.graw[lane];
            const float bs = hd.braw[lane];
            const float Gc = wave_inclusive_sum(gs, lane);
            const float G_last = __shfl(Gc, kC - 1, 64);
            const float gam = expf(Gc);
            hd.gate[GATE_G * kC + lane] = Gc;
            hd.gate[GATE_GAM * kC + lane] = gam;
            hd.gate[GATE_BET * kC + lane] = bs;
            hd.gate[GATE_BG * kC + lane] = bs * gam;
            hd.gate[GATE_KDEC * kC + lane] = expf(G_last - Gc);
        }
        f32x4 kkt[TPW];
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int t = wv + NW * j;
            const int mt = t >> 2, nt = t & 3;
            f32x4 ak = {0.f, 0.f, 0.f, 0.f};
            if (t < 16 && nt <= mt) {
#pragma unroll 2
                for (int kk = 0; kk < KS_DK; ++kk)
                    ak = M::mma(M::row_nat(sm.k + (16 * mt + li) * SM::QLD, kk, g4),
                                M::row_nat(sm.k + (16 * nt + li) * SM::QLD, kk, g4), ak);
            }
            kkt[j] = ak;
        }
        lds_barrier();

        // ---- phase 2: A for every head (zeros on and above the diagonal)
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int t = wv + NW * j;
            if (t >= 16) continue;
            const int mt = t >> 2, nt = t & 3;
#pragma unroll
            for (int x = 0; x < HG; ++x) {
                const float* gt = sm.hd[x].gate;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + 4 * g4 + i, s = 16 * nt + li;
                    const float val = s < r ? gt[GATE_BET * kC + r] * kkt[j][i] *
                                                  expf(gt[GATE_G * kC + r] - gt[GATE_G * kC + s])
                                            : 0.f;
                    sm.hd[x].a[r * SM::ALD + s] = val;
                }
            }
        }
        lds_barrier();

        // ---- phase 3: T = (I + A)^-1 in place, one wave per head
        if (wv - hh * NWH == 0) {
            float* as = hd.a;
            constexpr int ALD = SM::ALD;
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
                __builtin_amdgcn_wave_barrier();
                float* Tb = as + (16 * b) * ALD + 16 * b;
#pragma unroll
                for (int r = 0; r < 16; ++r) Tb[r * ALD + j] = t[r];
            }
            __builtin_amdgcn_wave_barrier();
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
                                as[(16 * ib + li) * ALD + 16 * kb + 4 * q + g4],    // A_ik[m][4q + g]
                                as[(16 * kb + 4 * q + g4) * ALD + 16 * jb + li],    // T_kj[4q + g][n]
                                X, 0, 0, 0);
                    f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q = 0; q < 4; ++q)   // B from X's registers: element q is row 4g + q
                        Y = __builtin_amdgcn_mfma_f32_16x16x4f32(as[(16 * ib + li) * ALD + 16 * ib + 4 * g4 + q],
                                                                 X[q], Y, 0, 0, 0);
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int i = 0; i < 4; ++i) as[(16 * ib + 4 * g4 + i) * ALD + 16 * jb + li] = -Y[i];
                    __builtin_amdgcn_wave_barrier();
                }
            }
        }
        lds_barrier();

        // ---- phase 4: T1 = T diag(beta) and -T2 = -T diag(beta gamma), split, all threads
#pragma unroll
        for (int x = 0; x < HG; ++x) {
            typename SM::Head& hx = sm.hd[x];
            for (int idx = tid; idx < kC * kC / 4; idx += NT) {
                const int r = idx >> 4, s4 = (idx & 15) * 4;
                const float4 tv = *reinterpret_cast<const float4*>(hx.a + r * SM::ALD + s4);
                const float tr[4] = {tv.x, tv.y, tv.z, tv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = s4 + e;
                    split_store<E>(hx.t1[0], hx.t1[SM::NS - 1], r * SM::TLD + s, tr[e] * hx.gate[GATE_BET * kC + s]);
                    split_store<E>(hx.t2[0], hx.t2[SM::NS - 1], r * SM::TLD + s, -tr[e] * hx.gate[GATE_BG * kC + s]);
                }
            }
        }
        lds_barrier();

        // ---- phase 5a: P for every head (into the dead A/T space); Z = K S; U = T1 V + (-T2) Z
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int t = wv + NW * j;
            if (t >= 16) continue;
            const int mt = t >> 2, nt = t & 3;
            f32x4 aq = {0.f, 0.f, 0.f, 0.f};
            if (nt <= mt) {
#pragma unroll 2
                for (int kk = 0; kk < KS_DK; ++kk)
                    aq = M::mma(M::row_nat(sm.q + (16 * mt + li) * SM::QLD, kk, g4),
                                M::row_nat(sm.k + (16 * nt + li) * SM::QLD, kk, g4), aq);
            }
#pragma unroll
            for (int x = 0; x < HG; ++x) {
                const float* gt = sm.hd[x].gate;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mt + 4 * g4 + i, s = 16 * nt + li;
                    const float val = s <= r ? aq[i] * expf(gt[GATE_G * kC + r] - gt[GATE_G * kC + s]) : 0.f;
                    sm.hd[x].p[r * SM::PLD + s] = (E)val;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 Uacc[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            Uacc[mt][0] = Uacc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS_C; ++kk) {
                if (kmin_nat<M>(kk) > 16 * mt + 15) continue;
                const typename M::pair ta = row_pair_nat<E>(hd.t1[0] + (16 * mt + li) * SM::TLD,
                                                            hd.t1[SM::NS - 1] + (16 * mt + li) * SM::TLD, kk, g4);
                Uacc[mt][0] = M::mma_sa(ta, vcur[kk * 2 + 0], Uacc[mt][0]);
                Uacc[mt][1] = M::mma_sa(ta, vcur[kk * 2 + 1], Uacc[mt][1]);
            }
        }
        // Z = K S and U += (-T2) Z, one 16-column tile at a time
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            __builtin_amdgcn_sched_barrier(0);   // keep the two tiles' live ranges apart
            f32x4 Zacc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) Zacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS_DK; ++kk) {
                const typename M::frag sb = M::acc_fromc(&Sacc[0][nt], kk, 2);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    Zacc[mt] = M::mma(M::row_fromc(sm.k + (16 * mt + li) * SM::QLD, kk, g4), sb, Zacc[mt]);
            }
#pragma unroll
            for (int kk = 0; kk < KS_C; ++kk) {
                const typename M::frag zb = M::acc_fromc(&Zacc[0], kk, 1);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (kmin_fromc<M>(kk) > 16 * mt + 15) continue;
                    const typename M::pair ta = row_pair_fromc<E>(hd.t2[0] + (16 * mt + li) * SM::TLD,
                                                                  hd.t2[SM::NS - 1] + (16 * mt + li) * SM::TLD, kk, g4);
                    Uacc[mt][nt] = M::mma_sa(ta, zb, Uacc[mt][nt]);
                }
            }
        }
        lds_barrier();   // P is complete

        // ---- phase 5b: O = gamma o (Q S) + P U, one 16-column tile at a time
        const float* gam = hd.gate + GATE_GAM * kC;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            __builtin_amdgcn_sched_barrier(0);
            f32x4 Oacc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) Oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS_DK; ++kk) {
                const typename M::frag sb = M::acc_fromc(&Sacc[0][nt], kk, 2);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    Oacc[mt] = M::mma(M::row_fromc(sm.q + (16 * mt + li) * SM::QLD, kk, g4), sb, Oacc[mt]);
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
                    Oacc[mt] = M::mma_sb(M::row_fromc(hd.p + (16 * mt + li) * SM::PLD, kk, g4), ub, Oacc[mt]);
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

        __builtin_amdgcn_sched_barrier(0);
        // ---- phase 5c: S = gamma_last S + K^T (diag(e^(G_last - G)) U)
        const float gl_last = gam[kC - 1];
        const float* kdec = hd.gate + GATE_KDEC * kC;
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
                const typename M::frag ka = M::col_fromc(sm.k, SM::QLD, 16 * mt + li, kk, g4);
                Sacc[mt][0] = M::mma_sb(ka, ub0, Sacc[mt][0]);
                Sacc[mt][1] = M::mma_sb(ka, ub1, Sacc[mt][1]);
            }
        }

        // ---- export on the grid
        if (a.export_grid > 0) {
            const int64_t p_end = pos0 + e0;
            if (p_end % a.export_grid == 0) {
                const int64_t m = p_end / a.export_grid - pos0 / a.export_grid - 1;
                const int64_t idx = (int64_t)a.export_offsets[seq] + m;
                float* dst = nullptr;
                if (idx >= 0 && idx < a.export_capacity) {
                    if (!a.export_slots) {
                        dst = a.export_states + ((size_t)idx * a.H_v + h) * SE;
                    } else {                    // straight into a cache slot
                        const int sl = a.export_slots[idx];
                        if (sl >= 0 && sl < a.num_slots) dst = a.pool + ((size_t)sl * a.H_v + h) * SE;
                    }
                }
                if (dst) {
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
        const int li = lane & 15, g4 = lane >> 4;
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

template <typename E, int DK, int DV, int HG>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
    const int G = a.H_v / a.H_k;
    const unsigned blocks = (unsigned)a.num_seqs * (unsigned)a.H_k * (unsigned)(G / HG);
    hipLaunchKernelGGL((scan_kernel<E, DK, DV, HG>), dim3(blocks), dim3(HG * DV * 2), 0, stream, a);
    return hipGetLastError();
}

template <typename E, int HG>
hipError_t launch_dims(const PrefillArgs& a, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_typed<E, 128, 128, HG>(a, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_typed<E, 128, 64, HG>(a, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_typed<E, 64, 128, HG>(a, stream);
    return launch_typed<E, 64, 64, HG>(a, stream);
}

}  // namespace

size_t prefill_workspace_bytes(int, int, int, int64_t) { return 0; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.dtype == 1) return launch_prefill_bf16(a, stream);
    return launch_dims<float, 1>(a, stream);
}

}  // namespace gdn
