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
//     R   = diag(beta) (V - diag(gamma) K S0)
//     U   = (I + A)^-1 R                           (a unit lower-triangular solve)
//     O   = scale (diag(gamma) Q S0 + (Q K^T o D o lower-incl-diagonal) U)
//     S1  = gamma_last S0 + K^T (diag(e^(G_last - G)) U)
// The solve runs on 16-row blocks: with N = -A and T_ii = (I + A_ii)^-1 (16 x 16),
//     U_i = T_ii (R_i + sum_{j<i} N_ij U_j).
//
// One kernel (for d_k = d_v = 64 in 16-column strips, scan_kernel_pipe below, the same
// work with the helper waves a chunk ahead).  A workgroup owns one sequence and one
// value head and walks the sequence's chunks in order.  Per value head, d_v is split into 32-column
// strips (16-column ones when the call has no more chains than compute units), one
// wave each; a wave keeps its strip of S (d_k x 32 or d_k x 16, fp32) in MFMA
// accumulator registers for the whole sequence.  The d_v columns of S, R, U and O are
// independent, so strips never exchange data.  Per chunk:
//   stage    Q, K, V rows and the raw gates from the registers they were prefetched
//            into during the previous chunk, into LDS
//   phase 1  each wave's V strip into registers; the gates by a wave scan (every
//            wave, the same table); the lower tiles of K K^T and Q K^T on MFMA, round
//            robin over the waves, written out as N = -A and P into LDS (fp32)
//   phase 2  the first wave inverts the four diagonal blocks by forward substitution
//            (lane 16b + j owns column j of block b); every wave forms Z = K S and R
//            for its strip
//   phase 3  per strip: the block solve for U on MFMA, X_i's accumulator feeding the
//            products directly; O = gamma o (Q S) + P U; the state update; the grid
//            export
// Precision.  The MFMAs are 16x16x4 fp32 and nothing is rounded below fp32: states,
// accumulators, gates and the diagonal inverses are fp32.  A sequence's work never
// depends on the other sequences of the call, so its results are bitwise
// independent of its batch-mates; the chunks lie on the absolute 64-token grid, so
// a resume from an exported grid state continues with the same arithmetic.
#include <hip/hip_runtime.h>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

using dev::kC;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- fp32 MFMA operands
//
// 16x16x4 fp32 products on 16x16 output tiles.  Lane l holds A[l % 16][k] and
// B[k][l % 16] for one k per step; the C/D tile is held as C[4 (l / 16) + i][l % 16],
// i = 0..3.  Which k a lane stands for only has to agree between A and B, so two k
// orders are used:
//   blocked   lane group g holds the contiguous k = (K / 4) g .. (K / 4) g + K / 4 - 1,
//             for products of two row-major LDS operands (16-byte reads)
//   from-C    the order in which a C tile's registers already sit, so that an fp32
//             accumulator tile can feed the next product as its B operand without an
//             LDS round trip: step ks is register (ks & 3) of C tile (ks >> 2), i.e.
//             row 16 (ks >> 2) + 4 g + (ks & 3).
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int k_fromc(int ks, int g) { return 16 * (ks >> 2) + 4 * g + (ks & 3); }
// e^x as 2^(x log2 e): log2 e split into an fp32 part and the remainder (Cody and
// Waite's argument splitting), so that t + tl carries x log2 e to about 2^-48 of it;
// the hardware base-2 exponential of t, and 2^tl ~ 1 + tl ln 2 for the tiny tl.  About
// 1-2 ulp; results below fp32's normal range lose precision (the decays there are
// negligible against the unit-sized terms they sit beside).
__device__ __forceinline__ float exp_fast(float x) {
    constexpr float kL2eHi = 1.44269502162933349609375f;
    constexpr float kL2eLo = 1.925963033500011079e-08f;
    constexpr float kLn2 = 0.693147180559945309f;
    const float t = x * kL2eHi;
    const float tl = fmaf(x, kL2eHi, -t) + x * kL2eLo;
    const float p = __builtin_amdgcn_exp2f(t);
    return fmaf(p * tl, kLn2, p);
}

// element k of a C-layout tile set (tiles[t * stride] holds rows 16 t ..), from-C order
__device__ __forceinline__ float acc_fromc(const f32x4* tiles, int ks, int stride) {
    return tiles[(ks >> 2) * stride][ks & 3];
}
// The 16x16 tile X Y^T of two row blocks of K columns in LDS (ra, rb: this lane's row
// of each), k in blocked order: every operand arrives in 16-byte reads issued ahead of
// the products.
template <int K>
__device__ __forceinline__ f32x4 row_tile(const float* ra, const float* rb, int g) {
    f32x4 xa[K / 16], xb[K / 16];
#pragma unroll
    for (int q = 0; q < K / 16; ++q) {
        xa[q] = *reinterpret_cast<const f32x4*>(ra + (K / 4) * g + 4 * q);
        xb[q] = *reinterpret_cast<const f32x4*>(rb + (K / 4) * g + 4 * q);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < K / 16; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mma(xa[q][e], xb[q][e], acc);
    return acc;
}

// A chunk's rows of a token-major tensor as a raw buffer of nrec bytes (the chunk's
// valid rows): a load at a byte offset at or past nrec returns zero without touching
// memory (the buffer's range check), so rows past a partial chunk's end enter as zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t rows_rsrc(const void* base, int nrec) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}
__device__ __forceinline__ uint4 ld16_rows(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Per-token gate rows of a chunk: G (inclusive cumsum of g), gamma = e^G, beta,
// e^(G_last - G), -beta and 1 (the row factors of the N and the P tiles).
constexpr int kGates = 6;
enum { GATE_G = 0, GATE_GAM = 1, GATE_BET = 2, GATE_KDEC = 3, GATE_NBET = 4, GATE_ONE = 5 };

template <int DK, int DV>
struct ScanSmem {
    static constexpr int QLD = DK + 4;        // Q and K rows (16-byte aligned, banks spread)
    static constexpr int ALD = kC + 4;        // A / T rows
    static constexpr int PLD = ALD;           // P rows (the same pitch: tiles of either)
    static constexpr int VLD = DV + 4;        // V rows
    float q[kC * QLD];
    float k[kC * QLD];
    float v[kC * VLD];            // V rows (staging to phase 1)
    float a[kC * ALD];            // N = -A, then T_bb in place of N_bb (phases 1-3)
    float p[kC * PLD];            // P (phases 1-3)
    float gate[kGates * kC];
    float graw[kC];
    float braw[kC];
};

// ---------------------------------------------------------------- the scan kernel

// SW is the width of a wave's strip of value columns: 32, or 16 for calls whose
// workgroups each get a compute unit of their own (twice the waves, half the products
// per wave along the chain of chunks).
// NX helper waves (0 or 4) join a workgroup of four strips: they share the tiles and
// invert the diagonal blocks, and sit out the strips' work.
template <int DK, int DV, int SW, int NX>
__global__ __launch_bounds__((DV / SW + NX) * 64) void scan_kernel(PrefillArgs a) {
    using SM = ScanSmem<DK, DV>;
    constexpr int NWS = DV / SW;             // strip waves (one strip each)
    constexpr int NW = NWS + NX;             // waves
    constexpr int SUBW = 0;                  // the wave that inverts the diagonal blocks
    constexpr int NTL = SW / 16;             // 16-column tiles per strip
    constexpr int NT = NW * 64;              // threads
    constexpr int MT_S = DK / 16;            // 16-row tiles of the state
    constexpr int KS_DK = DK / 4;            // k steps over d_k
    constexpr int KS_C = kC / 4;             // k steps over the chunk
    constexpr int VPR = DK / 4;              // 16-byte vectors per Q/K row
    constexpr int NPF = 2 * kC * VPR / NT;   // prefetched Q/K vectors per thread
    constexpr int VPRV = DV / 4;             // 16-byte vectors per V row
    constexpr int NPV = kC * VPRV / NT;      // prefetched V vectors per thread
    // The ten lower 16x16 tiles (mt, nt), nt <= mt, of a 64x64 matrix, numbered row by row,
    // of K K^T and then of Q K^T go round robin to the waves.
    constexpr int TPW = (20 + NW - 1) / NW;  // tiles per wave
    static_assert(NPF * NT == 2 * kC * VPR && (kC * VPR) % NT == 0, "Q/K prefetch must divide evenly");
    static_assert(NPV * NT == kC * VPRV, "V prefetch must divide evenly");
    __shared__ __attribute__((aligned(16))) SM sm;

    const int G = a.H_v / a.H_k;
    const int seq = blockIdx.x / a.H_v;
    const int h = blockIdx.x - seq * a.H_v;
    const int kh = h / G;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
    int lane = tid & 63;
    // Helpers are the first waves: waves wv and wv + 4 share a SIMD, and the older wave
    // wins the issue arbitration, so the helper's substitution runs ahead of its SIMD
    // partner's Z products.
    const bool strip = NX == 0 || wv >= NX;  // uniform
    const int col0 = SW * (wv - NX);         // (strip waves)

    const size_t SE = (size_t)DK * DV;
    // state strip in accumulator layout: Sacc[mt][nt] holds S[16mt + 4g + i][col0 + 16nt + li]
    f32x4 Sacc[MT_S][NTL];
    const int isl = a.init_slot ? a.init_slot[seq] : -1;
    if (strip && isl >= 0 && isl < a.num_slots) {
        const int li = lane & 15, g4 = lane >> 4;
        const float* src = a.pool + ((size_t)isl * a.H_v + h) * SE;
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sacc[mt][nt][i] = src[(size_t)(16 * mt + 4 * g4 + i) * DV + col0 + 16 * nt + li];
    } else {
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) Sacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int lo, len;
    dev::seq_range(a.cu_seqlens, seq, a.total_tokens, lo, len);
    const int64_t pos0 = a.start_pos ? a.start_pos[seq] : 0;
    const int off64 = (int)(pos0 & (kC - 1));
    const int nchunks = dev::seq_chunks(len, off64);

    const float* qg = static_cast<const float*>(a.q);
    const float* kg = static_cast<const float*>(a.k);
    const float* vg = static_cast<const float*>(a.v);
    float* og = static_cast<float*>(a.o);

    // ---- prefetch registers: Q/K row vectors, V row vectors, g/beta (16-byte vector
    //      loads that nothing consumes until the next chunk is staged)
    uint4 pf[NPF];
    uint4 pv[NPV];
    float gbpf = 0.f;
    auto prefetch = [&](int c, int t) {
        int b0, e0;
        dev::chunk_span(c, off64, len, b0, e0);
        const int tok = lo + b0, L = e0 - b0;
        // the chunk's rows as raw buffers: loads past its L rows return zeros
        const rsrc_t rq = rows_rsrc(qg + (size_t)tok * a.H_k * DK, L * a.H_k * DK * 4);
        const rsrc_t rk = rows_rsrc(kg + (size_t)tok * a.H_k * DK, L * a.H_k * DK * 4);
        const rsrc_t rv = rows_rsrc(vg + (size_t)tok * a.H_v * DV, L * a.H_v * DV * 4);
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int i = t + NT * j;
            const int which = NT * j / (kC * VPR);       // 0: Q, 1: K (uniform: NT divides kC VPR)
            const int r = (i / VPR) % kC, vi = i % VPR;
            const uint32_t off = (uint32_t)((r * a.H_k + kh) * DK + vi * 4) * 4u;
            pf[j] = ld16_rows(which == 0 ? rq : rk, off);
        }
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
            const int i = t + NT * j;
            const int r = i / VPRV, vi = i % VPRV;
            const uint32_t off = (uint32_t)((r * a.H_v + h) * DV + vi * 4) * 4u;
            pv[j] = ld16_rows(rv, off);
        }
        if (t < 2 * kC) {                                 // g then beta of this head
            const int which = t / kC, s = t % kC;
            const float* src = (which == 0 ? a.g : a.beta) + (size_t)tok * a.H_v;
            const uint32_t off = (uint32_t)(s * a.H_v + h) * 4u;
            gbpf = s < L ? *reinterpret_cast<const float*>(reinterpret_cast<const char*>(src) + off) : 0.f;
        }
    };
    if (nchunks > 0) prefetch(0, tid);

    for (int c = 0; c < nchunks; ++c) {
        int b0, e0;
        dev::chunk_span(c, off64, len, b0, e0);
        const int tok = lo + b0, L = e0 - b0;
        // Keep lane-derived addresses inside the loop: without this the compiler hoists
        // every unrolled access's address out of the chunk loop and runs out of registers.
        int tid_l = tid;
        asm volatile("" : "+v"(lane), "+v"(tid_l));
        const int li = lane & 15, g4 = lane >> 4;
        dev::lds_barrier();   // the previous chunk is done with LDS

        // ---- stage this chunk's inputs; prefetch the next chunk
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int i = tid + NT * j;
            const int which = i / (kC * VPR);
            const int r = (i / VPR) % kC, vi = i % VPR;
            *reinterpret_cast<uint4*>((which == 0 ? sm.q : sm.k) + r * SM::QLD + vi * 4) = pf[j];
        }
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
            const int i = tid + NT * j;
            const int r = i / VPRV, vi = i % VPRV;
            *reinterpret_cast<uint4*>(sm.v + r * SM::VLD + vi * 4) = pv[j];
        }
        if (tid < 2 * kC) (tid < kC ? sm.graw : sm.braw)[tid % kC] = gbpf;
        dev::lds_barrier();
        // the staged inputs are in LDS: fetch the next chunk's behind this chunk's compute
        if (c + 1 < nchunks) prefetch(c + 1, tid_l);

        // ---- phase 1: this wave's V strip in the accumulator layout; the gates (every
        //      wave scans them and writes the same table, so that none waits for
        //      another); the twenty tiles, the ten lower ones of K K^T (each written out
        //      as N = -A at once, zeros on and above the diagonal; nothing reads the
        //      upper tiles) and then the ten of P = Q K^T o D, round robin
        f32x4 Racc[4][NTL];          // V, then R = beta (V - gamma Z), then X_i of the solve
        if (strip) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Racc[mt][nt][i] = sm.v[(16 * mt + 4 * g4 + i) * SM::VLD + col0 + 16 * nt + li];
        }
        {
            const float gs = sm.graw[lane];
            const float bs = sm.braw[lane];
            const float Gc = dev::wave_inclusive_sum(gs);
            const float G_last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Gc), kC - 1));
            sm.gate[GATE_G * kC + lane] = Gc;
            sm.gate[GATE_GAM * kC + lane] = exp_fast(Gc);
            sm.gate[GATE_BET * kC + lane] = bs;
            sm.gate[GATE_NBET * kC + lane] = -bs;
            sm.gate[GATE_ONE * kC + lane] = 1.f;
            sm.gate[GATE_KDEC * kC + lane] = exp_fast(G_last - Gc);
        }
        __builtin_amdgcn_wave_barrier();   // the table is written before any lane reads it
        // Branch-free per tile (the N or P choice is a select), so that the unrolled
        // tiles form one block the compiler can overlap.
        auto tile = [&](int j) __attribute__((always_inline)) {
            const int u = wv + NW * j;
            if (NW * TPW > 20 && j == TPW - 1 && u >= 20) return;
            const bool isp = u >= 10;                         // uniform
            const int t = isp ? u - 10 : u;
            const int mt = (t >= 1) + (t >= 3) + (t >= 6), nt = t - mt * (mt + 1) / 2;
            const f32x4 x = row_tile<DK>((isp ? sm.q : sm.k) + (16 * mt + li) * SM::QLD, sm.k + (16 * nt + li) * SM::QLD, g4);
            float* dst = isp ? sm.p : sm.a;
            const float* fac = sm.gate + (isp ? GATE_ONE : GATE_NBET) * kC;   // 1 or -beta
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * g4 + i, s = 16 * nt + li;
                const float d = exp_fast(sm.gate[GATE_G * kC + r] - sm.gate[GATE_G * kC + s]);
                // zero outside the triangle by a bit mask (a select there becomes a branch
                // around the exponential)
                const unsigned keep = s < r + (int)isp ? ~0u : 0u;
                dst[r * SM::ALD + s] = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, fac[r] * x[i] * d) & keep);
            }
        };
        if constexpr (TPW <= 5) {
#pragma unroll
            for (int j = 0; j < TPW; ++j) tile(j);
        } else {                              // two waves: ten tiles each, not unrolled
#pragma unroll 1
            for (int j = 0; j < TPW; ++j) tile(j);
        }
        dev::lds_barrier();   // N and P are complete

        // ---- phase 2: the first wave (a helper, if any) inverts the diagonal
        //      blocks, T_bb = (I + A_bb)^-1 in place of N_bb, by forward substitution
        //      (lane 16 b + j owns column j of block b); every strip wave forms Z = K S
        //      and R = beta (V - gamma Z) for its strip
        if (wv == SUBW) {
            const int b = g4, j = li;
            const float* Nb = sm.a + (16 * b) * SM::ALD + 16 * b;
            // each row starts from column j of I: rows above j then sum products with
            // zeros only (t = 0 there), row j comes out as 1
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = r == j ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc = fmaf(Nb[r * SM::ALD + s], t[s], acc);
                t[r] = acc;
            }
            __builtin_amdgcn_wave_barrier();
            float* Tb = sm.a + (16 * b) * SM::ALD + 16 * b;
#pragma unroll
            for (int r = 0; r < 16; ++r) Tb[r * SM::ALD + j] = t[r];
        }
        if (strip) {
            // Z = K S and R = beta (V - gamma Z), one 16-column tile at a time
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                __builtin_amdgcn_sched_barrier(0);   // keep the two tiles' live ranges apart
                f32x4 Zacc[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) Zacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) {
                    const float sb = acc_fromc(&Sacc[0][nt], kk, NTL);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        Zacc[mt] = mma(sm.k[(16 * mt + li) * SM::QLD + k_fromc(kk, g4)], sb, Zacc[mt]);
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const f32x4 gam = *reinterpret_cast<const f32x4*>(sm.gate + GATE_GAM * kC + 16 * mt + 4 * g4);
                    const f32x4 bet = *reinterpret_cast<const f32x4*>(sm.gate + GATE_BET * kC + 16 * mt + 4 * g4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Racc[mt][nt][i] = bet[i] * fmaf(-gam[i], Zacc[mt][i], Racc[mt][nt][i]);
                }
            }
        }
        dev::lds_barrier();   // the T_bb are complete

        if (strip) {
            // ---- phase 3: the block solve U_i = T_ii X_i, X_i = R_i + sum_{j<i} N_ij U_j,
            //      right-looking: once U_i exists it enters every later X_k.  X_i's
            //      accumulator feeds the products as their B operand (from-C order).
            f32x4 Uacc[4][NTL];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        u = mma(sm.a[(16 * i + li) * SM::ALD + 16 * i + 4 * g4 + kk], Racc[i][nt][kk], u);
                    Uacc[i][nt] = u;
                }
#pragma unroll
                for (int k = i + 1; k < 4; ++k)
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            Racc[k][nt] = mma(sm.a[(16 * k + li) * SM::ALD + 16 * i + 4 * g4 + kk], Uacc[i][nt][kk], Racc[k][nt]);
            }

            // ---- O = gamma o (Q S) + P U, one 16-column tile at a time; the chunk's output
            //      rows as a raw buffer, whose range check drops the stores of rows past L
            const rsrc_t ro = rows_rsrc(og + ((size_t)tok * a.H_v + h) * DV + col0, L * a.H_v * DV * 4);
            const float* gam = sm.gate + GATE_GAM * kC;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                __builtin_amdgcn_sched_barrier(0);
                f32x4 Oacc[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) Oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) {
                    const float sb = acc_fromc(&Sacc[0][nt], kk, NTL);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        Oacc[mt] = mma(sm.q[(16 * mt + li) * SM::QLD + k_fromc(kk, g4)], sb, Oacc[mt]);
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) Oacc[mt][i] *= gam[16 * mt + 4 * g4 + i];
#pragma unroll
                for (int kk = 0; kk < KS_C; ++kk) {
                    const float ub = acc_fromc(&Uacc[0][nt], kk, NTL);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        if (16 * (kk >> 2) > 16 * mt + 15) continue;  // P is lower triangular
                        Oacc[mt] = mma(sm.p[(16 * mt + li) * SM::PLD + k_fromc(kk, g4)], ub, Oacc[mt]);
                    }
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t off = (uint32_t)((16 * mt + 4 * g4 + i) * a.H_v * DV + 16 * nt + li) * 4u;
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, a.scale * Oacc[mt][i]), ro, (int)off, 0, 0);
                    }
            }

            __builtin_amdgcn_sched_barrier(0);
            // ---- S = gamma_last S + K^T (diag(e^(G_last - G)) U)
            const float gl_last = gam[kC - 1];
            const float* kdec = sm.gate + GATE_KDEC * kC;
#pragma unroll
            for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt) Sacc[mt][nt][i] *= gl_last;
                }
#pragma unroll
            for (int kk = 0; kk < KS_C; ++kk) {
                const float d = kdec[k_fromc(kk, g4)];
                float ub[NTL];
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) ub[nt] = acc_fromc(&Uacc[0][nt], kk, NTL) * d;
#pragma unroll
                for (int mt = 0; mt < MT_S; ++mt) {
                    const float ka = sm.k[k_fromc(kk, g4) * SM::QLD + 16 * mt + li];
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt) Sacc[mt][nt] = mma(ka, ub[nt], Sacc[mt][nt]);
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
                            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    dst[(size_t)(16 * mt + 4 * g4 + i) * DV + col0 + 16 * nt + li] = Sacc[mt][nt][i];
                    }
                }
            }
        }
    }

    const int fsl = a.final_slot ? a.final_slot[seq] : -1;
    if (strip && fsl >= 0 && fsl < a.num_slots) {
        const int li = lane & 15, g4 = lane >> 4;
        float* dst = a.pool + ((size_t)fsl * a.H_v + h) * SE;
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[(size_t)(16 * mt + 4 * g4 + i) * DV + col0 + 16 * nt + li] = Sacc[mt][nt][i];
    }
}

// d_k = d_v = 64 in 16-column strips: the four strip waves (4-7) and four helper waves
// (0-3) work a chunk apart.  While the strips run chunk c's solve, output and state
// update, the helpers stage chunk c + 1 and form its tiles and diagonal inverses
// (helper b block b's diagonal K K^T tile and its inverse, so the helpers need no sync
// among themselves, then four of the sixteen other tiles).  Q, K, N, P and the gate
// table are double-buffered by chunk parity; the strips read V straight from HBM.
// Every wave runs the same two barriers per chunk, in straight-line code.  The
// arithmetic per element is the scan kernel's.
template <int DK, int DV>
struct PipeSmem {
    static constexpr int QLD = DK + 4;        // Q and K rows
    static constexpr int ALD = kC + 4;        // N / T rows
    static constexpr int PLD = ALD;           // P rows
    float q[2][kC * QLD];
    float k[2][kC * QLD];
    float a[2][kC * ALD];
    float p[2][kC * PLD];
    float gate[2][kGates * kC];
};

__device__ __forceinline__ float ld4_rows(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

__global__ __launch_bounds__(512) void scan_kernel_pipe(PrefillArgs a) {
    constexpr int DK = 64, DV = 64, SW = 16, NX = 4;
    using SM = PipeSmem<DK, DV>;
    constexpr int NTL = 1;                   // 16-column tiles per strip
    constexpr int MT_S = DK / 16;            // 16-row tiles of the state
    constexpr int KS_DK = DK / 4;            // k steps over d_k
    constexpr int KS_C = kC / 4;             // k steps over the chunk
    constexpr int VPR = DK / 4;              // 16-byte vectors per Q/K row
    constexpr int NTH = NX * 64;             // helper threads
    constexpr int NPF = 2 * kC * VPR / NTH;  // prefetched Q/K vectors per helper thread
    static_assert(NPF * NTH == 2 * kC * VPR && (kC * VPR) % NTH == 0, "Q/K prefetch must divide evenly");
    __shared__ __attribute__((aligned(16))) SM sm;

    const int G = a.H_v / a.H_k;
    const int seq = blockIdx.x / a.H_v;
    const int h = blockIdx.x - seq * a.H_v;
    const int kh = h / G;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
    int lane = tid & 63;
    const bool strip = wv >= NX;             // uniform
    const int col0 = SW * (wv - NX);         // (strip waves)

    const size_t SE = (size_t)DK * DV;
    // state strip in accumulator layout: Sacc[mt][nt] holds S[16mt + 4g + i][col0 + 16nt + li]
    f32x4 Sacc[MT_S][NTL];
    const int isl = a.init_slot ? a.init_slot[seq] : -1;
    if (strip && isl >= 0 && isl < a.num_slots) {
        const int li = lane & 15, g4 = lane >> 4;
        const float* src = a.pool + ((size_t)isl * a.H_v + h) * SE;
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sacc[mt][0][i] = src[(size_t)(16 * mt + 4 * g4 + i) * DV + col0 + li];
    } else {
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt) Sacc[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int lo, len;
    dev::seq_range(a.cu_seqlens, seq, a.total_tokens, lo, len);
    const int64_t pos0 = a.start_pos ? a.start_pos[seq] : 0;
    const int off64 = (int)(pos0 & (kC - 1));
    const int nchunks = dev::seq_chunks(len, off64);

    const float* qg = static_cast<const float*>(a.q);
    const float* kg = static_cast<const float*>(a.k);
    const float* vg = static_cast<const float*>(a.v);
    float* og = static_cast<float*>(a.o);

    // helpers: a chunk's Q and K rows (16-byte vectors) and, on the first helper, its g
    // and beta (lane = token)
    uint4 pf[NPF];
    float gpf = 0.f, bpf = 0.f;
    auto prefetch_h = [&](int c, int t) __attribute__((always_inline)) {
        int b0, e0;
        dev::chunk_span(c, off64, len, b0, e0);
        const int tok = lo + b0, L = e0 - b0;
        const rsrc_t rq = rows_rsrc(qg + (size_t)tok * a.H_k * DK, L * a.H_k * DK * 4);
        const rsrc_t rk = rows_rsrc(kg + (size_t)tok * a.H_k * DK, L * a.H_k * DK * 4);
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int i = t + NTH * j;
            const int which = NTH * j / (kC * VPR);      // 0: Q, 1: K (uniform)
            const int r = (i / VPR) % kC, vi = i % VPR;
            const uint32_t off = (uint32_t)((r * a.H_k + kh) * DK + vi * 4) * 4u;
            pf[j] = ld16_rows(which == 0 ? rq : rk, off);
        }
        if (t < kC) {
            const uint32_t off = (uint32_t)(t * a.H_v + h) * 4u;
            gpf = ld4_rows(rows_rsrc(a.g + (size_t)tok * a.H_v, L * a.H_v * 4), off);
            bpf = ld4_rows(rows_rsrc(a.beta + (size_t)tok * a.H_v, L * a.H_v * 4), off);
        }
    };
    // helpers: the prefetched chunk into buffer nb; the first helper scans its gates
    auto stage_h = [&](int nb, int t) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int i = t + NTH * j;
            const int which = i / (kC * VPR);
            const int r = (i / VPR) % kC, vi = i % VPR;
            *reinterpret_cast<uint4*>((which == 0 ? sm.q[nb] : sm.k[nb]) + r * SM::QLD + vi * 4) = pf[j];
        }
        if (wv == 0) {
            float* gt = sm.gate[nb];
            const float Gc = dev::wave_inclusive_sum(gpf);
            const float G_last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Gc), kC - 1));
            gt[GATE_G * kC + t] = Gc;
            gt[GATE_GAM * kC + t] = exp_fast(Gc);
            gt[GATE_BET * kC + t] = bpf;
            gt[GATE_NBET * kC + t] = -bpf;
            gt[GATE_ONE * kC + t] = 1.f;
            gt[GATE_KDEC * kC + t] = exp_fast(G_last - Gc);
        }
    };
    // strips: a chunk's V strip in accumulator layout, rows past the chunk as zeros
    float vpf[4 * MT_S];
    auto prefetch_v = [&](int c, int ln) __attribute__((always_inline)) {
        int b0, e0;
        dev::chunk_span(c, off64, len, b0, e0);
        const int tok = lo + b0, L = e0 - b0;
        const rsrc_t rv = rows_rsrc(vg + ((size_t)tok * a.H_v + h) * DV + col0, L * a.H_v * DV * 4);
        const unsigned li = (unsigned)ln & 15u, g4 = (unsigned)ln >> 4;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vpf[4 * mt + i] = ld4_rows(rv, (uint32_t)((16 * mt + 4 * g4 + i) * a.H_v * DV + li) * 4u);
    };
    // helpers: chunk n's tiles and diagonal inverses into buffer nb (helper b: block b's
    // diagonal K K^T tile and its inverse, then four of the sixteen other tiles)
    auto tiles_h = [&](int nb, int li, int g4) __attribute__((always_inline)) {
        const float* Q_ = sm.q[nb];
        const float* K_ = sm.k[nb];
        const float* GT_ = sm.gate[nb];
        float* A_ = sm.a[nb];
        float* P_ = sm.p[nb];
        auto tile = [&](int u) __attribute__((always_inline)) {
            const bool isp = u >= 10;                         // uniform
            const int t = isp ? u - 10 : u;
            const int mt = (t >= 1) + (t >= 3) + (t >= 6), nt = t - mt * (mt + 1) / 2;
            const f32x4 x = row_tile<DK>((isp ? Q_ : K_) + (16 * mt + li) * SM::QLD, K_ + (16 * nt + li) * SM::QLD, g4);
            float* dst = isp ? P_ : A_;
            const float* fac = GT_ + (isp ? GATE_ONE : GATE_NBET) * kC;   // 1 or -beta
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mt + 4 * g4 + i, s = 16 * nt + li;
                const float d = exp_fast(GT_[GATE_G * kC + r] - GT_[GATE_G * kC + s]);
                const unsigned keep = s < r + (int)isp ? ~0u : 0u;
                dst[r * SM::ALD + s] = __builtin_bit_cast(float, __builtin_bit_cast(unsigned, fac[r] * x[i] * d) & keep);
            }
        };
        const int b = wv;                    // this helper's diagonal block
        tile(b * (b + 3) / 2);
        __builtin_amdgcn_wave_barrier();     // N_bb is written before it is read
        {   // T_bb = (I + A_bb)^-1 in place of N_bb, lane owning column li (every lane
            // group the same column: same values to the same addresses)
            const float* Nb = A_ + (16 * b) * SM::ALD + 16 * b;
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = r == li ? 1.f : 0.f;
#pragma unroll
                for (int s2 = 0; s2 < r; ++s2) acc = fmaf(Nb[r * SM::ALD + s2], t[s2], acc);
                t[r] = acc;
            }
            __builtin_amdgcn_wave_barrier();
            float* Tb = A_ + (16 * b) * SM::ALD + 16 * b;
#pragma unroll
            for (int r = 0; r < 16; ++r) Tb[r * SM::ALD + li] = t[r];
        }
        // the others: off-diagonal K K^T tiles 1 3 4 6 7 8, then the Q K^T tiles 10..19
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int o = wv + NX * j;
            tile(o < 6 ? o + 1 + (o >= 1) + (o >= 3) : o + 4);
        }
    };

    if (nchunks > 0) {
        if (!strip) {
            prefetch_h(0, tid);
            stage_h(0, tid);
            if (nchunks > 1) prefetch_h(1, tid);
        } else {
            prefetch_v(0, lane);
        }
    }
    if (nchunks > 0) {
        dev::lds_barrier();                  // chunk 0 staged
        if (!strip) {
            const int li = lane & 15, g4 = lane >> 4;
            tiles_h(0, li, g4);
        }
        dev::lds_barrier();                  // chunk 0's tiles and inverses
    }

    for (int c = 0; c < nchunks; ++c) {
        int b0, e0;
        dev::chunk_span(c, off64, len, b0, e0);
        const int tok = lo + b0, L = e0 - b0;
        const int cb = c & 1, nb = cb ^ 1;
        int tid_l = tid;
        asm volatile("" : "+v"(lane), "+v"(tid_l));
        const int li = lane & 15, g4 = lane >> 4;
        const float* Q_ = sm.q[cb];
        const float* K_ = sm.k[cb];
        const float* GT_ = sm.gate[cb];
        const float* A_ = sm.a[cb];
        const float* P_ = sm.p[cb];

        // ---- first half: the helpers stage chunk c + 1 and fetch chunk c + 2; the strips
        //      take chunk c's V, fetch chunk c + 1's and form Z = K S and R
        f32x4 Racc[4][NTL];
        if (!strip) {
            if (c + 1 < nchunks) {
                stage_h(nb, tid_l);
                if (c + 2 < nchunks) prefetch_h(c + 2, tid_l);
            }
        } else {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) Racc[mt][0][i] = vpf[4 * mt + i];
            if (c + 1 < nchunks) prefetch_v(c + 1, lane);
            // Z = K S and R = beta (V - gamma Z), one 16-column tile at a time
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                __builtin_amdgcn_sched_barrier(0);   // keep the two tiles' live ranges apart
                f32x4 Zacc[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) Zacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) {
                    const float sb = acc_fromc(&Sacc[0][nt], kk, NTL);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        Zacc[mt] = mma(K_[(16 * mt + li) * SM::QLD + k_fromc(kk, g4)], sb, Zacc[mt]);
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const f32x4 gam = *reinterpret_cast<const f32x4*>(GT_ + GATE_GAM * kC + 16 * mt + 4 * g4);
                    const f32x4 bet = *reinterpret_cast<const f32x4*>(GT_ + GATE_BET * kC + 16 * mt + 4 * g4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Racc[mt][nt][i] = bet[i] * fmaf(-gam[i], Zacc[mt][i], Racc[mt][nt][i]);
                }
            }
        }
        dev::lds_barrier();   // chunk c + 1 staged

        // ---- second half: the helpers form chunk c + 1's tiles and inverses; the strips
        //      run chunk c's solve, output, state update and export
        if (!strip) {
            if (c + 1 < nchunks) tiles_h(nb, li, g4);
        }
        if (strip) {
            // ---- the block solve U_i = T_ii X_i, X_i = R_i + sum_{j<i} N_ij U_j,
            //      right-looking: once U_i exists it enters every later X_k.  X_i's
            //      accumulator feeds the products as their B operand (from-C order).
            f32x4 Uacc[4][NTL];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) {
                    f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        u = mma(A_[(16 * i + li) * SM::ALD + 16 * i + 4 * g4 + kk], Racc[i][nt][kk], u);
                    Uacc[i][nt] = u;
                }
#pragma unroll
                for (int k = i + 1; k < 4; ++k)
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            Racc[k][nt] = mma(A_[(16 * k + li) * SM::ALD + 16 * i + 4 * g4 + kk], Uacc[i][nt][kk], Racc[k][nt]);
            }

            // ---- O = gamma o (Q S) + P U, one 16-column tile at a time; the chunk's output
            //      rows as a raw buffer, whose range check drops the stores of rows past L
            const rsrc_t ro = rows_rsrc(og + ((size_t)tok * a.H_v + h) * DV + col0, L * a.H_v * DV * 4);
            const float* gam = GT_ + GATE_GAM * kC;
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                __builtin_amdgcn_sched_barrier(0);
                f32x4 Oacc[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) Oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS_DK; ++kk) {
                    const float sb = acc_fromc(&Sacc[0][nt], kk, NTL);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        Oacc[mt] = mma(Q_[(16 * mt + li) * SM::QLD + k_fromc(kk, g4)], sb, Oacc[mt]);
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) Oacc[mt][i] *= gam[16 * mt + 4 * g4 + i];
#pragma unroll
                for (int kk = 0; kk < KS_C; ++kk) {
                    const float ub = acc_fromc(&Uacc[0][nt], kk, NTL);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        if (16 * (kk >> 2) > 16 * mt + 15) continue;  // P is lower triangular
                        Oacc[mt] = mma(P_[(16 * mt + li) * SM::PLD + k_fromc(kk, g4)], ub, Oacc[mt]);
                    }
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t off = (uint32_t)((16 * mt + 4 * g4 + i) * a.H_v * DV + 16 * nt + li) * 4u;
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, a.scale * Oacc[mt][i]), ro, (int)off, 0, 0);
                    }
            }

            __builtin_amdgcn_sched_barrier(0);
            // ---- S = gamma_last S + K^T (diag(e^(G_last - G)) U)
            const float gl_last = gam[kC - 1];
            const float* kdec = GT_ + GATE_KDEC * kC;
#pragma unroll
            for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt) Sacc[mt][nt][i] *= gl_last;
                }
#pragma unroll
            for (int kk = 0; kk < KS_C; ++kk) {
                const float d = kdec[k_fromc(kk, g4)];
                float ub[NTL];
#pragma unroll
                for (int nt = 0; nt < NTL; ++nt) ub[nt] = acc_fromc(&Uacc[0][nt], kk, NTL) * d;
#pragma unroll
                for (int mt = 0; mt < MT_S; ++mt) {
                    const float ka = K_[k_fromc(kk, g4) * SM::QLD + 16 * mt + li];
#pragma unroll
                    for (int nt = 0; nt < NTL; ++nt) Sacc[mt][nt] = mma(ka, ub[nt], Sacc[mt][nt]);
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
                            for (int nt = 0; nt < NTL; ++nt)
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    dst[(size_t)(16 * mt + 4 * g4 + i) * DV + col0 + 16 * nt + li] = Sacc[mt][nt][i];
                    }
                }
            }
        }
        dev::lds_barrier();   // chunk c done; chunk c + 1's tiles complete
    }

    const int fsl = a.final_slot ? a.final_slot[seq] : -1;
    if (strip && fsl >= 0 && fsl < a.num_slots) {
        const int li = lane & 15, g4 = lane >> 4;
        float* dst = a.pool + ((size_t)fsl * a.H_v + h) * SE;
#pragma unroll
        for (int mt = 0; mt < MT_S; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(size_t)(16 * mt + 4 * g4 + i) * DV + col0 + li] = Sacc[mt][0][i];
    }
}

template <int DK, int DV, int SW>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
    const unsigned blocks = (unsigned)a.num_seqs * (unsigned)a.H_v;
    // four helper waves beside four 16-column strips (d_v 64): a compute unit of its
    // own then runs two waves per SIMD
    constexpr int NX = SW == 16 && DV == 64 ? 4 : 0;
    if constexpr (DK == 64 && DV == 64 && SW == 16) {   // the helpers a chunk ahead
        hipLaunchKernelGGL(scan_kernel_pipe, dim3(blocks), dim3(512), 0, stream, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((scan_kernel<DK, DV, SW, NX>), dim3(blocks), dim3((DV / SW + NX) * 64), 0, stream, a);
    return hipGetLastError();
}

template <int SW>
hipError_t launch_f32_dims(const PrefillArgs& a, hipStream_t stream) {
    if (a.d_k == 128 && a.d_v == 128) return launch_typed<128, 128, SW>(a, stream);
    if (a.d_k == 128 && a.d_v == 64) return launch_typed<128, 64, SW>(a, stream);
    if (a.d_k == 64 && a.d_v == 128) return launch_typed<64, 128, SW>(a, stream);
    return launch_typed<64, 64, SW>(a, stream);
}

// One value head per workgroup; 16-column strips when the (sequence, value head)
// chains do not outnumber the compute units.  Both strip widths run the same
// arithmetic per element.
hipError_t launch_f32(const PrefillArgs& a, hipStream_t stream) {
    if ((int64_t)a.num_seqs * a.H_v <= device_cus()) return launch_f32_dims<16>(a, stream);
    return launch_f32_dims<32>(a, stream);
}

}  // namespace

size_t prefill_workspace_bytes(int, int, int, int64_t) { return 0; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.dtype == 1) return launch_prefill_bf16(a, stream);
    return launch_f32(a, stream);
}

}  // namespace gdn
